// Tile summaries (mean pooling) and pooled tile scores.
//
// Zebra3D (abstract) runs tile-sparse attention with landmark summaries; SAF3R
// (abstract) chooses interactions per input.  The per-tile means computed here are
// both the selection signal (query/key means -> scores) and the landmark
// summaries (key/value means).  Both kernels are HBM-bound: the pool streams Q, K
// (and V) once, the score kernel writes the [H, Tq, Tk] fp32 score matrix once.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace s3d {

// One wave per (head, tile).  Lane = (row group rg = lane/8, 16-byte column chunk
// c8 = lane%8); a wave load covers 8 consecutive rows = 1 KiB of bf16, so every
// access is a full 128-byte line.  Sums run in fp32: sequentially over the rows of a
// lane, then a fixed butterfly over the 8 row groups, so results are reproducible.
// out_op (optional): the same means rounded to the operand dtype (bf16: round to nearest
// even, as sparse3d_cast), the form the bf16 attention reads landmark means in.
template <bool BF16, bool KEY>
__global__ __launch_bounds__(256) void k_tile_pool(const void* __restrict__ x, int T, Lay L,
                                                   float* __restrict__ out, void* __restrict__ out_op) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    const int h = blockIdx.y;
    if (t >= T) return;
    int lo, hi;
    if (KEY) {
        member_range(L, t, lo, hi);
    } else {
        lo = 0;
        hi = valid_rows(L, t);
    }
    const int c8 = lane & 7, rg = lane >> 3;
    const size_t row0 = (size_t)h * T * TILE + (size_t)t * TILE;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int i = rg + 8 * it;
        const bool in = (i >= lo) && (i < hi);
        float f[8];
        if (BF16) {
            const uint4 u = *reinterpret_cast<const uint4*>(
                static_cast<const uint16_t*>(x) + (row0 + i) * HD + c8 * 8);
            unpack_bf16x8(u, f);
        } else {
            const float4* p =
                reinterpret_cast<const float4*>(static_cast<const float*>(x) + (row0 + i) * HD + c8 * 8);
            const float4 a = p[0], b = p[1];
            f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
            f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
        }
        // pad rows may hold NaN: select, never multiply by a 0/1 mask
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += in ? f[e] : 0.f;
    }
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
    }
    if (rg == 0) {
        const int n = hi - lo;
        float r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = n > 0 ? acc[e] / (float)n : 0.f;
        const size_t e0 = ((size_t)h * T + t) * HD + c8 * 8;
        float4* o = reinterpret_cast<float4*>(out + e0);
        o[0] = make_float4(r[0], r[1], r[2], r[3]);
        o[1] = make_float4(r[4], r[5], r[6], r[7]);
        if (out_op) {
            if (BF16) {
                *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out_op) + e0) =
                    make_uint4(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                               pack_bf16x2(r[6], r[7]));
            } else {
                float4* c = reinterpret_cast<float4*>(static_cast<float*>(out_op) + e0);
                c[0] = o[0];
                c[1] = o[1];
            }
        }
    }
}

// Tile scores on the matrix cores: sigma = scale * qbar . kbar (-inf where either tile has
// no rows).  The fp32 means are split into two bf16 terms, x = hi + lo with hi = bf16(x) and
// lo = bf16(x - hi) (x - hi - lo is below 2^-17 |x|), and the product takes all four cross
// terms, exact products accumulated in fp32 (small terms first): the scores agree with the
// fp32 dot product to about 1e-6 relative, and the matrix cores leave the kernel bound by
// writing the score matrix.
// A workgroup of four waves owns 128 query tiles (32 per wave, their hi/lo operands held in
// registers) and walks a range of key blocks of 64 tiles: each block's means are loaded
// once for the workgroup, split, and written to LDS (double-buffered; the next block's
// loads are in flight while the current one is multiplied).  The product is formed
// transposed (keys as the accumulator rows); each wave stages its 32 x 32 results through
// LDS and stores whole 128-byte lines, eight query rows per store instruction, while the
// matrix cores go on with the next products.  Stores and loads share one in-order
// completion counter, so the next block is split into LDS after this block's products and
// before its stores: waiting for its loads then waits only for the previous block's stores,
// which have had the products' time to drain.
constexpr int SC_Q = 128;               // query tiles per workgroup (4 waves x 32)
constexpr int SC_K = 64;                // key tiles per block
constexpr int SC_RESIDENT = 3 * 256;     // workgroups resident at once on the 256 compute units
// Score stores carry the non-temporal hint: the matrix is read once, by the selection, and
// streaming it past the caches measured 0.116 against 0.132 ms at 2816 x 2816 tiles x 16 heads.
constexpr int SC_NT = 2;
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8& hi, bf16x8& lo) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 hp = {(__bf16)x[2 * i], (__bf16)x[2 * i + 1]};
        const uint32_t u = __builtin_bit_cast(uint32_t, hp);
        const float h0 = __uint_as_float(u << 16), h1 = __uint_as_float(u & 0xffff0000u);
        const bf16x2 lp = {(__bf16)(x[2 * i] - h0), (__bf16)(x[2 * i + 1] - h1)};
        hw[i] = u;
        lw[i] = __builtin_bit_cast(uint32_t, lp);
    }
    hi = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    lo = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
}
// byte offset of dims 8c .. 8c + 7 of key row r in a [64 keys][64 dims] bf16 block: 16-byte
// chunks XOR-swizzled so that 16 lanes reading 16 consecutive keys hit 16 distinct bank groups
__device__ __forceinline__ int sc_koff(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
// byte offset of keys 4c .. 4c + 3 of query row r in a wave's [32 rows][32 keys] fp32 staging
// block, with the same swizzle: the accumulator writes (16 rows, one chunk each) and the row
// reads (two rows, eight chunks each) both touch 16 distinct bank groups per 16 lanes
__device__ __forceinline__ int sc_soff(int r, int c) { return sc_koff(r, c); }

__global__ __launch_bounds__(256) void k_tile_scores_mfma(const float* __restrict__ qbar,
                                                          const float* __restrict__ kbar, int Tq, int Tk,
                                                          Lay ql, Lay kl, float scale, int kblocks,
                                                          float* __restrict__ scores) {
    __shared__ __align__(16) unsigned char s_kh[2][SC_K * 128];   // key means, bf16 hi terms
    __shared__ __align__(16) unsigned char s_kl[2][SC_K * 128];   // and lo terms
    __shared__ __align__(16) unsigned char s_stage[4][32 * 128];  // per wave: 32 rows x 32 keys
    __shared__ uint64_t s_kempty[2];                              // key tiles without members
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, g = lane >> 5;
    const int h = blockIdx.z;
    const int r0 = blockIdx.y * SC_Q + 32 * w;                    // this wave's first query tile
    const int kb0 = blockIdx.x * kblocks * SC_K;                  // first key tile of the range
    const int nkb = min(kblocks, (Tk - kb0 + SC_K - 1) / SC_K);   // key blocks in the range
    const float* qb = qbar + (size_t)h * Tq * HD;
    const float* kb = kbar + (size_t)h * Tk * HD;

    // query operands: row r0 + col, dims 16 ks + 8 g .. + 8, split once
    bf16x8 ah[4], al[4];
    const int r = r0 + col;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        float x[8];
        if (r < Tq) {
            const float4* p = reinterpret_cast<const float4*>(qb + (size_t)r * HD + 16 * ks + 8 * g);
            const float4 u = p[0], v = p[1];
            x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
        split_bf16x8(x, ah[ks], al[ks]);
    }
    const bool qempty = r < Tq && valid_rows(ql, r) == 0;
    const bool any_qempty = __ballot(qempty) != 0ull;

    // staging of a key block: thread t takes key t / 4, dims 16 (t % 4) .. + 16
    const int sk = tid >> 2, sd = tid & 3;
    float4 raw[4];
    // the head's key means through a buffer resource: keys past Tk read zeros
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(kb), 0, Tk * HD * 4,
                                                                        0x00020000);
    auto load_block = [&](int s) {
        const int key = kb0 + s * SC_K + sk;
        typedef float f32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4v u = __builtin_bit_cast(f32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                rk, key * (HD * 4) + 64 * sd + 16 * i, 0, 0));
            raw[i] = make_float4(u[0], u[1], u[2], u[3]);
        }
    };
    auto write_block = [&](int s, int buf) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const float x[8] = {raw[2 * half].x, raw[2 * half].y, raw[2 * half].z, raw[2 * half].w,
                                raw[2 * half + 1].x, raw[2 * half + 1].y, raw[2 * half + 1].z, raw[2 * half + 1].w};
            bf16x8 hi, lo;
            split_bf16x8(x, hi, lo);
            const int off = sc_koff(sk, 2 * sd + half);
            *reinterpret_cast<bf16x8*>(s_kh[buf] + off) = hi;
            *reinterpret_cast<bf16x8*>(s_kl[buf] + off) = lo;
        }
        if (w == 0) {                                 // key tiles of the block without members
            const int key = kb0 + s * SC_K + lane;
            int lo = 0, hi = 1;
            if (key < Tk) member_range(kl, key, lo, hi);
            const uint64_t m = __ballot(hi <= lo);
            if (lane == 0) s_kempty[buf] = m;
        }
    };
    // rows past Tq fall outside this wave's store resource (based at its first row in 64-bit
    // arithmetic; offsets below 32 * Tk * 4 bytes, which the host's Tk cap keeps in 32 bits)
    const long long rows_here = (long long)Tq - r0 < 0 ? 0 : ((long long)Tq - r0 < 32 ? (long long)Tq - r0 : 32);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        scores + ((size_t)h * Tq + (size_t)(r0 < Tq ? r0 : 0)) * (size_t)Tk, 0, (int)(rows_here * Tk * 4), 0x00020000);
    unsigned char* stg = s_stage[w];

    if (nkb > 0) {
        load_block(0);
        write_block(0, 0);
    }
    __syncthreads();
    for (int s = 0; s < nkb; ++s) {
        const int buf = s & 1;
        if (s + 1 < nkb) load_block(s + 1);          // lands while this block is multiplied
        const uint64_t ke = s_kempty[buf];
        const bool any_empty = any_qempty || ke != 0ull;
        // both 32-key halves' products, then the next block's split into the other buffer
        // (its loads, and the previous block's score stores issued before them, have had the
        // products' time to land), then this block's stores
        f32x16 accs[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            // sigma^T = kbar qbar^T: key rows 32 cb + col of the block, dims 16 ks + 8 g
            bf16x8 bh[4], bl[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int off = sc_koff(32 * cb + col, 2 * ks + g);
                bh[ks] = *reinterpret_cast<const bf16x8*>(s_kh[buf] + off);
                bl[ks] = *reinterpret_cast<const bf16x8*>(s_kl[buf] + off);
            }
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {         // small terms first
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[ks], al[ks], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[ks], al[ks], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[ks], ah[ks], acc, 0, 0, 0);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[ks], ah[ks], acc, 0, 0, 0);
            accs[cb] = acc;
        }
        if (s + 1 < nkb) write_block(s + 1, buf ^ 1);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const f32x16& acc = accs[cb];
            // lane: query row r0 + col; keys 8 a + 4 g + j of the 32 (accumulator rows)
            if (!any_empty) {                        // the common case: no empty tile in sight
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *reinterpret_cast<float4*>(stg + sc_soff(col, 2 * a + g)) =
                        make_float4(acc[4 * a] * scale, acc[4 * a + 1] * scale, acc[4 * a + 2] * scale,
                                    acc[4 * a + 3] * scale);
            } else {
                const uint32_t kw = (uint32_t)(ke >> (32 * cb)) >> (4 * g);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    float v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v[j] = acc[4 * a + j] * scale;
                        if (qempty || ((kw >> (8 * a + j)) & 1u)) v[j] = -INFINITY;
                    }
                    *reinterpret_cast<float4*>(stg + sc_soff(col, 2 * a + g)) = make_float4(v[0], v[1], v[2], v[3]);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // lanes 8 i .. 8 i + 7: query row 8 q + i, keys 4 (lane % 8) .. + 3 of the 32
            const int ch = lane & 7;
            const int cbase = kb0 + s * SC_K + 32 * cb + 4 * ch;
            const bool whole = kb0 + s * SC_K + 32 * cb + 32 <= Tk;   // no ragged column in this half
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            u32x4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[q] = *reinterpret_cast<const u32x4*>(stg + sc_soff(8 * q + (lane >> 3), ch));
            // the four 16-byte reads all issue before the first store: left to itself the
            // compiler splits each around the ragged-column branch into 12- and 4-byte reads,
            // which conflict on the LDS banks and are each waited for alone
            asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = 8 * q + (lane >> 3);
                const unsigned voff = ((unsigned)row * (unsigned)Tk + (unsigned)cbase) * 4u;
                if (whole || cbase + 3 < Tk) {
                    __builtin_amdgcn_raw_buffer_store_b128(v[q], rs, (int)voff, 0, SC_NT);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)         // a ragged last key block
                        if (cbase + j < Tk) __builtin_amdgcn_raw_buffer_store_b32(v[q][j], rs, (int)voff, 4 * j, SC_NT);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();         // read before the next stage overwrites it
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        __syncthreads();
    }
}

hipError_t launch_tile_pool(const void* x, int dtype, int heads, LayH lay, bool key_rows, float* out,
                            void* out_op, hipStream_t st) {
    const int T = lay.S * lay.P / TILE;
    const Lay L{lay.S, lay.N, lay.P, lay.nsp};
    const dim3 grid((T + 3) / 4, heads), block(256);
    const bool bf16 = dtype == SPARSE3D_BF16;
    if (bf16 && key_rows) hipLaunchKernelGGL((k_tile_pool<true, true>), grid, block, 0, st, x, T, L, out, out_op);
    else if (bf16) hipLaunchKernelGGL((k_tile_pool<true, false>), grid, block, 0, st, x, T, L, out, out_op);
    else if (key_rows) hipLaunchKernelGGL((k_tile_pool<false, true>), grid, block, 0, st, x, T, L, out, out_op);
    else hipLaunchKernelGGL((k_tile_pool<false, false>), grid, block, 0, st, x, T, L, out, out_op);
    return hipGetLastError();
}

hipError_t launch_tile_scores(const float* qbar, const float* kbar, int heads, LayH ql, LayH kl,
                              float scale, float* scores, hipStream_t st) {
    const int Tq = ql.S * ql.P / TILE, Tk = kl.S * kl.P / TILE;
    const Lay lq{ql.S, ql.N, ql.P, ql.nsp}, lk{kl.S, kl.N, kl.P, kl.nsp};
    // split each head's key blocks into as many ranges as one round of resident workgroups
    // holds (three per compute unit, bound by LDS): every workgroup then starts at once and
    // none waits for a second round (at 5632 x 5632 tiles x 16 heads one range per query
    // block, 0.41-0.42 ms, against 0.42-0.44 ms with about 2048 workgroups)
    const int qblocks = (Tq + SC_Q - 1) / SC_Q, kblocks_all = (Tk + SC_K - 1) / SC_K;
    const long long per = (long long)qblocks * heads;
    const int nsplit = (int)std::max(1LL, std::min<long long>(kblocks_all, SC_RESIDENT / per));
    const int kblocks = (kblocks_all + nsplit - 1) / nsplit;
    const dim3 grid((unsigned)((kblocks_all + kblocks - 1) / kblocks), (unsigned)qblocks, (unsigned)heads);
    hipLaunchKernelGGL(k_tile_scores_mfma, grid, dim3(256), 0, st, qbar, kbar, Tq, Tk, lq, lk, scale, kblocks,
                       scores);
    return hipGetLastError();
}

__global__ void k_cast_bf16(const float* __restrict__ src, int64_t n, __bf16* __restrict__ dst) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = (__bf16)src[i];
}

hipError_t launch_cast(const float* src, int64_t n, int dtype, void* dst, hipStream_t st) {
    if (dtype == 0) return hipMemcpyAsync(dst, src, (size_t)n * 4, hipMemcpyDeviceToDevice, st);
    const int blocks = (int)std::min<int64_t>((n + 255) / 256, 8192);
    hipLaunchKernelGGL(k_cast_bf16, dim3(blocks), dim3(256), 0, st, src, n, static_cast<__bf16*>(dst));
    return hipGetLastError();
}

}  // namespace s3d
