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
template <bool BF16, bool KEY>
__global__ __launch_bounds__(256) void k_tile_pool(const void* __restrict__ x, int T, Lay L,
                                                   float* __restrict__ out) {
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
        float4* o = reinterpret_cast<float4*>(out + ((size_t)h * T + t) * HD + c8 * 8);
        o[0] = make_float4(r[0], r[1], r[2], r[3]);
        o[1] = make_float4(r[4], r[5], r[6], r[7]);
    }
}

// Tile scores on the matrix cores: sigma = scale * qbar . kbar (-inf where either tile has
// no rows), a 128 x 128 block per workgroup of four waves, each wave a 64 x 64 quarter as
// 2 x 2 accumulators of v_mfma_f32_32x32x16_bf16.  The fp32 means are split into two bf16
// terms, x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) (x - hi - lo is below 2^-17 |x|),
// and the product takes all four cross terms, exact products accumulated in fp32: the
// scores agree with the fp32 dot product to about 1e-6 relative, while the kernel, bound by
// writing the score matrix, runs several times faster than fp32 FMAs on the vector ALU.
// The product is formed transposed (keys as accumulator rows), so a lane holds four runs
// of four consecutive scores of one query row and writes each with one 16-byte store.
constexpr int SC_T = 128;               // queries x keys per workgroup
constexpr int SC_STG = 68;              // staged score row stride (floats): conflict-free b128
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
__global__ __launch_bounds__(256) void k_tile_scores_mfma(const float* __restrict__ qbar,
                                                          const float* __restrict__ kbar, int Tq, int Tk,
                                                          Lay ql, Lay kl, float scale,
                                                          float* __restrict__ scores) {
    __shared__ uint64_t s_empty[2][2];                 // [query rows | key columns][64-bit half]
    __shared__ __align__(16) float s_stage[4][32 * SC_STG];   // per wave: 32 rows x 64 keys
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, g = lane >> 5;
    const int h = blockIdx.z;
    const int tq0 = blockIdx.y * SC_T, tk0 = blockIdx.x * SC_T;
    // tiles of this block without rows (their scores are -inf), one ballot per 64 tiles
    {
        const int i = tid & 127;
        bool e;
        if (tid < 128) {
            e = tq0 + i < Tq && valid_rows(ql, tq0 + i) == 0;
        } else {
            int lo = 0, hi = 1;
            if (tk0 + i < Tk) member_range(kl, tk0 + i, lo, hi);
            e = hi <= lo;
        }
        const uint64_t m = __ballot(e);
        if (lane == 0) s_empty[w >> 1][w & 1] = m;
    }
    const int r0 = tq0 + 64 * (w >> 1), c0 = tk0 + 64 * (w & 1);
    const float* qb = qbar + (size_t)h * Tq * HD;
    const float* kb = kbar + (size_t)h * Tk * HD;
    // operands: row (or key) 32 b + col of this wave's quarter, dims 16 ks + 8 g .. +8
    bf16x8 ah[2][4], al[2][4], bh[2][4], bl[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int r = r0 + 32 * b + col, c = c0 + 32 * b + col;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float x[8], y[8];
            if (r < Tq) {
                const float4* p = reinterpret_cast<const float4*>(qb + (size_t)r * HD + 16 * ks + 8 * g);
                const float4 u = p[0], v = p[1];
                x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = 0.f;
            }
            if (c < Tk) {
                const float4* p = reinterpret_cast<const float4*>(kb + (size_t)c * HD + 16 * ks + 8 * g);
                const float4 u = p[0], v = p[1];
                y[0] = u.x; y[1] = u.y; y[2] = u.z; y[3] = u.w; y[4] = v.x; y[5] = v.y; y[6] = v.z; y[7] = v.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = 0.f;
            }
            split_bf16x8(x, ah[b][ks], al[b][ks]);
            split_bf16x8(y, bh[b][ks], bl[b][ks]);
        }
    }
    __syncthreads();
    const uint64_t qe = s_empty[0][w >> 1];            // this wave's 64 query rows
    const uint64_t ke = s_empty[1][w & 1];             // this wave's 64 key columns
    // stores through a buffer resource over this wave's 64 query rows of the head's [Tq, Tk]
    // slice, based at its first row in 64-bit arithmetic: rows past Tq (last block row) fall
    // outside the resource and are dropped, and the offsets inside it stay below
    // 64 * Tk * 4 bytes (the host caps Tk at 2^23, so they fit 32 bits at any Tq)
    const long long rows_here = (long long)Tq - r0 < 0 ? 0 : ((long long)Tq - r0 < 64 ? (long long)Tq - r0 : 64);
    const unsigned slice = (unsigned)(rows_here * Tk * 4);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        scores + ((size_t)h * Tq + (size_t)r0) * (size_t)Tk, 0, (int)slice, 0x00020000);
    const bool any_empty = (s_empty[0][0] | s_empty[0][1] | s_empty[1][0] | s_empty[1][1]) != 0ull;
    // Each wave stages its 32 x 64 block of one row band through LDS and stores it row by
    // row: one 16-byte store per lane then covers 4 rows x 256 contiguous bytes (whole cache
    // lines), where the accumulator layout would spread it over 32 rows x 32 bytes.
    float* stg = s_stage[w];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        // lane: query row r (its column of sigma^T); keys 8 (i / 4) + 4 g + i % 4 of the block
        const bool qempty = (qe >> (32 * rb + col)) & 1ull;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            // sigma^T = kbar qbar^T: keys are the accumulator rows
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {           // small terms first
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[cb][ks], al[rb][ks], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[cb][ks], al[rb][ks], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[cb][ks], ah[rb][ks], acc, 0, 0, 0);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[cb][ks], ah[rb][ks], acc, 0, 0, 0);
            const uint32_t kw = (uint32_t)(ke >> (32 * cb)) >> (4 * g);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[j] = acc[4 * a + j] * scale;
                    if (any_empty && (qempty || ((kw >> (8 * a + j)) & 1u))) v[j] = -INFINITY;
                }
                *reinterpret_cast<float4*>(stg + col * SC_STG + 32 * cb + 8 * a + 4 * g) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lanes 16 i .. 16 i + 15: row 4 s + i of the band, keys 4 (lane % 16) .. + 3
        const int ch = lane & 15;
        const int cbase = c0 + 4 * ch;
#pragma unroll
        for (int sr = 0; sr < 8; ++sr) {
            const int row = 4 * sr + (lane >> 4);
            const float4 v = *reinterpret_cast<const float4*>(stg + row * SC_STG + 4 * ch);
            const unsigned voff = ((unsigned)(32 * rb + row) * (unsigned)Tk + (unsigned)cbase) * 4u;
            if (cbase + 3 < Tk) {
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 pk = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                                  __float_as_uint(v.w)};
                __builtin_amdgcn_raw_buffer_store_b128(pk, rs, (int)voff, 0, 0);
            } else {
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)                // a ragged last column block
                    if (cbase + j < Tk)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vv[j]), rs, (int)voff, 4 * j, 0);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();                   // the band is read before the next overwrites it
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

hipError_t launch_tile_pool(const void* x, int dtype, int heads, LayH lay, bool key_rows, float* out,
                            hipStream_t st) {
    const int T = lay.S * lay.P / TILE;
    const Lay L{lay.S, lay.N, lay.P, lay.nsp};
    const dim3 grid((T + 3) / 4, heads), block(256);
    const bool bf16 = dtype == SPARSE3D_BF16;
    if (bf16 && key_rows) hipLaunchKernelGGL((k_tile_pool<true, true>), grid, block, 0, st, x, T, L, out);
    else if (bf16) hipLaunchKernelGGL((k_tile_pool<true, false>), grid, block, 0, st, x, T, L, out);
    else if (key_rows) hipLaunchKernelGGL((k_tile_pool<false, true>), grid, block, 0, st, x, T, L, out);
    else hipLaunchKernelGGL((k_tile_pool<false, false>), grid, block, 0, st, x, T, L, out);
    return hipGetLastError();
}

hipError_t launch_tile_scores(const float* qbar, const float* kbar, int heads, LayH ql, LayH kl,
                              float scale, float* scores, hipStream_t st) {
    const int Tq = ql.S * ql.P / TILE, Tk = kl.S * kl.P / TILE;
    const Lay lq{ql.S, ql.N, ql.P, ql.nsp}, lk{kl.S, kl.N, kl.P, kl.nsp};
    const dim3 grid((Tk + SC_T - 1) / SC_T, (Tq + SC_T - 1) / SC_T, heads), block(256);
    hipLaunchKernelGGL(k_tile_scores_mfma, grid, block, 0, st, qbar, kbar, Tq, Tk, lq, lk, scale, scores);
    return hipGetLastError();
}

// fp32 -> bf16, round to nearest even; one value per thread, grid-stride (no alignment
// requirement on either pointer).
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
