// bf16 attention over a query tile's key-tile list, tuned for gfx950 (the hot kernel of
// the sparse layer; Zebra3D abstract: tile-sparse attention with landmark summaries).
//
// Workgroup = 2 waves = one (head, query tile); wave w owns queries [32w, 32w+32).
// Key and value tiles move HBM/L2 -> LDS by direct-to-LDS loads (global_load_lds,
// 16 bytes per lane), so staging costs no VGPRs and no VALU; each 128-byte row of a
// tile is stored as 8 chunks of 16 bytes in XOR-swizzled order (slot = chunk ^ row%8),
// which the loads realise by permuting their source chunks.  Two LDS buffers: the next
// tile streams in while the current one computes, one barrier per tile.
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows (ds_read_b128), B = Q (VGPRs)
//   O^T += V^T P^T   A = V^T read with ds_read_b64_tr_b16 (the transpose happens in the
//                    LDS read), B = P^T taken straight from the S^T accumulators
// Rows that are not keys load from a zero row and are masked to -inf by index, so pad
// rows (which may hold NaN) never reach the arithmetic.  Landmark blocks (fp32 tile
// means) are converted to bf16 through registers.
#include "attn_common.h"
#include "device.h"
#include "launch.h"

namespace s3d {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Source of masked rows: direct-to-LDS loads copy whatever they read, so rows that are
// not keys read these zeros.
__device__ __align__(16) const unsigned char kZeroRow[128] = {};

constexpr int TILE_BYTES = TILE * 128;           // one bf16 64x64 tile
constexpr int BUF_BYTES = 2 * TILE_BYTES;        // K + V

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ void dma16(const void* g, lds_u8* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
}

}  // namespace

// max of three floats without the NaN-quieting canonicalisation the compiler adds around
// fmaxf (scores come from the matrix core or are -inf, never signalling NaNs)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Rescale the running output only when some row max grew by more than this (base-2
// units); otherwise probabilities are taken against the stale max and stay <= 2^8.
constexpr float RESCALE_THRESHOLD = 8.0f;


template <bool F32OUT, bool DENSE, bool LM>
__global__ __launch_bounds__(128, 2) void k_attn_bf16(AttnDev p) {
    // two buffers, each [K | V] x 64 rows x 128 B: tile it computes from buffer it%2 while
    // tile it+1 streams into the other one
    __shared__ __align__(16) unsigned char s_buf[2 * BUF_BYTES];
    extern __shared__ uint32_t s_lm[];

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qc = lane & 31, g = lane >> 5;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int h = logical / p.Tq;
    const int rem = logical - h * p.Tq;
    const int tpfq = p.ql.P / TILE;
    const int tq = (rem % p.ql.S) * tpfq + rem / p.ql.S;
    const int Lq = p.ql.S * p.ql.P, Lk = p.kl.S * p.kl.P;
    const int qrow = tq * TILE + w * 32 + qc;
    const bool qvalid = (tq % tpfq) * TILE + w * 32 + qc < p.ql.N;

    bf16x8 qop[4];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((size_t)h * Lq + qrow) * HD;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 u = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * s + 8 * g)
                                   : make_uint4(0, 0, 0, 0);
            qop[s] = __builtin_bit_cast(bf16x8, u);
        }
    }
    // settle the Q loads here, on every path: otherwise the first matrix-core use inside
    // the tile loop waits on all vector-memory traffic, the next tile's loads included
    __builtin_amdgcn_s_waitcnt(0);

    int c = 0;
    const int32_t* myidx = nullptr;
    int ntiles;
    if (DENSE) {
        ntiles = p.Tk;
    } else {
        c = min(max(p.cnt[(size_t)h * p.Tq + tq], 0), p.kmax);
        myidx = p.idx + ((size_t)h * p.Tq + tq) * p.kmax;
        ntiles = p.Ts + c + (LM ? p.nlm : 0);
    }
    if (LM) init_landmark_bitmap(p, c, myidx, s_lm, tid, 128);
    // the selected-tile list, staged once in LDS (the first IDX_CACHE entries) so the
    // per-tile lookup is an LDS read instead of a dependent global load
    int32_t* s_idx = reinterpret_cast<int32_t*>(s_lm + (LM ? 2 * p.nlm : 0));
    if (!DENSE) {
        const int n = min(c, IDX_CACHE);
        for (int i = tid; i < n; i += 128) s_idx[i] = myidx[i];
        __syncthreads();
    }

    const unsigned char* kg = static_cast<const unsigned char*>(p.k) + (size_t)h * Lk * 128;
    const unsigned char* vg = static_cast<const unsigned char*>(p.v) + (size_t)h * Lk * 128;

    // ---- staging: wave w fills rows [32w, 32w+32) of K and of V; per instruction j the
    //      64 lanes cover rows 32w+8j .. +8, lane l -> (row l/8, slot l%8) in LDS order
    const int srow_in = lane >> 3, sslot = lane & 7;
    // byte offset of this lane's source chunk inside a 64-row tile, per instruction j
    int soff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 32 * w + 8 * j + srow_in;
        soff[j] = r * 128 + (sslot ^ (r & 7)) * 16;
    }
    uint4 lmk[4], lmv[4];                         // landmark rows staged through registers

    auto issue = [&](int it, lds_u8* dst, TileDesc& d) {
        d = describe<DENSE, LM>(p, it, c, myidx, s_idx, s_lm);
        if (d.kind == KIND_REG && d.mask == ~0ull) {
            // full tile: 64 consecutive rows
            const size_t base = (size_t)d.t * TILE_BYTES;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dma16(kg + base + soff[j], dst + (32 * w + 8 * j) * 128);
                dma16(vg + base + soff[j], dst + TILE_BYTES + (32 * w + 8 * j) * 128);
            }
        } else if (d.kind != KIND_LM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 32 * w + 8 * j + srow_in;
                const int ch = sslot ^ (r & 7);
                const bool ok = (d.mask >> r) & 1ull;
                const size_t off = (size_t)src_row(p, d, ok ? r : 0) * 128 + ch * 16;
                const void* ks = ok ? (const void*)(kg + off) : (const void*)(kZeroRow + ch * 16);
                const void* vs = ok ? (const void*)(vg + off) : (const void*)(kZeroRow + ch * 16);
                dma16(ks, dst + (32 * w + 8 * j) * 128);
                dma16(vs, dst + TILE_BYTES + (32 * w + 8 * j) * 128);
            }
        } else if (LM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 32 * w + 8 * j + srow_in;
                const int ch = sslot ^ (r & 7);
                const bool ok = (d.mask >> r) & 1ull;
                float4 a0 = make_float4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
                if (ok) {
                    const size_t o = ((size_t)h * p.Tk + d.t * TILE + r) * HD + ch * 8;
                    a0 = *reinterpret_cast<const float4*>(p.kbar + o);
                    a1 = *reinterpret_cast<const float4*>(p.kbar + o + 4);
                    b0 = *reinterpret_cast<const float4*>(p.vbar + o);
                    b1 = *reinterpret_cast<const float4*>(p.vbar + o + 4);
                }
                lmk[j] = make_uint4(pack_bf16x2(a0.x, a0.y), pack_bf16x2(a0.z, a0.w),
                                    pack_bf16x2(a1.x, a1.y), pack_bf16x2(a1.z, a1.w));
                lmv[j] = make_uint4(pack_bf16x2(b0.x, b0.y), pack_bf16x2(b0.z, b0.w),
                                    pack_bf16x2(b1.x, b1.y), pack_bf16x2(b1.z, b1.w));
            }
        }
    };
    auto commit = [&](unsigned char* dst, const TileDesc& d) {
        if (LM && d.kind == KIND_LM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 32 * w + 8 * j + srow_in;
                *reinterpret_cast<uint4*>(dst + r * 128 + sslot * 16) = lmk[j];
                *reinterpret_cast<uint4*>(dst + TILE_BYTES + r * 128 + sslot * 16) = lmv[j];
            }
        }
    };

    // per-lane LDS offsets (bytes, within a buffer) of the MFMA operands
    int koff[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int r = 32 * kb + qc;
            koff[kb][st] = r * 128 + swz(r, 2 * st + g) * 16;
        }
    // V^T through the transposing read: lane j of each 16-lane group points at
    // V[16ks + 8half + 4g + j/4][32cb + 16*((lane/16)%2) + 4*(j%4)]; rows differ from the
    // ks=0/half=0 row by multiples of 8, so (row & 7) and the swizzle are per-lane constants
    const int vrow0 = 4 * g + ((lane & 15) >> 2);
    const int vcol_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int vsub = (lane & 1) * 8;
    int voff[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
        voff[cb] = TILE_BYTES + vrow0 * 128 + swz(vrow0, 4 * cb + vcol_chunk) * 16 + vsub;
    // key index of accumulator register r of block kb: 32kb + 8(r/4) + 4g + r%4
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    float m = -INFINITY, l = 0.f;
    f32x16 o0 = {}, o1 = {};

    // operands of one tile, read from LDS before the next tile's loads are issued: after
    // that point the iteration reads no LDS, so nothing has to wait for the loads in flight
    bf16x8 ka[2][4], va[2][4];
    auto fetch_operands = [&](const unsigned char* kb) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            ka[0][st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + koff[0][st]));
            ka[1][st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + koff[1][st]));
        }
        const lds_u8* lb = (const lds_u8*)kb;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16*)(lb + voff[cb] + ks * 16 * 128));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16*)(lb + voff[cb] + ks * 16 * 128 + 8 * 128));
                va[cb][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
    };

    auto compute = [&](const TileDesc& cur) {
        f32x16 s0 = {}, s1 = {};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0][st], qop[st], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[1][st], qop[st], s1, 0, 0, 0);
        }
        if (cur.mask != ~0ull) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * g + (r & 3);
                if (!((cur.mask >> key) & 1ull)) s0[r] = -INFINITY;
                if (!((cur.mask >> (32 + key)) & 1ull)) s1[r] = -INFINITY;
            }
        }
        const float bias = (LM && cur.kind == KIND_LM) ? p.lm_bias_l2 : 0.f;
        float mx = max3f(s0[0], s1[0], -INFINITY);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = max3f(mx, s0[r], s1[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx == -INFINITY ? -INFINITY : fmaf(mx, p.scale_l2, bias);
        // lazy rescale: move the reference max only when some row grew past the threshold
        if (__ballot(mt > m + RESCALE_THRESHOLD)) {
            const float mnew = fmaxf(m, mt);
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);   // 0 when m was -inf
            l *= alpha;
            o0 *= alpha;
            o1 *= alpha;
            m = mnew;
        }
        const float off = bias - (m == -INFINITY ? 0.f : m);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f32x16& sp = (ks < 2) ? s0 : s1;
            const int j0 = 2 * (ks & 1);
            float pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                pv[i] = __builtin_amdgcn_exp2f(fmaf(sp[4 * j0 + i], p.scale_l2, off));
            bf16x2 pp[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pp[i] = bf16x2{(__bf16)pv[2 * i], (__bf16)pv[2 * i + 1]};
                l = __builtin_amdgcn_fdot2_f32_bf16(pp[i], ones, l, false);   // sum of rounded P
            }
            const bf16x8 pb = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                                      __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                                      0, 1, 2, 3, 4, 5, 6, 7);
            o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[0][ks], pb, o0, 0, 0, 0);
            o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[1][ks], pb, o1, 0, 0, 0);
        }
    };

    TileDesc cur, nxt;
    lds_u8* const lbuf = (lds_u8*)s_buf;
    if (ntiles > 0) {
        issue(0, lbuf, cur);
        __builtin_amdgcn_s_waitcnt(0);
        commit(s_buf, cur);
        __syncthreads();
    }
    for (int it = 0; it < ntiles; ++it) {
        const int b = it & 1;
        const bool live = cur.mask != 0;
        if (live) fetch_operands(s_buf + b * BUF_BYTES);
        if (it + 1 < ntiles) issue(it + 1, lbuf + (b ^ 1) * BUF_BYTES, nxt);
        if (live) compute(cur);
        if (it + 1 < ntiles) {
            __builtin_amdgcn_s_waitcnt(0);      // this wave's tile-(it+1) loads have landed
            commit(s_buf + (b ^ 1) * BUF_BYTES, nxt);
            cur = nxt;
        }
        __syncthreads();                        // all loads landed; all reads of buffer b done
    }

    const float ltot = l + __shfl_xor(l, 32);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const size_t obase = ((size_t)h * Lq + qrow) * HD;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const f32x16& oc = cb ? o1 : o0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c0 = 32 * cb + 8 * j + 4 * g;
            float v4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v4[i] = qvalid ? oc[4 * j + i] * inv : 0.f;
            if (F32OUT) {
                *reinterpret_cast<float4*>(static_cast<float*>(p.out) + obase + c0) =
                    make_float4(v4[0], v4[1], v4[2], v4[3]);
            } else {
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + obase + c0) =
                    make_uint2(pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3]));
            }
        }
    }
    if (p.lse && g == 0) {
        float v = 0.f;
        if (qvalid) v = ltot > 0.f ? (m + log2f(ltot)) * LN2 : -INFINITY;
        p.lse[(size_t)h * Lq + qrow] = v;
    }
}

template <bool F32OUT>
static void launch_t(const AttnDev& d, int heads, bool dense, bool lm, hipStream_t st) {
    const dim3 grid((unsigned)(heads * d.Tq)), block(128);
    const size_t shm = ((lm ? (size_t)(2 * d.nlm) : 0) + (dense ? 0 : (size_t)min(d.kmax, IDX_CACHE))) *
                       sizeof(uint32_t);
    if (dense) hipLaunchKernelGGL((k_attn_bf16<F32OUT, true, false>), grid, block, 0, st, d);
    else if (lm) hipLaunchKernelGGL((k_attn_bf16<F32OUT, false, true>), grid, block, shm, st, d);
    else hipLaunchKernelGGL((k_attn_bf16<F32OUT, false, false>), grid, block, shm, st, d);
}

hipError_t launch_attn_bf16(const AttnDev& d, int heads, bool dense, bool lm, bool f32out,
                            hipStream_t st) {
    if (f32out) launch_t<true>(d, heads, dense, lm, st);
    else launch_t<false>(d, heads, dense, lm, st);
    return hipGetLastError();
}

}  // namespace s3d
