// bf16 attention over a query tile's key-tile list, tuned for gfx950 (the hot kernel of
// the sparse layer; Zebra3D abstract: tile-sparse attention with landmark summaries).
//
// Workgroup = 2 waves = one (head, query tile); wave w owns queries [32w, 32w+32).  (Dense
// and frame attention: 4 waves = two query tiles that share every staged key tile.)
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows (ds_read_b128), B = Q (VGPRs)
//   O^T += V^T P^T   A = V^T read with ds_read_b64_tr_b16 (the transpose happens in the
//                    LDS read), B = P^T taken straight from the S^T accumulators
// Three waves share each SIMD: at most 168 VGPRs per wave and 24 KiB of tile buffers per
// workgroup, so six workgroups fit a CU.  Step `it` forms S(it) = K(it) Q^T at its start,
// then the softmax and P V of tile it; the third wave hides the latency that a single
// wave's chain (LDS read, matrix core, softmax, matrix core) exposes.  K has one buffer:
// once every wave has read K(it) (first barrier of the step) the loads of K(it+1) go out.
// V has two: V(it+1) loads from the start of step it into the buffer V(it-1) left.  Tiles
// reach LDS by direct-to-LDS buffer loads (16 bytes per lane; per-lane constant offsets,
// the tile base in a scalar register), every 128-byte row stored as 8 XOR-swizzled 16-byte
// chunks (see swz_key).  Rows that are not keys load through an out-of-range offset, which
// reads as zeros, and are masked to -inf by index, so pad rows (which may hold NaN) never
// reach the arithmetic.  Landmark blocks (tile means in the operand precision) are staged
// like key tiles.
#include <type_traits>

#include "attn_common.h"
#include "device.h"
#include "launch.h"
#include "tile_lds.h"

namespace s3d {

using namespace tl;

// max of three floats without the NaN-quieting canonicalisation the compiler adds around
// fmaxf (scores come from the matrix core or are -inf, never signalling NaNs)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// x in the lanes whose bit is set in `lanes` (a wave-uniform mask in scalar registers),
// -inf in the others: one v_cndmask with the mask as its condition operand
__device__ __forceinline__ float keep_lanes(float x, uint64_t lanes) {
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(-INFINITY), "v"(x), "s"(lanes));
    return r;
}

// Global row (within the head) of special token e, numbering every frame's special tokens
// in frame order: frame e / nsp, in-frame position e % nsp.  The quotient is one fp64 FMA
// and a truncation, trunc((e + 1/2) * fl(1/nsp)): (e + 1/2) / nsp lies at least 1 / (2 nsp)
// from an integer, and the computed product is within a relative 2^-51 of it, far inside
// that margin for every 32-bit e.  (An integer division by the runtime nsp costs about 26
// vector instructions per row.)
__device__ __forceinline__ unsigned spec_src_row(unsigned e, unsigned nsp, double inv_nsp, unsigned P) {
    const unsigned f = (unsigned)fma((double)e, inv_nsp, 0.5 * inv_nsp);
    return f * P + (e - f * nsp);
}

// all ones if bit b of w is set, else zero
__device__ __forceinline__ uint32_t bit_to_word(uint32_t w, int b) {
    return (uint32_t)((int32_t)(w << (31 - b)) >> 31);
}

// max over the 32 scores of a lane (two 16-element accumulators), as two asm blocks of
// eight dependent v_max3_f32 each: one block per chain keeps the compiler from padding
// every step of the chain with wait states, as it does between separate asm statements
__device__ __forceinline__ float max32f(const f32x16& a, const f32x16& b) {
    float m;
    asm("v_max3_f32 %0, %1, %2, %3\n\t"
        "v_max3_f32 %0, %0, %4, %5\n\t"
        "v_max3_f32 %0, %0, %6, %7\n\t"
        "v_max3_f32 %0, %0, %8, %9\n\t"
        "v_max3_f32 %0, %0, %10, %11\n\t"
        "v_max3_f32 %0, %0, %12, %13\n\t"
        "v_max3_f32 %0, %0, %14, %15\n\t"
        "v_max3_f32 %0, %0, %16, %17"
        : "=&v"(m)
        : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]), "v"(a[2]), "v"(b[2]), "v"(a[3]), "v"(b[3]),
          "v"(a[4]), "v"(b[4]), "v"(a[5]), "v"(b[5]), "v"(a[6]), "v"(b[6]), "v"(a[7]), "v"(b[7]),
          "v"(-INFINITY));
    asm("v_max3_f32 %0, %0, %1, %2\n\t"
        "v_max3_f32 %0, %0, %3, %4\n\t"
        "v_max3_f32 %0, %0, %5, %6\n\t"
        "v_max3_f32 %0, %0, %7, %8\n\t"
        "v_max3_f32 %0, %0, %9, %10\n\t"
        "v_max3_f32 %0, %0, %11, %12\n\t"
        "v_max3_f32 %0, %0, %13, %14\n\t"
        "v_max3_f32 %0, %0, %15, %16"
        : "+v"(m)
        : "v"(a[8]), "v"(b[8]), "v"(a[9]), "v"(b[9]), "v"(a[10]), "v"(b[10]), "v"(a[11]), "v"(b[11]),
          "v"(a[12]), "v"(b[12]), "v"(a[13]), "v"(b[13]), "v"(a[14]), "v"(b[14]), "v"(a[15]), "v"(b[15]));
    return m;
}

// Dense and frame attention: rescale the running output only when some row max grew by
// more than this (base-2 units); otherwise probabilities are taken against the stale max
// and stay <= 2^8.
constexpr float RESCALE_THRESHOLD = 8.0f;
// Sparse attention: largest sum of one half tile's probabilities (16 per lane) taken
// without moving the reference max.
constexpr float PROB_SUM_LIMIT = 65536.0f;
// Sparse attention: the reference of a row that has seen no key yet.  Finite and far below
// any score, so the first probabilities against it overflow to +inf, the half's sum check
// fails and the half forms its max: no separate test for rows without a reference.  (A
// row that never sees a key ends with it and is treated as having no reference.)
constexpr float M_NONE = -0x1p126f;


// SGA: the subsample completion (own key of dropped positions, mean pair) is applied to
// each finished row; a separate instantiation so the other variants carry none of it.
// QT = 2 (dense and frame attention only): a workgroup of four waves takes two query tiles
// that sweep the same key tiles, so every staged tile serves 128 queries.
template <bool F32OUT, bool DENSE, bool LM, bool SGA, int QT = 1>
__global__ __launch_bounds__(128 * QT, 3) void k_attn_bf16(AttnDev p) {
    static_assert(QT == 1 || (QT == 2 && DENSE), "two query tiles per workgroup need a shared key sweep");
    __shared__ __align__(16) unsigned char s_k[TILE_BYTES];
    __shared__ __align__(16) unsigned char s_v0[TILE_BYTES];
    __shared__ __align__(16) unsigned char s_v1[TILE_BYTES];
    extern __shared__ uint32_t s_dyn[];

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qc = lane & 31, g = lane >> 5;
    const int tpfq = p.ql.P / TILE;
    int h, tq;
    if (QT == 1) {
        attn_work_item(blockIdx.x, gridDim.x, p.ql.S, tpfq, gridDim.x / p.Tq, h, tq, !p.frame);
    } else {
        // pairs of query tiles in plain order (the launcher takes QT = 2 only when Tq and the
        // tiles per frame are even, so a pair never straddles a frame)
        const int pairs = p.Tq / 2;
        h = blockIdx.x / pairs;
        tq = 2 * (blockIdx.x - h * pairs);
    }
    const int wt = QT == 1 ? 0 : (w >> 1);         // this wave's query tile within the workgroup
    const int wh = QT == 1 ? w : (w & 1);          // and its 32-row half
    const int Lq = p.ql.S * p.ql.P, Lk = p.kl.S * p.kl.P;
    const int qrow = (tq + wt) * TILE + wh * 32 + qc;
    const bool qvalid = ((tq + wt) % tpfq) * TILE + wh * 32 + qc < p.ql.N;
    // In the sparse paths a wave whose 32 rows are all padding (the second half of a frame's
    // last tile) still stages its half of every tile and meets every barrier, but skips the
    // products.  (Dense and frame attention keep every wave busy: there the workgroups sweep
    // the keys in lockstep and share them through L2, and one finishing early was slower.)
    // (an int from readfirstlane: kept as a bool, the compiler re-derives it on the vector
    // unit in every step)
    int wq = DENSE ? 1 : __builtin_amdgcn_readfirstlane((int)(__ballot(qvalid) != 0ull));
    asm volatile("" : "+s"(wq));

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
    __builtin_amdgcn_s_waitcnt(0);

    int c = 0, rot = 0, t0 = 0;
    const int32_t* myidx = nullptr;
    int ntiles;
    if (DENSE) {
        ntiles = p.frame ? p.kl.P / TILE : p.Tk;
        t0 = p.frame ? (tq / tpfq) * (p.kl.P / TILE) : 0;
    } else {
        c = min(max(p.cnt[(size_t)h * p.Tq + tq], 0), p.kmax);
        myidx = p.idx + ((size_t)h * p.Tq + tq) * p.kmax;
        ntiles = p.Ts + c + (LM ? p.nlm : 0);
    }
    uint32_t* s_lm = s_dyn;                          // landmark bitmap (2 nlm words), then the list
    if (LM) init_landmark_bitmap(p.kl, p.Tk, p.nlm, c, myidx, s_lm, tid, 128);
    int32_t* s_idx = reinterpret_cast<int32_t*>(s_dyn + (LM ? 2 * p.nlm : 0));
    if (!DENSE) {
        // the selected-tile list, staged once in LDS so that each step's lookup is an LDS read
        // (the launcher guarantees kmax <= IDX_LDS_MAX)
        for (int i = tid; i < c; i += 128) s_idx[i] = pack_tile_entry(p, myidx[i]);
        __syncthreads();
        // Sweep the list starting at the query's own frame (wrapping round): its tiles hold the
        // highest scores, so the softmax reference settles on the first steps (the list order
        // changes the result only by rounding).
        const int thr = (tq / tpfq) * (p.kl.P / TILE);
        int n = 0;
        for (int b = 0; b < c; b += 128)
            n += __syncthreads_count(b + tid < c && (s_idx[b + tid] & 0xFFFF) < thr);
        rot = n < c ? n : 0;
    }

    const unsigned head_bytes = (unsigned)Lk * 128u;
    const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(static_cast<const unsigned char*>(p.k)) + (size_t)h * head_bytes, 0,
        (int)head_bytes, BUF_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(static_cast<const unsigned char*>(p.v)) + (size_t)h * head_bytes, 0,
        (int)head_bytes, BUF_RSRC_WORD3);
    // landmark means (operand dtype, [heads, Tk, 64]): block b of 64 consecutive tile means
    // is staged like a key tile
    __amdgpu_buffer_rsrc_t rs_lk = rs_k, rs_lv = rs_v;
    if (LM) {
        const unsigned mean_bytes = (unsigned)p.Tk * 128u;
        rs_lk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(static_cast<const unsigned char*>(p.kbar)) + (size_t)h * mean_bytes, 0,
            (int)mean_bytes, BUF_RSRC_WORD3);
        rs_lv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(static_cast<const unsigned char*>(p.vbar)) + (size_t)h * mean_bytes, 0,
            (int)mean_bytes, BUF_RSRC_WORD3);
    }

    const int srow_in = lane >> 3, sslot = lane & 7;
    // each wave stages 32 / QT rows of every tile (8 rows per 16-byte-per-lane load)
    constexpr int NJ = 4 / QT;
    int srow[NJ], soff[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        srow[j] = (32 / QT) * w + 8 * j + srow_in;
        soff[j] = srow[j] * 128 + swz(srow[j], sslot) * 16;
    }
    auto desc = [&](int it) { return describe<DENSE, LM, !DENSE>(p, it, c, myidx, s_idx, s_lm, rot, t0); };
    // 1 / nsp for the special rows' quotient, uniform, so kept in scalar registers
    double inv_nsp;
    {
        const double x = 1.0 / (double)p.kl.nsp;
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
        inv_nsp = __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
    }
    auto plan = [&](const TileDesc& dd, unsigned (&voff)[NJ], unsigned& base) {
        const TileDesc d = uniform(dd);
        const bool spec = d.kind == KIND_SPEC;
        base = spec ? 0u : (unsigned)d.t * TILE_BYTES;
        if (spec) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int r = srow[j];
                const unsigned srcr = spec_src_row((unsigned)(d.t * TILE + r), (unsigned)p.kl.nsp, inv_nsp, (unsigned)p.kl.P);
                const unsigned o = srcr * 128u + swz(r, sslot) * 16u;
                voff[j] = ((d.mask >> r) & 1ull) ? o : OOB_OFFSET;
            }
        } else if (d.mask == ~0ull) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) voff[j] = (unsigned)soff[j];
        } else {
#pragma unroll
            for (int j = 0; j < NJ; ++j) voff[j] = ((d.mask >> srow[j]) & 1ull) ? (unsigned)soff[j] : OOB_OFFSET;
        }
    };
    auto dma4 = [&](const __amdgpu_buffer_rsrc_t& rs, lds_u8* dst, const unsigned (&voff)[NJ], unsigned base) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            dma_buf(rs, dst + ((32 / QT) * w + 8 * j) * 128, voff[j], __builtin_amdgcn_readfirstlane(base));
    };

    TileOffsets to;
    to.init(lane);
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    // m: running reference (base 2) of the lane's row; negm = -m, kept beside it so that the
    // sparse paths' probabilities need no per-step negation
    float m = DENSE ? -INFINITY : M_NONE, l = 0.f;
    float negm = -M_NONE;
    f32x16 o0 = {}, o1 = {};

    auto step = [&](int it, TileDesc& dcur, const unsigned char* vcur, unsigned char* vnext) {
        const TileDesc cur = uniform(dcur);
        const bool more = it + 1 < ntiles;
        TileDesc dn{};
        unsigned vk[NJ], vv[NJ], bk = 0, bv = 0;
        bool nlmk = false;                                  // tile it+1 is a landmark block
        if (more) {
            dn = desc(it + 1);
            plan(dn, vk, bk);
#pragma unroll
            for (int j = 0; j < NJ; ++j) vv[j] = vk[j];
            bv = bk;
            nlmk = LM && uniform(dn).kind == KIND_LM;
        } else {
#pragma unroll
            for (int j = 0; j < NJ; ++j) vk[j] = vv[j] = OOB_OFFSET;
        }
        dma4(nlmk ? rs_lv : rs_v, (lds_u8*)vnext, vv, bv);  // V(it+1)
        f32x16 s0, s1;
        if (wq) {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                bf16x8 a0, a1;
                read_rows(s_k, to, st, a0, a1);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qop[st], st ? s0 : f32x16{}, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qop[st], st ? s1 : f32x16{}, 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
        __builtin_amdgcn_s_barrier();                       // every wave has read K(it)
        dma4(nlmk ? rs_lk : rs_k, (lds_u8*)s_k, vk, bk);    // K(it+1)
        __builtin_amdgcn_sched_barrier(0);
        // the two 32-key halves of the row mask as scalars (left to itself the compiler folds a
        // test of the upper half back into a 64-bit compare, which runs on the vector unit)
        uint32_t mlo = (uint32_t)cur.mask, mhi = (uint32_t)(cur.mask >> 32);
        asm volatile("" : "+s"(mlo), "+s"(mhi));
        if (wq) {
            if ((mlo & mhi) != ~0u) {
                // slot r of a lane in half-wave g holds key 8 (r / 4) + 4 g + r % 4 (+32 in s1): its
                // lane mask takes one row bit for lanes 0-31 and another for lanes 32-63, formed
                // on the scalar unit from the uniform row mask.  The scores come from the matrix
                // core; the compiler does not see the reads inside the asm, so a few idle
                // cycles keep them clear of the products' write-back
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_nop 7\n\ts_nop 7");
                // Only a half holding both keys and non-keys needs the masks: a full half has
                // none to mask, and the sparse paths skip a half without keys before reading
                // its scores (the dense paths take the max over both halves, so there a half
                // without keys is masked too).
                auto mask_half = [&](f32x16& sc, uint32_t mh) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int cr = 8 * (r >> 2) + (r & 3);
                        // each 32-bit half of a lane mask is one row bit sign-extended (s_bfe_i32)
                        const uint64_t km = (uint64_t)bit_to_word(mh, cr) | ((uint64_t)bit_to_word(mh, cr + 4) << 32);
                        sc[r] = keep_lanes(sc[r], km);
                    }
                };
                if (mlo != ~0u && (DENSE || mlo != 0u)) mask_half(s0, mlo);
                if (mhi != ~0u && (DENSE || mhi != 0u)) mask_half(s1, mhi);
            }
            if constexpr (DENSE) {
                // every workgroup sweeps the keys in the same order, so the probabilities are
                // taken against the tile's row max (lazy rescale)
                float mx = max32f(s0, s1);
                {
                    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                    mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
                }
                const float mt = mx == -INFINITY ? -INFINITY : mx * p.scale_l2;
                if (__ballot(mt > m + RESCALE_THRESHOLD)) {
                    const float mnew = fmaxf(m, mt);
                    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
                    l *= alpha;
                    o0 *= alpha;
                    o1 *= alpha;
                    m = mnew;
                }
                const float off = -(m == -INFINITY ? 0.f : m);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    if ((ks < 2 ? mlo : mhi) == 0u) continue;   // no key in this half
                    const f32x16& sp = (ks < 2) ? s0 : s1;
                    const int j0 = 2 * (ks & 1);
                    bf16x8 va0, va1;
                    read_tr(vcur, to, ks, va0, va1);
                    float pv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(sp[4 * j0 + i], p.scale_l2, off));
                    bf16x2 pp[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pp[i] = bf16x2{(__bf16)pv[2 * i], (__bf16)pv[2 * i + 1]};
                        l = __builtin_amdgcn_fdot2_f32_bf16(pp[i], ones, l, false);
                    }
                    const bf16x8 pb = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                                              __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                                              0, 1, 2, 3, 4, 5, 6, 7);
                    o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va0, pb, o0, 0, 0, 0);
                    o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va1, pb, o1, 0, 0, 0);
                }
            } else {
                // Probabilities are taken against the running reference m without first forming
                // the tile's row max.  Each half tile (32 keys) checks afterwards that its rounded
                // probabilities sum to at most 2^16 (then none exceeds 2^16: nothing overflowed,
                // and the accumulators keep ample range); only a half that fails (as every half
                // does while a row has no reference yet, see M_NONE) forms the max of its scores,
                // moves the reference (rescaling O and l) and recomputes.  Rounding is relative, so
                // the reference only has to keep the probabilities in range, not equal the running
                // max.
                const bool lmk = LM && cur.kind == KIND_LM;
                const float bias = lmk ? p.lm_bias_l2 : 0.f;   // landmark logit bias
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    if ((hf ? mhi : mlo) == 0u) continue;   // no key in this half
                    // this half's V operands, requested before the exponentials so that the LDS
                    // reads overlap them
                    bf16x8 va[2][2];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) read_tr(vcur, to, 2 * hf + kk, va[kk][0], va[kk][1]);
                    const f32x16& sp = hf ? s1 : s0;
                    bf16x8 pb[2];
                    float lh;
                    auto probs = [&]() {
                        const float off = lmk ? negm + bias : negm;
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk) {
                            float pv[8];
#pragma unroll
                            for (int i = 0; i < 8; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(sp[8 * kk + i], p.scale_l2, off));
                            bf16x2 pp[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                pp[i] = bf16x2{(__bf16)pv[2 * i], (__bf16)pv[2 * i + 1]};
                                lh = __builtin_amdgcn_fdot2_f32_bf16(pp[i], ones, (kk | i) ? lh : 0.f, false);
                            }
                            pb[kk] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                                             __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                                             0, 1, 2, 3, 4, 5, 6, 7);
                        }
                    };
                    probs();
                    if (__ballot(!(lh <= PROB_SUM_LIMIT))) {
                        float mx = sp[0];
#pragma unroll
                        for (int i = 1; i < 15; i += 2) mx = max3f(mx, sp[i], sp[i + 1]);
                        mx = fmaxf(mx, sp[15]);
                        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                        mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
                        // (a half of -inf scores leaves m alone: fma(-inf, scale, bias) = -inf;
                        // from M_NONE, alpha = 2^(M_NONE - mnew) is 0 or, m unmoved, 1 on a zero O)
                        const float mnew = fmaxf(m, fmaf(mx, p.scale_l2, bias));
                        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
                        l *= alpha;
                        o0 *= alpha;
                        o1 *= alpha;
                        m = mnew;
                        negm = -mnew;
                        probs();
                    }
                    l += lh;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk][0], pb[kk], o0, 0, 0, 0);
                        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk][1], pb[kk], o1, 0, 0, 0);
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WAITCNT_VM0_LGKM0);      // K(it+1), V(it+1) landed; V(it) read
        __builtin_amdgcn_s_barrier();
        dcur = dn;
    };

    TileDesc d{};
    if (ntiles > 0) {
        d = desc(0);
        unsigned v0[NJ], b0;
        plan(d, v0, b0);
        const bool lmk = LM && uniform(d).kind == KIND_LM;
        dma4(lmk ? rs_lk : rs_k, (lds_u8*)s_k, v0, b0);
        dma4(lmk ? rs_lv : rs_v, (lds_u8*)s_v0, v0, b0);
        __builtin_amdgcn_s_waitcnt(WAITCNT_VM0_LGKM0);
        __builtin_amdgcn_s_barrier();
    }
    int it = 0;
    for (; it + 1 < ntiles; it += 2) {
        step(it, d, s_v0, s_v1);
        step(it + 1, d, s_v1, s_v0);
    }
    if (it < ntiles) step(it, d, s_v0, s_v1);

    if (!DENSE && m == M_NONE) m = -INFINITY;         // the row saw no key
    float ltot = l + __shfl_xor(l, 32);
    if (SGA) sga_finish<false>(p, h, qrow, qvalid, g, m, ltot, o0, o1);
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

template <bool F32OUT, bool SGA>
static void launch_t(const AttnDev& d, int heads, bool dense, bool lm, hipStream_t st) {
    const dim3 grid((unsigned)(heads * d.Tq)), block(128);
    const size_t shm = ((lm ? (size_t)(2 * d.nlm) : 0) + (dense ? 0 : (size_t)d.kmax)) *
                       sizeof(uint32_t);
    const int tpfq = d.ql.P / TILE;
    if (dense && d.Tq % 2 == 0 && tpfq % 2 == 0)
        hipLaunchKernelGGL((k_attn_bf16<F32OUT, true, false, SGA, 2>), dim3((unsigned)(heads * d.Tq / 2)),
                           dim3(256), 0, st, d);
    else if (dense) hipLaunchKernelGGL((k_attn_bf16<F32OUT, true, false, SGA>), grid, block, 0, st, d);
    else if (lm) hipLaunchKernelGGL((k_attn_bf16<F32OUT, false, true, SGA>), grid, block, shm, st, d);
    else hipLaunchKernelGGL((k_attn_bf16<F32OUT, false, false, SGA>), grid, block, shm, st, d);
}

hipError_t launch_attn_bf16(const AttnDev& d, int heads, bool dense, bool lm, bool f32out,
                            hipStream_t st) {
    const bool sga = d.sga_kf || d.sga_km;
    if (f32out) sga ? launch_t<true, true>(d, heads, dense, lm, st) : launch_t<true, false>(d, heads, dense, lm, st);
    else sga ? launch_t<false, true>(d, heads, dense, lm, st) : launch_t<false, false>(d, heads, dense, lm, st);
    return hipGetLastError();
}

}  // namespace s3d
