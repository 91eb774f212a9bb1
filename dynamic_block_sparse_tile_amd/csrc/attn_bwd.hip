// Backward of the tile-sparse attention (bf16 operands, fp32 accumulation), for training
// after conversion (Zebra3D abstract: landmark summaries, post-conversion training) and
// sparse training (EPFL "(Full) Attention is More Than You Need").  The selection is held
// fixed (top-k is piecewise constant).  With P the softmax weights (recomputed from the
// forward's log-sum-exp), D = rowsum(dO * O):
//   dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// Three kernels, each with the forward's operand machinery (tile_lds.h):
//  - k_attn_bwd_dq: one workgroup per (head, query tile) walks the query tile's list
//    (special pseudo-tiles, its selected tiles, then with landmarks the blocks of 64 tile
//    means) like the forward and accumulates dQ^T += K^T dS^T; it also writes D.  Each step
//    forms dP for its 64 keys first (the only use of V, whose single buffer then takes the
//    next tile), then S, dS and dQ for one half of 32 keys at a time (K is double
//    buffered): 24 KiB of LDS and at most 168 VGPRs, three waves per SIMD.
//  - k_attn_bwd_dkv<true> (landmarks only): one workgroup per (head, block of 64 tile means)
//    walks every query tile and accumulates the means' gradients dvbar^T += dO^T P and
//    dkbar^T += Q^T dS, a tile's column masked for the query tiles that selected it.
//  - k_attn_bwd_dkv<false>: one workgroup per key block walks the query tiles that attend
//    it (the selection transposed; every query tile for a special pseudo-tile) and
//    accumulates dV^T += dO^T P and dK^T += Q^T dS; with landmarks it adds the means'
//    gradients, divided by the member count, to each member row (the means are averages
//    over the member rows).  Four waves per workgroup: two key halves times two query
//    halves, whose partial sums are added in a fixed order at the end, so three waves share
//    a SIMD.  Every output row gets exactly one writer, so the result is deterministic.
#include <algorithm>

#include "attn_common.h"
#include "device.h"
#include "launch.h"
#include "tile_lds.h"

namespace s3d {

using namespace tl;

namespace {

struct BwdDev {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    Lay ql, kl;
    int Tq, Tk, Ts;
    const int32_t* idx;
    const int32_t* cnt;
    int kmax;
    const int32_t* t_end;
    const int32_t* t_list;
    const void* kbar;    // landmark means [heads, Tk, 64] bf16, or null (no landmarks)
    const void* vbar;
    int nlm;             // blocks of 64 tile means
    float lm_bias_l2;    // landmark logit bias in base-2 units
    float scale, scale_l2;
    float* dq;
    float* dk;
    float* dv;
    float* delta;
    float* dkbar;        // [heads, Tk, 64], landmarks only
    float* dvbar;
};

constexpr float LOG2E_F = 1.4426950408889634f;

// Key/query row r of a 64-row block: where it lives (row within the head) and whether it
// takes part.  kind: 0 = a frame tile t, members only (keys) or valid rows (queries);
// 1 = special pseudo-tile t (gathered special rows of all frames); 2 = block t of the tile
// means (rows 64 t .. 64 t + 63 of kbar/vbar), landmarks of the query tile only.
struct Block {
    int kind, t;
    uint64_t mask;
};

__device__ __forceinline__ int block_row(const Lay& L, const Block& b, int r) {
    if (b.kind == 1) {
        const int e = b.t * TILE + r;
        return (e / L.nsp) * L.P + e % L.nsp;
    }
    return b.t * TILE + r;
}

__device__ __forceinline__ Block key_block(const BwdDev& p, int it, int ts, int c, const int32_t* s_idx,
                                          const uint32_t* s_lm) {
    Block b;
    if (it < ts) {
        b.kind = 1;
        b.t = it;
        b.mask = range_mask(0, min(TILE, p.kl.nsp * p.kl.S - it * TILE));
        return b;
    }
    if (it >= ts + c) {
        b.kind = 2;
        b.t = it - ts - c;
        const uint32_t w0 = __builtin_amdgcn_readfirstlane(s_lm[2 * b.t]);
        const uint32_t w1 = __builtin_amdgcn_readfirstlane(s_lm[2 * b.t + 1]);
        b.mask = (uint64_t)w0 | ((uint64_t)w1 << 32);
        return b;
    }
    b.kind = 0;
    b.t = __builtin_amdgcn_readfirstlane(s_idx[it - ts]);
    if (b.t < 0 || b.t >= p.Tk) {
        b.t = 0;
        b.mask = 0;
    } else {
        int lo, hi;
        member_range(p.kl, b.t, lo, hi);
        b.mask = range_mask(lo, hi);
    }
    return b;
}

// Stage rows of a 64-row block into LDS (this wave's 64 / NW rows, 8-row DMA loads, NW
// waves per workgroup); rows outside `mask` load zeros.
template <int NW = 2>
__device__ __forceinline__ void stage_block(const __amdgpu_buffer_rsrc_t& rs, const Lay& L, const Block& b,
                                            lds_u8* dst, int w, int lane) {
    const int srow_in = lane >> 3, sslot = lane & 7;
    const unsigned base = b.kind == 1 ? 0u : (unsigned)b.t * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < 8 / NW; ++j) {
        const int r = (64 / NW) * w + 8 * j + srow_in;
        unsigned vo = OOB_OFFSET;
        if ((b.mask >> r) & 1ull) {
            const int row_in_block = b.kind == 1 ? block_row(L, b, r) : r;
            vo = (unsigned)row_in_block * 128u + swz(r, sslot) * 16u;
        }
        dma_buf(rs, dst + ((64 / NW) * w + 8 * j) * 128, vo, __builtin_amdgcn_readfirstlane(base));
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, int h, unsigned head_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(static_cast<const unsigned char*>(base)) + (size_t)h * head_bytes, 0,
        (int)head_bytes, BUF_RSRC_WORD3);
}

// 8 bf16 values (16 bytes) as the B operand, or zeros
__device__ __forceinline__ bf16x8 load_b(const void* base, size_t elem, bool ok) {
    const uint4 u = ok ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem)
                       : make_uint4(0, 0, 0, 0);
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float dot_bf16x8(const bf16x8& a, const bf16x8& b, float acc) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)a[i], (float)b[i], acc);
    return acc;
}

}  // namespace

// ------------------------------------------------------------------------------ dQ
template <bool LM>
__global__ __launch_bounds__(128, 3) void k_attn_bwd_dq(BwdDev p) {
    // K is read at both ends of a step (S, then dQ), V only at its start (dP): K is double
    // buffered, V single, reloaded once every wave has formed its dP
    // (one array per buffer: with both K buffers in one array indexed by the step's parity
    // the compiler cannot tell the buffer being read from the one being loaded, and waits
    // for the next tile's loads before reading this one)
    __shared__ __align__(16) unsigned char s_k0[TILE_BYTES];
    __shared__ __align__(16) unsigned char s_k1[TILE_BYTES];
    __shared__ __align__(16) unsigned char s_v[TILE_BYTES];
    extern __shared__ int32_t s_idx[];                  // kmax list entries, then the bitmap
    uint32_t* s_lm = reinterpret_cast<uint32_t*>(s_idx + p.kmax);

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qc = lane & 31, g = lane >> 5;
    const int tpfq = p.ql.P / TILE;
    int h, tq;
    attn_work_item(blockIdx.x, gridDim.x, p.ql.S, tpfq, gridDim.x / p.Tq, h, tq);
    const int Lq = p.ql.S * p.ql.P, Lk = p.kl.S * p.kl.P;
    const int qrow = tq * TILE + w * 32 + qc;
    const bool qvalid = (tq % tpfq) * TILE + w * 32 + qc < p.ql.N;
    const size_t qbase = ((size_t)h * Lq + qrow) * HD;

    bf16x8 qop[4], dop[4];
    float dpart = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        qop[s] = load_b(p.q, qbase + 16 * s + 8 * g, qvalid);
        dop[s] = load_b(p.dout, qbase + 16 * s + 8 * g, qvalid);
        dpart = dot_bf16x8(dop[s], load_b(p.o, qbase + 16 * s + 8 * g, qvalid), dpart);
    }
    const float D = dpart + __shfl_xor(dpart, 32);       // rowsum(dO * O), both halves
    // a wave whose 32 query rows are all padding stages and meets the barriers but skips
    // the products
    const bool wq = __ballot(qvalid) != 0ull;
    const float lse = qvalid ? p.lse[(size_t)h * Lq + qrow] : INFINITY;
    // base-2 offset of P = exp(s - lse); a row with nothing attended (lse = -inf) or not a
    // query gets P = 0
    const float lse_l2 = (qvalid && lse > -INFINITY) ? lse * LOG2E_F : INFINITY;
    if (g == 0) p.delta[(size_t)h * Lq + qrow] = qvalid ? D : 0.f;
    __builtin_amdgcn_s_waitcnt(0);

    const int c = min(max(p.cnt[(size_t)h * p.Tq + tq], 0), p.kmax);
    const int32_t* myidx = p.idx + ((size_t)h * p.Tq + tq) * p.kmax;
    for (int i = tid; i < c; i += 128) s_idx[i] = myidx[i];
    if (LM) init_landmark_bitmap(p.kl, p.Tk, p.nlm, c, myidx, s_lm, tid, 128);   // has barriers
    __syncthreads();
    const int ntiles = p.Ts + c + (LM ? p.nlm : 0);

    const unsigned head_bytes = (unsigned)Lk * 128u;
    const __amdgpu_buffer_rsrc_t rs_k = head_rsrc(p.k, h, head_bytes);
    const __amdgpu_buffer_rsrc_t rs_v = head_rsrc(p.v, h, head_bytes);
    // the tile means of this head: Tk rows of 128 bytes
    const unsigned mean_bytes = (unsigned)p.Tk * 128u;
    const __amdgpu_buffer_rsrc_t rs_kb = head_rsrc(LM ? p.kbar : p.k, h, LM ? mean_bytes : head_bytes);
    const __amdgpu_buffer_rsrc_t rs_vb = head_rsrc(LM ? p.vbar : p.v, h, LM ? mean_bytes : head_bytes);
    TileOffsets off;
    off.init(lane);

    f32x16 dq0 = {}, dq1 = {};
    auto stage_k = [&](int it, unsigned char* dst) {
        const Block kb = key_block(p, it, p.Ts, c, s_idx, s_lm);
        const bool mean = LM && __builtin_amdgcn_readfirstlane(kb.kind) == 2;
        stage_block(mean ? rs_kb : rs_k, p.kl, kb, (lds_u8*)dst, w, lane);
        return kb;
    };
    auto stage_v = [&](const Block& kb) {
        const bool mean = LM && __builtin_amdgcn_readfirstlane(kb.kind) == 2;
        stage_block(mean ? rs_vb : rs_v, p.kl, kb, (lds_u8*)s_v, w, lane);
    };
    Block cur{}, nxt{};
    if (ntiles > 0) {
        cur = stage_k(0, s_k0);
        stage_v(cur);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    // step it reads K(it) from kt while K(it+1) loads into kn (steps alternate the buffers)
    auto kstep = [&](int it, const unsigned char* kt, unsigned char* kn) __attribute__((always_inline)) {
        if (it + 1 < ntiles) nxt = stage_k(it + 1, kn);
        const unsigned char* vt = s_v;
        // landmark logits carry the bias
        const float nl = (LM && __builtin_amdgcn_readfirstlane(cur.kind) == 2 ? p.lm_bias_l2 : 0.f) - lse_l2;
        const uint64_t km = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(cur.mask >> 32)) << 32) |
                            __builtin_amdgcn_readfirstlane((uint32_t)cur.mask);
        // keys 32 hk .. 32 hk + 31 of the step: S^T and dP^T (lane = query column), then
        // dS^T = P^T (dP^T - D) with key rows outside the block's mask taking no part, then
        // dQ^T += K^T dS^T over the half's two k-steps
        auto products = [&](int hk, f32x16& acc, const unsigned char* t, const bf16x8 (&op)[4]) {
            acc = f32x16{};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(t + off.row[st] + 4096 * hk));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, op[st], acc, 0, 0, 0);
            }
        };
        auto finish = [&](int hk, const f32x16& sk, f32x16& pk) {
            const uint32_t wm = (uint32_t)(km >> (32 * hk));
            if (wm == 0xffffffffu) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    pk[r] = __builtin_amdgcn_exp2f(fmaf(sk[r], p.scale_l2, nl)) * (pk[r] - D);
            } else {
                // this lane's keys 8i + 4g + (0..3) of the half, tested against constant bits
                const uint32_t wl = wm >> (4 * g);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t bit = 1u << (8 * (r >> 2) + (r & 3));
                    const float pa = (wl & bit) ? __builtin_amdgcn_exp2f(fmaf(sk[r], p.scale_l2, nl)) : 0.f;
                    pk[r] = pa * (pk[r] - D);
                }
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 a0, a1;
                read_tr(kt, off, 2 * hk + kk, a0, a1);
                const bf16x8 bs = acc_to_b(pk, pk, kk, [](float x, int, int) { return x; });
                dq0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bs, dq0, 0, 0, 0);
                dq1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bs, dq1, 0, 0, 0);
            }
        };
        f32x16 p0, p1;
        if (wq) {                                            // dP of both halves: every V read
            products(0, p0, vt, dop);
            products(1, p1, vt, dop);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);          // this wave's V reads are done
        // and every wave's (a plain barrier: __syncthreads would also wait for K(it+1)'s loads)
        __builtin_amdgcn_s_barrier();
        if (it + 1 < ntiles) stage_v(nxt);                   // V(it+1) into the one V buffer
        __builtin_amdgcn_sched_barrier(0);
        if (wq) {                                            // S, dS and dQ half by half
            f32x16 s0;
            products(0, s0, kt, qop);
            finish(0, s0, p0);
            __builtin_amdgcn_sched_barrier(0);
            f32x16 s1;
            products(1, s1, kt, qop);
            finish(1, s1, p1);
        }
        cur = nxt;
        __builtin_amdgcn_s_waitcnt(0x0070);
        __syncthreads();
    };
    int it = 0;
    for (; it + 1 < ntiles; it += 2) {
        kstep(it, s_k0, s_k1);
        kstep(it + 1, s_k1, s_k0);
    }
    if (it < ntiles) kstep(it, s_k0, s_k1);
    // dQ = scale * dQ^T accumulators: lane holds query qc, dims 8 (r/4) + 4 g + r % 4 (+32)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const f32x16& acc = cb ? dq1 : dq0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c0 = 32 * cb + 8 * j + 4 * g;
            const float4 v4 = qvalid ? make_float4(acc[4 * j] * p.scale, acc[4 * j + 1] * p.scale,
                                                   acc[4 * j + 2] * p.scale, acc[4 * j + 3] * p.scale)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<float4*>(p.dq + qbase + c0) = v4;
        }
    }
}

// ------------------------------------------------------------------------------ dK, dV
// MEANS = false: work items are H * Ts special pseudo-tiles first (attended by every query
// tile, the longest items), then H * Tk frame tiles, taken in launch order: workgroup i runs
// on XCD i % 8, so the long special items spread evenly over the XCDs and all XCDs work
// through the same head's key tiles at a time (their query tiles then share the last-level
// cache).  Giving each XCD a contiguous range of items instead put every special item on
// one XCD, which then carried about 40 % more work than the others.
// MEANS = true: work items are H * nlm blocks of 64 tile means, each walking every query
// tile in order (all items stream the same query tiles, which then come from the cache).
// Lane (w, kc) owns key tile t = 64 b + 32 w + kc, a landmark of every query tile that did
// not select it; those that did are the ascending entries of t's transposed list, which the
// lane walks in step with the loop (one comparison per query tile; the next entry loads
// under the step's products).
template <bool MEANS>
__global__ __launch_bounds__(256, MEANS ? 2 : 3) void k_attn_bwd_dkv(BwdDev p) {
    // the staging buffers (32 KiB) also carry the query halves' partial sums at the end
    __shared__ __align__(16) unsigned char s_q[2][TILE_BYTES];
    __shared__ __align__(16) unsigned char s_do[2][TILE_BYTES];
    __shared__ __align__(16) float s_lse[2][TILE];
    __shared__ __align__(16) float s_d[2][TILE];

    // four waves: wave w owns key rows 32 (w & 1) .. + 31 of the block and query rows
    // 32 (w >> 1) .. + 31 of every query tile; the two query halves' partial sums of dK and dV
    // are added in a fixed order at the end
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wk_half = w & 1, qh = w >> 1;
    const int kc = lane & 31, g = lane >> 5;
    const int kr = 32 * wk_half + kc;                            // key row within the block
    const int Lq = p.ql.S * p.ql.P, Lk = p.kl.S * p.kl.P;
    int h;
    Block kb;
    bool kvalid;
    size_t kbase;                                                // this lane's key row (elements)
    int sel_next = 0x7fffffff, sel_pos = 0, sel_end = 0;         // MEANS: the lane's transposed list
    const int32_t* sel_list = nullptr;
    if (MEANS) {
        h = blockIdx.x / p.nlm;
        kb.kind = 2;
        kb.t = blockIdx.x - h * p.nlm;
        const int t = kb.t * TILE + kr;
        kvalid = false;
        if (t < p.Tk) {
            int lo, hi;
            member_range(p.kl, t, lo, hi);
            kvalid = hi > lo;
            const int32_t* te = p.t_end + (size_t)h * p.Tk;
            sel_pos = t == 0 ? 0 : te[t - 1];
            sel_end = te[t];
        }
        kbase = ((size_t)h * p.Tk + min(t, p.Tk - 1)) * HD;
        if (p.t_list) {
            sel_list = p.t_list + (size_t)h * p.Tq * p.kmax;
            if (sel_pos < sel_end) sel_next = sel_list[sel_pos];
        }
    } else {
        const int heads = gridDim.x / (p.Ts + p.Tk);
        const int item = blockIdx.x;
        const int nspec = heads * p.Ts;
        if (item < nspec) {
            h = item / p.Ts;
            kb.kind = 1;
            kb.t = item - h * p.Ts;
            kb.mask = range_mask(0, min(TILE, p.kl.nsp * p.kl.S - kb.t * TILE));
        } else {
            const int r = item - nspec;
            h = r / p.Tk;
            kb.kind = 0;
            kb.t = r - h * p.Tk;
            int lo, hi;
            member_range(p.kl, kb.t, lo, hi);
            kb.mask = range_mask(lo, hi);
        }
        kvalid = (kb.mask >> kr) & 1ull;
        kbase = ((size_t)h * Lk + block_row(p.kl, kb, kr)) * HD;
    }
    // a wave with no key row in this block stages and meets the barriers but skips the
    // products (its accumulators stay zero)
    const bool wk = __ballot(kvalid) != 0ull;

    const void* ksrc = MEANS ? p.kbar : p.k;
    const void* vsrc = MEANS ? p.vbar : p.v;
    bf16x8 kop[4], vop[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        kop[s] = load_b(ksrc, kbase + 16 * s + 8 * g, kvalid);
        vop[s] = load_b(vsrc, kbase + 16 * s + 8 * g, kvalid);
    }
    __builtin_amdgcn_s_waitcnt(0);

    // the query tiles that attend this block
    int nq, q0 = 0;
    const int32_t* qlist = nullptr;
    if (MEANS || kb.kind == 1) {
        nq = p.Tq;
    } else {
        const int32_t* te = p.t_end + (size_t)h * p.Tk;
        q0 = kb.t == 0 ? 0 : te[kb.t - 1];
        nq = te[kb.t] - q0;
        qlist = p.t_list + (size_t)h * p.Tq * p.kmax + q0;
    }
    // the list through the constant address space: a uniform index makes a scalar load, which
    // does not wait behind the vector loads in flight
    typedef __attribute__((address_space(4))) const int32_t cint32;
    cint32* const qlist_s = (cint32*)qlist;
    auto qtile = [&](int i) {
        return (MEANS || kb.kind == 1) ? i : (int)qlist_s[i];
    };

    const unsigned head_bytes = (unsigned)Lq * 128u;
    const __amdgpu_buffer_rsrc_t rs_q = head_rsrc(p.q, h, head_bytes);
    const __amdgpu_buffer_rsrc_t rs_do = head_rsrc(p.dout, h, head_bytes);
    TileOffsets off;
    off.init(lane);
    const int tpfq = p.ql.P / TILE;

    // lse and D of the 64 rows of a query tile, one value per thread of the first 64 (lse,
    // +inf for rows that are not queries) and last 64 (D) lanes.  The value is stored as
    // loaded and converted (row_value) when it goes to LDS at the end of the step: converted
    // at once, its use would wait for the load, and so (loads complete in order) for the
    // staging loads of the next tile issued just before it.
    auto fetch_rows = [&](int tq, float& val) {
        const int r = tid & 63;
        const int row = tq * TILE + r;
        const bool ok = (tq % tpfq) * TILE + r < p.ql.N;
        if (tid < 64) val = ok ? p.lse[(size_t)h * Lq + row] : INFINITY;
        else val = ok ? p.delta[(size_t)h * Lq + row] : 0.f;
    };
    // as the steps read them: lse in base 2 (+inf, so P = 0, for a row with nothing attended
    // or not a query), D as it is
    auto row_value = [&](float val) {
        return tid < 64 ? (val > -INFINITY ? val * LOG2E_F : INFINITY) : val;
    };
    auto stage = [&](int tq, int b) {
        Block qb;
        qb.kind = 0;
        qb.t = tq;
        qb.mask = range_mask(0, valid_rows(p.ql, tq));
        stage_block<4>(rs_q, p.ql, qb, (lds_u8*)s_q[b], w, lane);
        stage_block<4>(rs_do, p.ql, qb, (lds_u8*)s_do[b], w, lane);
    };

    f32x16 dk0 = {}, dk1 = {}, dv0 = {}, dv1 = {};
    float rowval = 0.f;
    if (nq > 0) {
        const int t0 = qtile(0);
        stage(t0, 0);
        if (tid < 128) fetch_rows(t0, rowval);
        __builtin_amdgcn_s_waitcnt(0x0070);
        if (tid < 128) (tid < 64 ? s_lse[0] : s_d[0])[tid & 63] = row_value(rowval);
    }
    __syncthreads();
    for (int i = 0; i < nq; ++i) {
        const int b = i & 1;
        if (i + 1 < nq) {
            const int tn = qtile(i + 1);
            stage(tn, b ^ 1);
            if (tid < 128) fetch_rows(tn, rowval);
        }
        // exponent offset of this lane's key column: 0 for keys, the landmark bias for a
        // tile mean that query tile i did not select, -inf (P = 0) otherwise
        float nb = 0.f;
        if (MEANS) {
            while (sel_next < i) {                               // a tile listed twice in a row
                ++sel_pos;
                sel_next = sel_pos < sel_end ? sel_list[sel_pos] : 0x7fffffff;
            }
            const bool selected = sel_next == i;
            if (selected) {
                ++sel_pos;
                sel_next = sel_pos < sel_end ? sel_list[sel_pos] : 0x7fffffff;
            }
            nb = (kvalid && !selected) ? p.lm_bias_l2 : -INFINITY;
        }
        const unsigned char* qt = s_q[b];
        const unsigned char* dt = s_do[b];
        if (wk) {
            // S = Q K^T and dP = dO V^T over this wave's 32 query rows (lane = key column)
            f32x16 sq = {}, pq = {};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qt + off.row[st] + 4096 * qh));
                const bf16x8 o = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(dt + off.row[st] + 4096 * qh));
                sq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kop[st], sq, 0, 0, 0);
                pq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, vop[st], pq, 0, 0, 0);
            }
            // P (in sq) and dS (in pq) per query row 32 qh + 8 (r/4) + 4 g + r % 4
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int q4 = 32 * qh + 8 * a + 4 * g;
                const float4 la = *reinterpret_cast<const float4*>(&s_lse[b][q4]);
                const float4 da = *reinterpret_cast<const float4*>(&s_d[b][q4]);
                const float lav[4] = {la.x, la.y, la.z, la.w}, dav[4] = {da.x, da.y, da.z, da.w};
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int r = 4 * a + i4;
                    sq[r] = __builtin_amdgcn_exp2f(fmaf(sq[r], p.scale_l2, nb - lav[i4]));
                    pq[r] = sq[r] * (pq[r] - dav[i4]);
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS over the wave's queries (k-steps 2 qh, 2 qh + 1)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int ks = 2 * qh + kk;
                bf16x8 a0, a1, c0, c1;
                read_tr(dt, off, ks, a0, a1);
                read_tr(qt, off, ks, c0, c1);
                const bf16x8 bp = acc_to_b(sq, sq, kk, [](float x, int, int) { return x; });
                const bf16x8 bd = acc_to_b(pq, pq, kk, [](float x, int, int) { return x; });
                dv0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bp, dv0, 0, 0, 0);
                dv1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bp, dv1, 0, 0, 0);
                dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c0, bd, dk0, 0, 0, 0);
                dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c1, bd, dk1, 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0070);
        if (i + 1 < nq && tid < 128) (tid < 64 ? s_lse[b ^ 1] : s_d[b ^ 1])[tid & 63] = row_value(rowval);
        __syncthreads();
    }
    // the second query half hands its partial sums to the first through the staging buffers
    // (the loop's last barrier is behind every read of them), which adds them in this order
    {
        float* red = reinterpret_cast<float*>(wk_half ? &s_do[0][0] : &s_q[0][0]);   // 16 KiB per key half
        if (qh == 1) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                red[(0 * 16 + r) * 64 + lane] = dk0[r];
                red[(1 * 16 + r) * 64 + lane] = dk1[r];
                red[(2 * 16 + r) * 64 + lane] = dv0[r];
                red[(3 * 16 + r) * 64 + lane] = dv1[r];
            }
        }
        __syncthreads();
        if (qh == 1) return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk0[r] += red[(0 * 16 + r) * 64 + lane];
            dk1[r] += red[(1 * 16 + r) * 64 + lane];
            dv0[r] += red[(2 * 16 + r) * 64 + lane];
            dv1[r] += red[(3 * 16 + r) * 64 + lane];
        }
    }
    float* dk_out = MEANS ? p.dkbar : p.dk;
    float* dv_out = MEANS ? p.dvbar : p.dv;
    // MEANS: every tile's row (zeros for tiles without members).  Otherwise member rows of a
    // frame tile (pad rows get zeros; special rows inside the tile belong to the special
    // pseudo-tiles) and every special row of a pseudo-tile.
    bool write;
    if (MEANS) {
        write = kb.t * TILE + kr < p.Tk;
    } else {
        write = kvalid;
        if (kb.kind == 0 && !kvalid) write = block_row(p.kl, kb, kr) % p.kl.P >= p.kl.N;   // pad
    }
    if (!write) return;
    // with landmarks, a member row also takes its tile mean's gradient over the member count
    const bool chain = !MEANS && p.dkbar != nullptr && kb.kind == 0 && kvalid;
    float inv = 0.f;
    const float* mk = nullptr;
    const float* mv = nullptr;
    if (chain) {
        int lo, hi;
        member_range(p.kl, kb.t, lo, hi);
        inv = 1.f / (float)(hi - lo);
        mk = p.dkbar + ((size_t)h * p.Tk + kb.t) * HD;
        mv = p.dvbar + ((size_t)h * p.Tk + kb.t) * HD;
    }
    const float sk = kvalid ? p.scale : 0.f, sv = kvalid ? 1.f : 0.f;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const f32x16& ak = cb ? dk1 : dk0;
        const f32x16& av = cb ? dv1 : dv0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c0 = 32 * cb + 8 * j + 4 * g;
            float4 k4 = make_float4(ak[4 * j] * sk, ak[4 * j + 1] * sk, ak[4 * j + 2] * sk, ak[4 * j + 3] * sk);
            float4 v4 = make_float4(av[4 * j] * sv, av[4 * j + 1] * sv, av[4 * j + 2] * sv, av[4 * j + 3] * sv);
            if (chain) {
                const float4 gk = *reinterpret_cast<const float4*>(mk + c0);
                const float4 gv = *reinterpret_cast<const float4*>(mv + c0);
                k4 = make_float4(fmaf(gk.x, inv, k4.x), fmaf(gk.y, inv, k4.y), fmaf(gk.z, inv, k4.z),
                                 fmaf(gk.w, inv, k4.w));
                v4 = make_float4(fmaf(gv.x, inv, v4.x), fmaf(gv.y, inv, v4.y), fmaf(gv.z, inv, v4.z),
                                 fmaf(gv.w, inv, v4.w));
            }
            *reinterpret_cast<float4*>(dk_out + kbase + c0) = k4;
            *reinterpret_cast<float4*>(dv_out + kbase + c0) = v4;
        }
    }
}

// ------------------------------------------------------------------------------ transpose
__global__ void k_fill_i32(int32_t* x, size_t n, int32_t v) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        x[i] = v;
}

// count, then (after the scan) place: one thread per (head, query tile, list entry)
template <bool FILL>
__global__ void k_tr_scatter(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int Tq,
                             int kmax, int Tk, int32_t* __restrict__ t_end, int32_t* __restrict__ t_list,
                             size_t total) {
    const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int e = (int)(i % kmax);
    const size_t row = i / kmax;                                  // h * Tq + tq
    const int c = min(max(cnt[row], 0), kmax);
    if (e >= c) return;
    const int t = idx[i];
    if (t < 0 || t >= Tk) return;
    const int h = (int)(row / Tq), tq = (int)(row % Tq);
    int32_t* slot = t_end + (size_t)h * Tk + t;
    if (!FILL) {
        atomicAdd(slot, 1);
    } else {
        const int pos = atomicAdd(slot, 1);
        t_list[(size_t)h * Tq * kmax + pos] = tq;
    }
}

// exclusive scan of the counts of one head, in place (one workgroup per head)
constexpr int SCAN_THREADS = 1024;
__global__ __launch_bounds__(SCAN_THREADS) void k_tr_scan(int32_t* t_end, int Tk) {
    __shared__ int32_t s_part[SCAN_THREADS];
    int32_t* x = t_end + (size_t)blockIdx.x * Tk;
    const int per = (Tk + SCAN_THREADS - 1) / SCAN_THREADS;
    const int b = threadIdx.x * per, e = min(Tk, b + per);
    int32_t sum = 0;
    for (int i = b; i < e; ++i) sum += x[i];
    s_part[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < SCAN_THREADS; off <<= 1) {            // inclusive Hillis-Steele
        const int32_t v = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
        __syncthreads();
        s_part[threadIdx.x] += v;
        __syncthreads();
    }
    int32_t run = threadIdx.x ? s_part[threadIdx.x - 1] : 0;
    for (int i = b; i < e; ++i) {
        const int32_t c = x[i];
        x[i] = run;
        run += c;
    }
}

// Order each key tile's list ascending.  The entries are distinct query tiles (a selection
// row names a tile once), so the list is a set: mark its members in an LDS bitmap of Tq bits
// and write them back in bit order, each thread a contiguous run of words at the offset a
// block scan of the word popcounts gives.  A list whose marks do not add up to its length
// (a row that repeats a tile, or an index outside [0, Tq)) is sorted by a bitonic network.
constexpr int SORT_THREADS = 256;
constexpr int TR_WORDS_MAX = 512;                     // bitmap words: Tq <= 16384
__global__ __launch_bounds__(SORT_THREADS) void k_tr_sort(const int32_t* __restrict__ t_end,
                                                          int32_t* __restrict__ t_list, int Tq, int kmax,
                                                          int Tk, int cap) {
    extern __shared__ int32_t s_v[];                  // cap entries (a power of two >= Tq)
    __shared__ uint32_t s_bits[TR_WORDS_MAX];
    __shared__ int s_part[SORT_THREADS];
    const int tid = threadIdx.x;
    const int h = blockIdx.x / Tk, t = blockIdx.x % Tk;
    const int32_t* te = t_end + (size_t)h * Tk;
    const int b = t == 0 ? 0 : te[t - 1];
    // a list is at most Tq long unless a selection row repeats a tile; never exceed LDS
    const int n = min(te[t] - b, cap);
    if (n <= 1) return;
    int32_t* seg = t_list + (size_t)h * Tq * kmax + b;
    const int nw = (Tq + 31) >> 5;
    for (int i = tid; i < nw; i += SORT_THREADS) s_bits[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += SORT_THREADS) {
        const int v = seg[i];
        if (v >= 0 && v < Tq) atomicOr(&s_bits[v >> 5], 1u << (v & 31));
    }
    __syncthreads();
    const int per = (nw + SORT_THREADS - 1) / SORT_THREADS;
    const int w0 = min(tid * per, nw), w1 = min(w0 + per, nw);
    int local = 0;
    for (int w = w0; w < w1; ++w) local += __popc(s_bits[w]);
    s_part[tid] = local;
    __syncthreads();
    for (int off = 1; off < SORT_THREADS; off <<= 1) {   // inclusive Hillis-Steele scan
        const int v = tid >= off ? s_part[tid - off] : 0;
        __syncthreads();
        s_part[tid] += v;
        __syncthreads();
    }
    const int total = s_part[SORT_THREADS - 1];
    if (total == n) {
        int pos = s_part[tid] - local;
        for (int w = w0; w < w1; ++w) {
            uint32_t m = s_bits[w];
            while (m) {
                seg[pos++] = 32 * w + __builtin_ctz(m);
                m &= m - 1u;
            }
        }
        return;
    }
    int np = 1;
    while (np < n) np <<= 1;
    for (int i = tid; i < np; i += SORT_THREADS) s_v[i] = i < n ? seg[i] : 0x7fffffff;
    __syncthreads();
    for (int k = 2; k <= np; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < np; i += SORT_THREADS) {
                const int l = i ^ j;
                if (l > i) {
                    const bool up = (i & k) == 0;
                    const int32_t a = s_v[i], c = s_v[l];
                    if ((a > c) == up) {
                        s_v[i] = c;
                        s_v[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < n; i += SORT_THREADS) seg[i] = s_v[i];
}

hipError_t launch_selection_transpose(const int32_t* idx, const int32_t* cnt, int heads, int tq, int tk,
                                      int kmax, int32_t* t_end, int32_t* t_list, hipStream_t st) {
    const size_t ne = (size_t)heads * tk;
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)std::min<size_t>((ne + 255) / 256, 4096)), dim3(256), 0, st,
                       t_end, ne, 0);
    const size_t total = (size_t)heads * tq * kmax;
    if (total > 0) {
        const unsigned blocks = (unsigned)((total + 255) / 256);
        hipLaunchKernelGGL(k_tr_scatter<false>, dim3(blocks), dim3(256), 0, st, idx, cnt, tq, kmax, tk, t_end,
                           t_list, total);
        hipLaunchKernelGGL(k_tr_scan, dim3((unsigned)heads), dim3(SCAN_THREADS), 0, st, t_end, tk);
        hipLaunchKernelGGL(k_tr_scatter<true>, dim3(blocks), dim3(256), 0, st, idx, cnt, tq, kmax, tk, t_end,
                           t_list, total);
        int np = 1;
        while (np < tq) np <<= 1;
        hipLaunchKernelGGL(k_tr_sort, dim3((unsigned)ne), dim3(SORT_THREADS), (size_t)np * 4, st, t_end, t_list,
                           tq, kmax, tk, np);
    }
    return hipGetLastError();
}

hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t st) {
    BwdDev d;
    d.q = a.q;
    d.k = a.k;
    d.v = a.v;
    d.o = a.out;
    d.dout = a.dout;
    d.lse = a.lse;
    d.ql = Lay{a.ql.S, a.ql.N, a.ql.P, a.ql.nsp};
    d.kl = Lay{a.kl.S, a.kl.N, a.kl.P, a.kl.nsp};
    d.Tq = a.ql.S * a.ql.P / TILE;
    d.Tk = a.kl.S * a.kl.P / TILE;
    d.Ts = (a.kl.nsp * a.kl.S + TILE - 1) / TILE;
    d.idx = a.idx;
    d.cnt = a.cnt;
    d.kmax = a.kmax;
    d.t_end = a.t_end;
    d.t_list = a.t_list;
    const bool lm = a.kbar != nullptr;
    d.kbar = a.kbar;
    d.vbar = a.vbar;
    d.nlm = lm ? (d.Tk + TILE - 1) / TILE : 0;
    d.lm_bias_l2 = a.landmark_bias * LOG2E_F;
    d.scale = a.scale;
    d.scale_l2 = a.scale * LOG2E_F;
    d.dq = a.dq;
    d.dk = a.dk;
    d.dv = a.dv;
    d.delta = a.delta;
    d.dkbar = lm ? a.dkbar : nullptr;
    d.dvbar = lm ? a.dvbar : nullptr;
    const size_t shm = ((size_t)a.kmax + 2 * (size_t)d.nlm) * 4;
    const dim3 gq((unsigned)(a.heads * d.Tq));
    if (lm)
        hipLaunchKernelGGL(k_attn_bwd_dq<true>, gq, dim3(128), shm, st, d);
    else
        hipLaunchKernelGGL(k_attn_bwd_dq<false>, gq, dim3(128), shm, st, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the means' gradients first: the dK/dV kernel adds them to the member rows
    if (lm) {
        hipLaunchKernelGGL(k_attn_bwd_dkv<true>, dim3((unsigned)(a.heads * d.nlm)), dim3(256), 0, st, d);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_attn_bwd_dkv<false>, dim3((unsigned)(a.heads * (d.Ts + d.Tk))), dim3(256), 0, st, d);
    return hipGetLastError();
}

}  // namespace s3d
