// Backward of the tile-sparse attention (bf16 operands, fp32 accumulation), for training
// after conversion (Zebra3D abstract) and sparse training (EPFL "(Full) Attention is More
// Than You Need").  The selection is held fixed (top-k is piecewise constant).  With P the
// softmax weights (recomputed from the forward's log-sum-exp), D = rowsum(dO * O):
//   dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// Two kernels, each with the forward's operand machinery (tile_lds.h):
//  - k_attn_bwd_dq: one workgroup per (head, query tile) walks the query tile's list
//    (special pseudo-tiles, then its selected tiles) like the forward and accumulates
//    dQ^T += K^T dS^T; it also writes D.
//  - k_attn_bwd_dkv: one workgroup per key block walks the query tiles that attend it (the
//    selection transposed; every query tile for a special pseudo-tile) and accumulates
//    dV^T += dO^T P and dK^T += Q^T dS.  Every key row gets exactly one writer, so the
//    result is deterministic.
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
    float scale, scale_l2;
    float* dq;
    float* dk;
    float* dv;
    float* delta;
};

constexpr float LOG2E_F = 1.4426950408889634f;

// Key/query row r of a 64-row block: where it lives (row within the head) and whether it
// takes part.  kind: 0 = a frame tile t, members only (keys) or valid rows (queries);
// 1 = special pseudo-tile t (gathered special rows of all frames).
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

__device__ __forceinline__ Block key_block(const BwdDev& p, int it, int ts, const int32_t* s_idx) {
    Block b;
    if (it < ts) {
        b.kind = 1;
        b.t = it;
        b.mask = range_mask(0, min(TILE, p.kl.nsp * p.kl.S - it * TILE));
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

// Stage rows of a 64-row block into LDS (this wave's 32 rows, four 8-row DMA loads);
// rows outside `mask` load zeros.
__device__ __forceinline__ void stage_block(const __amdgpu_buffer_rsrc_t& rs, const Lay& L, const Block& b,
                                            lds_u8* dst, int w, int lane) {
    const int srow_in = lane >> 3, sslot = lane & 7;
    const unsigned base = b.kind == 1 ? 0u : (unsigned)b.t * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 32 * w + 8 * j + srow_in;
        unsigned vo = OOB_OFFSET;
        if ((b.mask >> r) & 1ull) {
            const int row_in_block = b.kind == 1 ? block_row(L, b, r) : r;
            vo = (unsigned)row_in_block * 128u + swz(r, sslot) * 16u;
        }
        dma_buf(rs, dst + (32 * w + 8 * j) * 128, vo, __builtin_amdgcn_readfirstlane(base));
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
__global__ __launch_bounds__(128, 2) void k_attn_bwd_dq(BwdDev p) {
    __shared__ __align__(16) unsigned char s_k[2][TILE_BYTES];
    __shared__ __align__(16) unsigned char s_v[2][TILE_BYTES];
    extern __shared__ int32_t s_idx[];

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
    __syncthreads();
    const int ntiles = p.Ts + c;

    const unsigned head_bytes = (unsigned)Lk * 128u;
    const __amdgpu_buffer_rsrc_t rs_k = head_rsrc(p.k, h, head_bytes);
    const __amdgpu_buffer_rsrc_t rs_v = head_rsrc(p.v, h, head_bytes);
    TileOffsets off;
    off.init(lane);

    f32x16 dq0 = {}, dq1 = {};
    auto stage = [&](int it, int b) {
        const Block kb = key_block(p, it, p.Ts, s_idx);
        stage_block(rs_k, p.kl, kb, (lds_u8*)s_k[b], w, lane);
        stage_block(rs_v, p.kl, kb, (lds_u8*)s_v[b], w, lane);
        return kb;
    };
    Block cur{}, nxt{};
    if (ntiles > 0) cur = stage(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int b = it & 1;
        if (it + 1 < ntiles) nxt = stage(it + 1, b ^ 1);
        const unsigned char* kt = s_k[b];
        const unsigned char* vt = s_v[b];
        if (wq) {
            f32x16 s0 = {}, s1 = {}, p0 = {}, p1 = {};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                bf16x8 a0, a1, v0, v1;
                read_rows(kt, off, st, a0, a1);
                read_rows(vt, off, st, v0, v1);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qop[st], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qop[st], s1, 0, 0, 0);
                p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, dop[st], p0, 0, 0, 0);
                p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, dop[st], p1, 0, 0, 0);
            }
            // dS^T = P^T (dP^T - D); key rows outside the block's mask take no part
            // this lane's keys 8i + 4g + (0..3) of each half, tested against constant bits
            const uint32_t w0 = __builtin_amdgcn_readfirstlane((uint32_t)cur.mask) >> (4 * g);
            const uint32_t w1 = __builtin_amdgcn_readfirstlane((uint32_t)(cur.mask >> 32)) >> (4 * g);
            f32x16 d0, d1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t bit = 1u << (8 * (r >> 2) + (r & 3));
                const float pa = (w0 & bit) ? __builtin_amdgcn_exp2f(fmaf(s0[r], p.scale_l2, -lse_l2)) : 0.f;
                const float pb = (w1 & bit) ? __builtin_amdgcn_exp2f(fmaf(s1[r], p.scale_l2, -lse_l2)) : 0.f;
                d0[r] = pa * (p0[r] - D);
                d1[r] = pb * (p1[r] - D);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 a0, a1;
                read_tr(kt, off, ks, a0, a1);
                const bf16x8 bs = acc_to_b(d0, d1, ks, [](float x, int, int) { return x; });
                dq0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bs, dq0, 0, 0, 0);
                dq1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bs, dq1, 0, 0, 0);
            }
        }
        cur = nxt;
        __builtin_amdgcn_s_waitcnt(0x0070);
        __syncthreads();
    }
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
// Work items: H * Ts special pseudo-tiles first (attended by every query tile, the longest
// items), then H * Tk frame tiles, taken in launch order: workgroup i runs on XCD i % 8, so
// the long special items spread evenly over the XCDs and all XCDs work through the same
// head's key tiles at a time (their query tiles then share the last-level cache).  Giving
// each XCD a contiguous range of items instead put every special item on one XCD, which
// then carried about 40 % more work than the others.
__global__ __launch_bounds__(128, 2) void k_attn_bwd_dkv(BwdDev p) {
    __shared__ __align__(16) unsigned char s_q[2][TILE_BYTES];
    __shared__ __align__(16) unsigned char s_do[2][TILE_BYTES];
    __shared__ __align__(16) float s_lse[2][TILE];
    __shared__ __align__(16) float s_d[2][TILE];

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int kc = lane & 31, g = lane >> 5;
    const int heads = gridDim.x / (p.Ts + p.Tk);
    const int item = blockIdx.x;
    const int nspec = heads * p.Ts;
    int h;
    Block kb;
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
    const int Lq = p.ql.S * p.ql.P, Lk = p.kl.S * p.kl.P;
    const int kr = 32 * w + kc;                                  // key row within the block
    const bool kvalid = (kb.mask >> kr) & 1ull;
    const int krow = block_row(p.kl, kb, kr);                    // row within the head
    // a wave with no key row in this block stages and meets the barriers but skips the
    // products (its accumulators stay zero)
    const bool wk = __ballot(kvalid) != 0ull;
    const size_t kbase = ((size_t)h * Lk + krow) * HD;

    bf16x8 kop[4], vop[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        kop[s] = load_b(p.k, kbase + 16 * s + 8 * g, kvalid);
        vop[s] = load_b(p.v, kbase + 16 * s + 8 * g, kvalid);
    }
    __builtin_amdgcn_s_waitcnt(0);

    // the query tiles that attend this block
    int nq, q0 = 0;
    const int32_t* qlist = nullptr;
    if (kb.kind == 1) {
        nq = p.Tq;
    } else {
        const int32_t* te = p.t_end + (size_t)h * p.Tk;
        q0 = kb.t == 0 ? 0 : te[kb.t - 1];
        nq = te[kb.t] - q0;
        qlist = p.t_list + (size_t)h * p.Tq * p.kmax + q0;
    }
    auto qtile = [&](int i) { return kb.kind == 1 ? i : __builtin_amdgcn_readfirstlane(qlist[i]); };

    const unsigned head_bytes = (unsigned)Lq * 128u;
    const __amdgpu_buffer_rsrc_t rs_q = head_rsrc(p.q, h, head_bytes);
    const __amdgpu_buffer_rsrc_t rs_do = head_rsrc(p.dout, h, head_bytes);
    TileOffsets off;
    off.init(lane);
    const int tpfq = p.ql.P / TILE;

    // lse (base 2, +inf where P must be 0) and D of the 64 rows of a query tile, one value
    // per thread of the first 64 (lse) and last 64 (D) lanes
    auto fetch_rows = [&](int tq, float& val) {
        const int r = tid & 63;
        const int row = tq * TILE + r;
        const bool ok = (tq % tpfq) * TILE + r < p.ql.N;
        if (tid < 64) {
            const float l = ok ? p.lse[(size_t)h * Lq + row] : INFINITY;
            val = (ok && l > -INFINITY) ? l * LOG2E_F : INFINITY;
        } else {
            val = ok ? p.delta[(size_t)h * Lq + row] : 0.f;
        }
    };
    auto stage = [&](int tq, int b) {
        Block qb;
        qb.kind = 0;
        qb.t = tq;
        qb.mask = range_mask(0, valid_rows(p.ql, tq));
        stage_block(rs_q, p.ql, qb, (lds_u8*)s_q[b], w, lane);
        stage_block(rs_do, p.ql, qb, (lds_u8*)s_do[b], w, lane);
    };

    f32x16 dk0 = {}, dk1 = {}, dv0 = {}, dv1 = {};
    float rowval = 0.f;
    if (nq > 0) {
        const int t0 = qtile(0);
        stage(t0, 0);
        fetch_rows(t0, rowval);
        __builtin_amdgcn_s_waitcnt(0x0070);
        (tid < 64 ? s_lse[0] : s_d[0])[tid & 63] = rowval;
    }
    __syncthreads();
    for (int i = 0; i < nq; ++i) {
        const int b = i & 1;
        if (i + 1 < nq) {
            const int tn = qtile(i + 1);
            stage(tn, b ^ 1);
            fetch_rows(tn, rowval);
        }
        const unsigned char* qt = s_q[b];
        const unsigned char* dt = s_do[b];
        if (wk) {
            // S = Q K^T and dP = dO V^T, lane = key column, rows = queries
            f32x16 s0 = {}, s1 = {}, p0 = {}, p1 = {};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                bf16x8 a0, a1, o0, o1;
                read_rows(qt, off, st, a0, a1);
                read_rows(dt, off, st, o0, o1);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, kop[st], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, kop[st], s1, 0, 0, 0);
                p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o0, vop[st], p0, 0, 0, 0);
                p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o1, vop[st], p1, 0, 0, 0);
            }
            // P and dS per query row (8 (r/4) + 4 g + r % 4, +32)
            f32x16 pp0, pp1, d0, d1;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int q4 = 8 * a + 4 * g;
                const float4 la = *reinterpret_cast<const float4*>(&s_lse[b][q4]);
                const float4 lb = *reinterpret_cast<const float4*>(&s_lse[b][q4 + 32]);
                const float4 da = *reinterpret_cast<const float4*>(&s_d[b][q4]);
                const float4 db = *reinterpret_cast<const float4*>(&s_d[b][q4 + 32]);
                const float lav[4] = {la.x, la.y, la.z, la.w}, lbv[4] = {lb.x, lb.y, lb.z, lb.w};
                const float dav[4] = {da.x, da.y, da.z, da.w}, dbv[4] = {db.x, db.y, db.z, db.w};
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int r = 4 * a + i4;
                    pp0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], p.scale_l2, -lav[i4]));
                    pp1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], p.scale_l2, -lbv[i4]));
                    d0[r] = pp0[r] * (p0[r] - dav[i4]);
                    d1[r] = pp1[r] * (p1[r] - dbv[i4]);
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS (k = queries)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 a0, a1, c0, c1;
                read_tr(dt, off, ks, a0, a1);
                read_tr(qt, off, ks, c0, c1);
                const bf16x8 bp = acc_to_b(pp0, pp1, ks, [](float x, int, int) { return x; });
                const bf16x8 bd = acc_to_b(d0, d1, ks, [](float x, int, int) { return x; });
                dv0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bp, dv0, 0, 0, 0);
                dv1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bp, dv1, 0, 0, 0);
                dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c0, bd, dk0, 0, 0, 0);
                dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c1, bd, dk1, 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0070);
        if (i + 1 < nq) (tid < 64 ? s_lse[b ^ 1] : s_d[b ^ 1])[tid & 63] = rowval;
        __syncthreads();
    }
    // write this lane's key row: member rows of a frame tile (pad rows get zeros; special
    // rows inside the tile belong to the special pseudo-tiles), every special row of a
    // pseudo-tile
    bool write = kvalid;
    if (kb.kind == 0 && !kvalid) {
        const int j = krow % p.kl.P;
        write = j >= p.kl.N;                                     // pad: zeros
    }
    if (!write) return;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const f32x16& ak = cb ? dk1 : dk0;
        const f32x16& av = cb ? dv1 : dv0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c0 = 32 * cb + 8 * j + 4 * g;
            const float sk = kvalid ? p.scale : 0.f, sv = kvalid ? 1.f : 0.f;
            *reinterpret_cast<float4*>(p.dk + kbase + c0) =
                make_float4(ak[4 * j] * sk, ak[4 * j + 1] * sk, ak[4 * j + 2] * sk, ak[4 * j + 3] * sk);
            *reinterpret_cast<float4*>(p.dv + kbase + c0) =
                make_float4(av[4 * j] * sv, av[4 * j + 1] * sv, av[4 * j + 2] * sv, av[4 * j + 3] * sv);
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
    d.scale = a.scale;
    d.scale_l2 = a.scale * LOG2E_F;
    d.dq = a.dq;
    d.dk = a.dk;
    d.dv = a.dv;
    d.delta = a.delta;
    hipLaunchKernelGGL(k_attn_bwd_dq, dim3((unsigned)(a.heads * d.Tq)), dim3(128), (size_t)a.kmax * 4, st, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_bwd_dkv, dim3((unsigned)(a.heads * (d.Ts + d.Tk))), dim3(128), 0, st, d);
    return hipGetLastError();
}

}  // namespace s3d
