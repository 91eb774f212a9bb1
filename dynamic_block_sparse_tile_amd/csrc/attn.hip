// Exact softmax attention of each 64-row query tile over a list of 64-row key tiles:
// the sparse layer (specials + selected tiles + optional landmark summaries; Zebra3D
// abstract: tile-sparse attention with landmark summaries of unselected context) and
// the dense reference (every key tile; SAF3R abstract: the quadratic global attention
// the sparse layer replaces).
//
// Workgroup = 2 waves = one (head, query tile); wave w owns queries [32w, 32w+32).
// Per key tile the workgroup stages K (row-major) and V^T (transposed, XOR-swizzled)
// in LDS, then each wave computes on the matrix cores
//     S^T[key, q] = K Q^T          (A = K tile rows, B = this wave's Q, held in VGPRs)
//     O^T[c, q]  += V^T P^T        (A = V^T from LDS, B = P^T straight from S^T's
//                                   accumulator layout -- no cross-lane shuffle)
// with an online softmax in fp32 (base-2 exponent, scale*log2(e) folded into one FMA).
// In the 32x32 accumulator layout lane l holds column l%32 (one query) and rows
// 8*(r/4) + 4*(l/32) + r%4, so every statistic a lane keeps belongs to one query and the
// only cross-lane step is combining the two 32-lane halves (keys split by l/32).
// K and V of the next tile are fetched into registers while the current tile computes.
#include "attn_common.h"
#include "device.h"
#include "launch.h"

namespace s3d {

template <bool F32IN, bool F32OUT, bool DENSE, bool LM>
__global__ __launch_bounds__(128, 2) void k_attn(AttnDev p) {
    constexpr int KBYTES = F32IN ? TILE * FST * 4 : TILE * KST * 2;
    constexpr int VBYTES = F32IN ? TILE * FST * 4 : TILE * TILE * 2;
    __shared__ __align__(16) unsigned char s_k[KBYTES];
    __shared__ __align__(16) unsigned char s_v[VBYTES];
    extern __shared__ uint32_t s_lm[];   // landmark bitmap: unselected tiles with members

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 31, g = lane >> 5;
    const int tpfq = p.ql.P / TILE;
    int h, tq;
    attn_work_item(blockIdx.x, gridDim.x, p.ql.S, tpfq, gridDim.x / p.Tq, h, tq, !p.frame);
    const int Lq = p.ql.S * p.ql.P, Lk = p.kl.S * p.kl.P;
    const int qrow = tq * TILE + w * 32 + qc;
    const bool qvalid = (tq % tpfq) * TILE + w * 32 + qc < p.ql.N;

    // ---- this lane's query operand (B of S^T = K Q^T), zero for invalid rows
    bf16x8 qop[4];
    float qf[32];
    {
        const size_t base = ((size_t)h * Lq + qrow) * HD;
        if (!F32IN) {
            const uint16_t* qp = static_cast<const uint16_t*>(p.q) + base;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint4 u = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * s + 8 * g)
                                 : make_uint4(0, 0, 0, 0);
                qop[s] = __builtin_bit_cast(bf16x8, u);
            }
        } else {
            // k-step s of the fp32 product uses head-dim 32*g + s
            const float* qp = static_cast<const float*>(p.q) + base + 32 * g;
#pragma unroll
            for (int s = 0; s < 32; s += 4) {
                float4 u = qvalid ? *reinterpret_cast<const float4*>(qp + s) : make_float4(0, 0, 0, 0);
                qf[s] = u.x; qf[s + 1] = u.y; qf[s + 2] = u.z; qf[s + 3] = u.w;
            }
        }
    }

    int c = 0, t0 = 0;
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
    if (LM) init_landmark_bitmap(p.kl, p.Tk, p.nlm, c, myidx, s_lm, tid, 128);

    // ---- staging assignment: thread -> rows {2rp, 2rp+1, 32+2rp, 33+2rp}, chunk c8
    //      (bf16: 16-byte chunks of 8 elements; fp32: two 16-byte chunks per c8)
    const int rp = tid >> 3, c8 = tid & 7;
    const uint16_t* kb16 = static_cast<const uint16_t*>(p.k) + (size_t)h * Lk * HD;
    const uint16_t* vb16 = static_cast<const uint16_t*>(p.v) + (size_t)h * Lk * HD;
    const float* kb32 = static_cast<const float*>(p.k) + (size_t)h * Lk * HD;
    const float* vb32 = static_cast<const float*>(p.v) + (size_t)h * Lk * HD;

    uint4 kr[4], vr[4];        // bf16 staging registers
    float4 kf[8], vf[8];       // fp32 staging registers
    TileDesc nxt;

    auto fetch = [&](int it) {
        nxt = describe<DENSE, LM, false>(p, it, c, myidx, nullptr, s_lm, 0, t0);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = (x >> 1) * 32 + 2 * rp + (x & 1);
            const bool ok = (nxt.mask >> r) & 1ull;
            if (nxt.kind == KIND_LM) {
                // landmark rows come from the tile means (operand dtype)
                const size_t o = ((size_t)h * p.Tk + nxt.t * TILE + r) * HD + c8 * 8;
                if (!F32IN) {
                    const uint16_t* km = static_cast<const uint16_t*>(p.kbar);
                    const uint16_t* vm = static_cast<const uint16_t*>(p.vbar);
                    kr[x] = ok ? *reinterpret_cast<const uint4*>(km + o) : make_uint4(0, 0, 0, 0);
                    vr[x] = ok ? *reinterpret_cast<const uint4*>(vm + o) : make_uint4(0, 0, 0, 0);
                } else {
                    const float* km = static_cast<const float*>(p.kbar);
                    const float* vm = static_cast<const float*>(p.vbar);
                    float4 a0 = make_float4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
                    if (ok) {
                        a0 = *reinterpret_cast<const float4*>(km + o);
                        a1 = *reinterpret_cast<const float4*>(km + o + 4);
                        b0 = *reinterpret_cast<const float4*>(vm + o);
                        b1 = *reinterpret_cast<const float4*>(vm + o + 4);
                    }
                    kf[2 * x] = a0; kf[2 * x + 1] = a1;
                    vf[2 * x] = b0; vf[2 * x + 1] = b1;
                }
            } else {
                const size_t o = (size_t)src_row(p, nxt, ok ? r : 0) * HD + c8 * 8;
                if (!F32IN) {
                    kr[x] = ok ? *reinterpret_cast<const uint4*>(kb16 + o) : make_uint4(0, 0, 0, 0);
                    vr[x] = ok ? *reinterpret_cast<const uint4*>(vb16 + o) : make_uint4(0, 0, 0, 0);
                } else {
                    const float4 z = make_float4(0, 0, 0, 0);
                    kf[2 * x] = ok ? *reinterpret_cast<const float4*>(kb32 + o) : z;
                    kf[2 * x + 1] = ok ? *reinterpret_cast<const float4*>(kb32 + o + 4) : z;
                    vf[2 * x] = ok ? *reinterpret_cast<const float4*>(vb32 + o) : z;
                    vf[2 * x + 1] = ok ? *reinterpret_cast<const float4*>(vb32 + o + 4) : z;
                }
            }
        }
    };

    auto stage = [&]() {
        if (!F32IN) {
            uint16_t* ks = reinterpret_cast<uint16_t*>(s_k);
            uint32_t* vt = reinterpret_cast<uint32_t*>(s_v);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = (x >> 1) * 32 + 2 * rp + (x & 1);
                *reinterpret_cast<uint4*>(ks + r * KST + c8 * 8) = kr[x];
            }
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                const uint4 a = vr[2 * hp], b = vr[2 * hp + 1];      // rows r0, r0+1
                const int wd = hp * 16 + rp;                          // key-pair word
                const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t lo16 = (e & 1) ? (aw[e >> 1] >> 16) : (aw[e >> 1] & 0xffffu);
                    const uint32_t hi16 = (e & 1) ? (bw[e >> 1] & 0xffff0000u) : (bw[e >> 1] << 16);
                    const int cc = c8 * 8 + e;
                    vt[cc * 32 + (wd ^ vt_swz(cc))] = lo16 | hi16;
                }
            }
        } else {
            float* ks = reinterpret_cast<float*>(s_k);
            float* vt = reinterpret_cast<float*>(s_v);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = (x >> 1) * 32 + 2 * rp + (x & 1);
                *reinterpret_cast<float4*>(ks + r * FST + c8 * 8) = kf[2 * x];
                *reinterpret_cast<float4*>(ks + r * FST + c8 * 8 + 4) = kf[2 * x + 1];
                const float e8[8] = {vf[2 * x].x, vf[2 * x].y, vf[2 * x].z, vf[2 * x].w,
                                     vf[2 * x + 1].x, vf[2 * x + 1].y, vf[2 * x + 1].z, vf[2 * x + 1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) vt[(c8 * 8 + e) * FST + r] = e8[e];
            }
        }
    };

    float m = -INFINITY, l = 0.f;   // running max (base-2 units) and partial row sum
    f32x16 o0 = {}, o1 = {};        // O^T accumulators, head-dim blocks [0,32) and [32,64)

    if (ntiles > 0) fetch(0);
    for (int it = 0; it < ntiles; ++it) {
        const TileDesc cur = nxt;
        __syncthreads();             // every wave is done reading the previous tile
        stage();
        __syncthreads();
        if (it + 1 < ntiles) fetch(it + 1);
        if (cur.mask == 0) continue;

        // ---- S^T = K Q^T for keys [32kb, 32kb+32)
        f32x16 s0 = {}, s1 = {};
        if (!F32IN) {
            const uint16_t* ks = reinterpret_cast<const uint16_t*>(s_k);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ks + qc * KST + 16 * st + 8 * g));
                const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ks + (32 + qc) * KST + 16 * st + 8 * g));
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qop[st], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qop[st], s1, 0, 0, 0);
            }
        } else {
            const float* ks = reinterpret_cast<const float*>(s_k);
#pragma unroll
            for (int s4 = 0; s4 < 8; ++s4) {
                const float4 a0 = *reinterpret_cast<const float4*>(ks + qc * FST + 32 * g + 4 * s4);
                const float4 a1 = *reinterpret_cast<const float4*>(ks + (32 + qc) * FST + 32 * g + 4 * s4);
                const float av0[4] = {a0.x, a0.y, a0.z, a0.w}, av1[4] = {a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av0[i], qf[4 * s4 + i], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av1[i], qf[4 * s4 + i], s1, 0, 0, 0);
                }
            }
        }

        // ---- mask rows that are not keys (pad, specials inside a tile, non-landmarks)
        if (cur.mask != ~0ull) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * g + (r & 3);
                if (!((cur.mask >> key) & 1ull)) s0[r] = -INFINITY;
                if (!((cur.mask >> (32 + key)) & 1ull)) s1[r] = -INFINITY;
            }
        }

        // ---- online softmax (base 2): logit2 = s * scale*log2(e) + bias
        const float bias = (cur.kind == KIND_LM) ? p.lm_bias_l2 : 0.f;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx == -INFINITY ? -INFINITY : fmaf(mx, p.scale_l2, bias);
        const float mnew = fmaxf(m, mt);
        const float muse = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m - muse);
        const float off = bias - muse;
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], p.scale_l2, off));
            s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], p.scale_l2, off));
            rs += s0[r] + s1[r];
        }
        l = l * alpha + rs;
        m = mnew;
        if (__ballot(alpha != 1.f)) {
            o0 *= alpha;
            o1 *= alpha;
        }

        // ---- O^T += V^T P^T
        if (!F32IN) {
            const uint32_t* vt = reinterpret_cast<const uint32_t*>(s_v);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const f32x16& sp = (ks < 2) ? s0 : s1;
                const int j0 = 2 * (ks & 1);
                const uint4 pu = make_uint4(pack_bf16x2(sp[4 * j0 + 0], sp[4 * j0 + 1]),
                                            pack_bf16x2(sp[4 * j0 + 2], sp[4 * j0 + 3]),
                                            pack_bf16x2(sp[4 * j0 + 4], sp[4 * j0 + 5]),
                                            pack_bf16x2(sp[4 * j0 + 6], sp[4 * j0 + 7]));
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pu);
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const int cc = 32 * cb + qc;
                    const int sw = vt_swz(cc);
                    const uint2 x0 = *reinterpret_cast<const uint2*>(vt + cc * 32 + ((8 * ks + 2 * g) ^ sw));
                    const uint2 x1 = *reinterpret_cast<const uint2*>(vt + cc * 32 + ((8 * ks + 4 + 2 * g) ^ sw));
                    const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
                    if (cb == 0) o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o0, 0, 0, 0);
                    else o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o1, 0, 0, 0);
                }
            }
        } else {
            const float* vt = reinterpret_cast<const float*>(s_v);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const f32x16& sp = kb ? s1 : s0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 a0 = *reinterpret_cast<const float4*>(vt + qc * FST + 32 * kb + 8 * j + 4 * g);
                    const float4 a1 = *reinterpret_cast<const float4*>(vt + (32 + qc) * FST + 32 * kb + 8 * j + 4 * g);
                    const float av0[4] = {a0.x, a0.y, a0.z, a0.w}, av1[4] = {a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        o0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av0[i], sp[4 * j + i], o0, 0, 0, 0);
                        o1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av1[i], sp[4 * j + i], o1, 0, 0, 0);
                    }
                }
            }
        }
    }

    // ---- epilogue: combine the two key halves' row sums, normalise, write
    float ltot = l + __shfl_xor(l, 32);
    sga_finish<F32IN>(p, h, qrow, qvalid, g, m, ltot, o0, o1);
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

template <bool F32IN, bool F32OUT>
static hipError_t launch_attn_t(const AttnDev& d, int heads, bool dense, bool lm, hipStream_t st) {
    const dim3 grid((unsigned)(heads * d.Tq)), block(128);
    const size_t shm = lm ? (size_t)(2 * d.nlm) * sizeof(uint32_t) : 0;
    if (dense) hipLaunchKernelGGL((k_attn<F32IN, F32OUT, true, false>), grid, block, 0, st, d);
    else if (lm) hipLaunchKernelGGL((k_attn<F32IN, F32OUT, false, true>), grid, block, shm, st, d);
    else hipLaunchKernelGGL((k_attn<F32IN, F32OUT, false, false>), grid, block, 0, st, d);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
    AttnDev d;
    d.q = a.q;
    d.k = a.k;
    d.v = a.v;
    d.ql = Lay{a.ql.S, a.ql.N, a.ql.P, a.ql.nsp};
    d.kl = Lay{a.kl.S, a.kl.N, a.kl.P, a.kl.nsp};
    d.Tq = a.ql.S * a.ql.P / TILE;
    d.Tk = a.kl.S * a.kl.P / TILE;
    d.Ts = a.dense ? 0 : (a.kl.nsp * a.kl.S + TILE - 1) / TILE;
    d.frame = a.frame ? 1 : 0;
    const bool lm = !a.dense && a.kbar != nullptr;
    d.nlm = lm ? (d.Tk + TILE - 1) / TILE : 0;
    d.idx = a.idx;
    d.cnt = a.cnt;
    d.kmax = a.kmax;
    d.kbar = a.kbar;
    d.vbar = a.vbar;
    d.lm_bias_l2 = a.landmark_bias * LOG2E;
    const sparse3d_sga* sg = a.sga;
    d.sga_kf = sg ? sg->k_full : nullptr;
    d.sga_vf = sg ? sg->v_full : nullptr;
    d.sga_km = sg ? sg->kmean : nullptr;
    d.sga_vm = sg ? sg->vmean : nullptr;
    d.sga_bias_l2 = (sg && sg->kmean) ? sg->mean_bias * LOG2E : 0.f;
    d.sga_gw = sg ? sg->grid_w : 1;
    d.sga_win = sg ? sg->window : 1;
    d.scale_l2 = a.scale * LOG2E;
    d.out = a.out;
    d.lse = a.lse;
    const bool f32in = a.dtype == SPARSE3D_F32, f32out = a.out_dtype == SPARSE3D_F32;
    if (!f32in && (a.dense || a.kmax <= IDX_LDS_MAX))
        return launch_attn_bf16(d, a.heads, a.dense, lm, f32out, st);
    // fp32 operands, or a bf16 selection list too long to stage in LDS
    if (f32in && f32out) return launch_attn_t<true, true>(d, a.heads, a.dense, lm, st);
    if (f32in) return launch_attn_t<true, false>(d, a.heads, a.dense, lm, st);
    if (f32out) return launch_attn_t<false, true>(d, a.heads, a.dense, lm, st);
    return launch_attn_t<false, false>(d, a.heads, a.dense, lm, st);
}

}  // namespace s3d
