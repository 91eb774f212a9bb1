// Tile-list description shared by the attention kernels: which 64-row key block the
// it-th step of a query tile's loop stages, and which of its rows are real keys.
#pragma once

#include "device.h"

namespace s3d {

struct AttnDev {
    const void* q;
    const void* k;
    const void* v;
    Lay ql, kl;
    int Tq, Tk, Ts, nlm;
    const int32_t* idx;
    const int32_t* cnt;
    int kmax;
    const void* kbar;   // landmark means [heads, Tk, 64], operand dtype
    const void* vbar;
    int frame;          // dense over the query's own frame only (frame attention)
    float lm_bias_l2;   // landmark bias in base-2 logit units
    float scale_l2;     // scale * log2(e)
    // subsample completion (own key of dropped positions; one mean pair), off when NULL
    const void* sga_kf;
    const void* sga_vf;
    const float* sga_km;
    const float* sga_vm;
    float sga_bias_l2;
    int sga_gw, sga_win;
    void* out;
    float* lse;
};

constexpr int KST = 72;    // bf16 K tile row stride (elements): 144 B, conflict-free b128 reads
constexpr int FST = 68;    // fp32 K and V^T tile row stride (floats)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// V^T tile (bf16): 64 rows (head-dim c) x 32 words (key pairs); word w of row c lives at
// w ^ vt_swz(c).  The XOR keeps key pairs together and spreads both the transposing
// b32 writes and the b64 operand reads over all 32 banks.
__device__ __forceinline__ int vt_swz(int c) { return 2 * ((c & 3) | ((c >> 1) & 12)); }

enum { KIND_REG = 0, KIND_SPEC = 1, KIND_LM = 2 };

struct TileDesc {
    int kind;
    int t;             // key tile (REG), pseudo-tile (SPEC) or landmark block (LM)
    uint64_t mask;     // which of the 64 staged rows are real keys
};

// The same description with every field forced into scalar registers.  A TileDesc that
// has travelled through the kernel's rotating registers may sit in vector registers, where
// a branch on it becomes divergent and a buffer resource chosen by it needs a loop over
// lanes; the values are workgroup-uniform, so reading lane 0 is exact.
__device__ __forceinline__ TileDesc uniform(const TileDesc& d) {
    TileDesc u;
    u.kind = __builtin_amdgcn_readfirstlane(d.kind);
    u.t = __builtin_amdgcn_readfirstlane(d.t);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)d.mask);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(d.mask >> 32));
    u.mask = (uint64_t)lo | ((uint64_t)hi << 32);
    return u;
}

// A list entry with its member-row range precomputed: tile | lo << 16 | hi << 23, or -1
// for an entry outside [0, Tk) (skipped).  Needs Tk < 65536 (the library allows 12288).
__device__ __forceinline__ int32_t pack_tile_entry(const AttnDev& p, int32_t t) {
    if (t < 0 || t >= p.Tk) return -1;
    int lo, hi;
    member_range(p.kl, t, lo, hi);
    return t | (lo << 16) | (hi << 23);
}

// Longest selection list the bf16 kernel stages in LDS (next to its 24 KiB of tile
// buffers, within 64 KiB); longer lists run on the generic kernel.
constexpr int IDX_LDS_MAX = 8000;

// IDX_LDS: the list is read from its LDS copy (bf16 kernel) rather than from global memory.
// The selected tiles are visited starting at list position `rot` (and wrapping round).
// DENSE: the list is every key tile from t0 on (t0 = first tile of the frame in frame
// attention, 0 otherwise).
template <bool DENSE, bool LM, bool IDX_LDS>
__device__ __forceinline__ TileDesc describe(const AttnDev& p, int it, int c, const int32_t* myidx,
                                             const int32_t* s_idx, const uint32_t* s_lm, int rot = 0,
                                             int t0 = 0) {
    TileDesc d;
    if (DENSE) {
        d.kind = KIND_REG;
        d.t = t0 + it;
        d.mask = range_mask(0, valid_rows(p.kl, t0 + it));
        return d;
    }
    if (it < p.Ts) {
        d.kind = KIND_SPEC;
        d.t = it;
        d.mask = range_mask(0, min(TILE, p.kl.nsp * p.kl.S - it * TILE));
        return d;
    }
    it -= p.Ts;
    if (it < c) {
        const int pos = it + rot < c ? it + rot : it + rot - c;
        d.kind = KIND_REG;
        if (IDX_LDS) {
            // the LDS copy holds pack_tile_entry() words, decoded when the list was staged;
            // the entry is uniform across the workgroup, so it goes to a scalar register and
            // the whole description (and every branch on it) stays on the scalar unit
            const int word = __builtin_amdgcn_readfirstlane(s_idx[pos]);
            d.t = word < 0 ? 0 : (word & 0xFFFF);
            d.mask = word < 0 ? 0ull : range_mask((word >> 16) & 127, (word >> 23) & 127);
            return d;
        }
        const int t = __builtin_amdgcn_readfirstlane(myidx[pos]);
        d.t = t;
        if (t < 0 || t >= p.Tk) {
            d.t = 0;
            d.mask = 0;
        } else {
            int lo, hi;
            member_range(p.kl, t, lo, hi);
            d.mask = range_mask(lo, hi);
        }
        return d;
    }
    it -= c;
    d.kind = KIND_LM;
    d.t = it;
    if (LM) {
        const uint32_t w0 = __builtin_amdgcn_readfirstlane(s_lm[2 * it]);
        const uint32_t w1 = __builtin_amdgcn_readfirstlane(s_lm[2 * it + 1]);
        d.mask = (uint64_t)w0 | ((uint64_t)w1 << 32);
    } else {
        d.mask = 0;
    }
    return d;
}

// Global row (within the head) of staged row r of a REG or SPEC tile.
__device__ __forceinline__ int src_row(const AttnDev& p, const TileDesc& d, int r) {
    if (d.kind == KIND_SPEC) {
        const int e = d.t * TILE + r;
        return (e / p.kl.nsp) * p.kl.P + e % p.kl.nsp;
    }
    return d.t * TILE + r;
}


// Bitmap of the landmarks of one query tile, 2 * nlm words: bit t set <=> key tile t has
// member rows and is not among the c entries of `list` (the tile's selection).
__device__ __forceinline__ void init_landmark_bitmap(const Lay& kl, int Tk, int nlm, int c, const int32_t* list,
                                                     uint32_t* s_lm, int tid, int nthreads) {
    const int nw = 2 * nlm;
    for (int i = tid; i < nw; i += nthreads) {
        uint32_t bits = 0;
        for (int b = 0; b < 32; ++b) {
            const int t = i * 32 + b;
            if (t < Tk) {
                int lo, hi;
                member_range(kl, t, lo, hi);
                if (hi > lo) bits |= 1u << b;
            }
        }
        s_lm[i] = bits;
    }
    __syncthreads();
    for (int i = tid; i < c; i += nthreads) {
        const int t = list[i];
        if (t >= 0 && t < Tk) atomicAnd(&s_lm[t >> 5], ~(1u << (t & 31)));
    }
    __syncthreads();
}

// Subsample completion of one finished query row (AVGGT technical summary, section 2B.2):
// fold the row's own key (when the subsample dropped its position) and the mean pair into
// the running softmax state (m: base-2 reference, ltot: row sum relative to m, o0/o1: the
// O^T accumulators of this lane, dims 8*(r/4) + 4g + r%4 and 32 more).  Each lane of the
// pair (qc, g) and (qc, g^1) forms half of each 64-dim dot product.
template <bool F32IN>
__device__ __forceinline__ void sga_finish(const AttnDev& p, int h, int qrow, bool qvalid, int g,
                                           float& m, float& ltot, f32x16& o0, f32x16& o1) {
    if (!p.sga_kf && !p.sga_km) return;
    // Pass the row indices through an empty asm so nothing below can be computed ahead
    // of the tile loop: hoisted, it would hold registers across the whole loop.
    asm volatile("" : "+v"(qrow), "+v"(g));
    asm volatile("" : "+s"(h));
    const int Lq = p.ql.S * p.ql.P;
    const size_t rbase = ((size_t)h * Lq + qrow) * HD;
    auto load8 = [&](const void* base, size_t off, float (&x)[8]) {   // 8 values at base[off..]
        if (F32IN) {
            const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
            const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + 4);
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        } else {
            const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = __uint_as_float(w4[i] << 16);
                x[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
            }
        }
    };
    // own key applies to valid rows whose in-frame position is a dropped patch
    const int j = qrow % p.ql.P;
    const int pp = j - p.ql.nsp;
    const bool dropped = p.sga_kf && qvalid && pp >= 0 && j < p.ql.N &&
                         (((pp / p.sga_gw) % p.sga_win) != 0 || ((pp % p.sga_gw) % p.sga_win) != 0);
    float dd = 0.f, dm = 0.f;
    if (qvalid && (dropped || p.sga_km)) {
#pragma unroll
        for (int c = 0; c < 32; c += 8) {
            float qv[8], kv[8];
            load8(p.q, rbase + 32 * g + c, qv);
            if (dropped) {
                load8(p.sga_kf, rbase + 32 * g + c, kv);
#pragma unroll
                for (int i = 0; i < 8; ++i) dd = fmaf(qv[i], kv[i], dd);
            }
            if (p.sga_km) {
                const float* km = p.sga_km + (size_t)h * HD + 32 * g + c;
#pragma unroll
                for (int i = 0; i < 8; ++i) dm = fmaf(qv[i], km[i], dm);
            }
        }
    }
    dd += __shfl_xor(dd, 32);
    dm += __shfl_xor(dm, 32);
    const float xd = dropped ? dd * p.scale_l2 : -INFINITY;
    const float xm = (p.sga_km && qvalid) ? fmaf(dm, p.scale_l2, p.sga_bias_l2) : -INFINITY;
    const float mnew = fmaxf(m, fmaxf(xd, xm));
    if (mnew == -INFINITY) return;                         // nothing at all to attend
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
    const float pd = __builtin_amdgcn_exp2f(xd - mnew);    // 0 when the term is absent
    const float pm = __builtin_amdgcn_exp2f(xm - mnew);
    ltot = ltot * alpha + pd + pm;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        f32x16& oc = cb ? o1 : o0;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int c0 = 32 * cb + 8 * a + 4 * g;        // dims c0 .. c0+3 of this lane
            float vd[4] = {0.f, 0.f, 0.f, 0.f}, vm[4] = {0.f, 0.f, 0.f, 0.f};
            if (dropped) {
                if (F32IN) {
                    const float4 t = *reinterpret_cast<const float4*>(static_cast<const float*>(p.sga_vf) + rbase + c0);
                    vd[0] = t.x; vd[1] = t.y; vd[2] = t.z; vd[3] = t.w;
                } else {
                    const uint2 t = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.sga_vf) + rbase + c0);
                    vd[0] = __uint_as_float(t.x << 16); vd[1] = __uint_as_float(t.x & 0xffff0000u);
                    vd[2] = __uint_as_float(t.y << 16); vd[3] = __uint_as_float(t.y & 0xffff0000u);
                }
            }
            if (p.sga_km) {
                const float4 t = *reinterpret_cast<const float4*>(p.sga_vm + (size_t)h * HD + c0);
                vm[0] = t.x; vm[1] = t.y; vm[2] = t.z; vm[3] = t.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) oc[4 * a + i] = oc[4 * a + i] * alpha + pd * vd[i] + pm * vm[i];
        }
    }
    m = mnew;
}

hipError_t launch_attn_bf16(const AttnDev& d, int heads, bool dense, bool lm, bool f32out,
                            hipStream_t st);

}  // namespace s3d
