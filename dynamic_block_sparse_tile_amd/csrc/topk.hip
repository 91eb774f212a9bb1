// Per-row top-k tile selection united with the anchor frame (SAF3R abstract: keep
// only the most promising interactions for this input; Zebra3D abstract: tile-sparse
// attention), for every (head, query tile) row of the score matrix.  Rows of at most
// 6144 tiles take one wave each (k_select_topk_wave, below); longer rows one workgroup
// each (k_select_topk), described here.
//
// Scores become order-preserving unsigned keys (-0 folded into +0, so equal values
// give equal keys).  The k-th largest key T is found by a radix select whose digit
// range adapts to the live key interval: each round histograms the candidates of
// [lo, hi] into 2048 bins (LDS atomics), a suffix scan finds the bin holding the k-th
// largest, and the interval shrinks to that bin -- at most three rounds for 32-bit
// keys.  Then every key > T is selected, plus the (k - #greater) lowest-index keys
// equal to T, plus every anchor-frame tile, and the selection is compacted in
// ascending tile order.  Integer-only after the key transform: bit-exact and
// deterministic for a given score row.
#include <algorithm>

#include "device.h"
#include "launch.h"
#include "tile_lds.h"

namespace s3d {

constexpr int TK_THREADS = 256;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int NBINS = 2048;
constexpr int BIN_BITS = 11;

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0) u = 0;            // -0.0 and +0.0 are one value
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float whose order_key() is k (+0.0 for the folded zero).
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Block-wide exclusive prefix sum over thread order; also returns the total.
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_tmp[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) {
        const int t = s_tmp[w];
        before += (w < wave) ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

// Budgets of up to TK_HEAD_CHUNK heads, passed by value with the launch.
constexpr int TK_HEAD_CHUNK = 64;
struct KBudget {
    int32_t k[TK_HEAD_CHUNK];
};

__global__ __launch_bounds__(TK_THREADS) void k_select_topk(const float* __restrict__ scores, int Tk,
                                                            int Tq, KBudget kb, int tpf, int anchor,
                                                            int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ cnt, int kmax) {
    extern __shared__ uint32_t s_keys[];           // Tk keys
    __shared__ uint32_t s_hist[NBINS];
    __shared__ int s_tmp[TK_WAVES];
    __shared__ uint32_t s_mm[2 * TK_WAVES];
    __shared__ uint32_t s_bin;
    __shared__ int s_above;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t row = blockIdx.x;
    const int k = kb.k[blockIdx.x / Tq];           // this row's head budget
    const float* src = scores + row * (size_t)Tk;

    uint32_t kmin = 0xffffffffu, kmaxk = 0u;
    // eight loads in flight per thread before any is used
    constexpr int LB = 8;
    for (int i0 = 0; i0 < Tk; i0 += LB * TK_THREADS) {
        float f[LB];
#pragma unroll
        for (int u = 0; u < LB; ++u) f[u] = src[min(i0 + u * TK_THREADS + tid, Tk - 1)];
#pragma unroll
        for (int u = 0; u < LB; ++u) {
            const int i = i0 + u * TK_THREADS + tid;
            if (i < Tk) {
                const uint32_t key = order_key(f[u]);
                s_keys[i] = key;
                kmin = min(kmin, key);
                kmaxk = max(kmaxk, key);
            }
        }
    }
    kmin = wave_min(kmin);
    kmaxk = wave_max(kmaxk);
    if (lane == 0) {
        s_mm[wave] = kmin;
        s_mm[TK_WAVES + wave] = kmaxk;
    }
    __syncthreads();
    uint32_t lo = s_mm[0], hi = s_mm[TK_WAVES];
#pragma unroll
    for (int w = 1; w < TK_WAVES; ++w) {
        lo = min(lo, s_mm[w]);
        hi = max(hi, s_mm[TK_WAVES + w]);
    }

    // mode: 0 = nothing from top-k, 1 = everything, 2 = threshold (thr, need_eq)
    int mode = 2;
    if (k <= 0) mode = 0;
    else if (k >= Tk) mode = 1;
    int above = 0;
    if (mode == 2) {
        while (lo != hi) {
            const uint32_t span = hi - lo;
            const int bits = 32 - __clz(span);
            const int shift = bits > BIN_BITS ? bits - BIN_BITS : 0;
            for (int b = tid; b < NBINS; b += TK_THREADS) s_hist[b] = 0;
            __syncthreads();
            for (int i = tid; i < Tk; i += TK_THREADS) {
                const uint32_t key = s_keys[i];
                if (key >= lo && key <= hi) atomicAdd(&s_hist[(key - lo) >> shift], 1u);
            }
            __syncthreads();
            // thread t owns bins [8t, 8t+8); count from the top: scan over reversed threads
            constexpr int PER = NBINS / TK_THREADS;
            const int myb = (TK_THREADS - 1 - tid) * PER;   // reversed: thread 0 owns the top bins
            int local = 0;
#pragma unroll
            for (int j = 0; j < PER; ++j) local += (int)s_hist[myb + j];
            int total;
            const int before = block_excl_scan(local, s_tmp, total);
            const int run0 = above + before;
            if (run0 < k && k <= run0 + local) {
                int run = run0;
                for (int j = PER - 1; j >= 0; --j) {
                    const int c = (int)s_hist[myb + j];
                    if (run + c >= k) {
                        s_bin = (uint32_t)(myb + j);
                        s_above = run;
                        break;
                    }
                    run += c;
                }
            }
            __syncthreads();
            const uint32_t b = s_bin;
            above = s_above;
            const uint64_t nlo = (uint64_t)lo + ((uint64_t)b << shift);
            const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
            lo = (uint32_t)nlo;
            hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
            __syncthreads();
        }
    }
    const uint32_t thr = lo;
    const int need_eq = k - above;                   // how many keys equal to thr to take

    // contiguous chunk of tile indices per thread, so selection order = index order
    const int E = (Tk + TK_THREADS - 1) / TK_THREADS;
    const int i0 = min(tid * E, Tk), i1 = min(i0 + E, Tk);
    int eq_local = 0;
    if (mode == 2)
        for (int i = i0; i < i1; ++i) eq_local += (s_keys[i] == thr);
    int eq_total;
    int eq_rank = block_excl_scan(eq_local, s_tmp, eq_total);
    const int a0 = anchor >= 0 ? anchor * tpf : 0, a1 = anchor >= 0 ? a0 + tpf : 0;
    int sel_local = 0;
    {
        int r = eq_rank;
        for (int i = i0; i < i1; ++i) {
            const uint32_t key = s_keys[i];
            bool s = (i >= a0 && i < a1);
            if (mode == 1) s = true;
            else if (mode == 2) {
                if (key > thr) s = true;
                else if (key == thr) {
                    s = s || (r < need_eq);
                    ++r;
                }
            }
            sel_local += s;
        }
    }
    int total;
    int pos = block_excl_scan(sel_local, s_tmp, total);
    int32_t* out = idx + row * (size_t)kmax;
    {
        int r = eq_rank;
        for (int i = i0; i < i1; ++i) {
            const uint32_t key = s_keys[i];
            bool s = (i >= a0 && i < a1);
            if (mode == 1) s = true;
            else if (mode == 2) {
                if (key > thr) s = true;
                else if (key == thr) {
                    s = s || (r < need_eq);
                    ++r;
                }
            }
            if (s) {
                if (pos < kmax) out[pos] = i;
                ++pos;
            }
        }
    }
    for (int p = total + tid; p < kmax; p += TK_THREADS) out[p] = -1;
    if (tid == 0) cnt[row] = min(total, kmax);
}

// The same selection with one wave per score row (rows of at most 64 NS tiles).  Lane l holds
// the scores of tiles 64 s + l for slots s = 0 .. NS-1 in registers, so a ballot over one slot
// lists that slot's tiles in ascending order, and every count is a ballot and a scalar
// popcount: a row needs no histogram and no barrier.
//
// The k-th largest key T is bracketed by bisection, keeping count(key >= lo) >= k >
// count(key > hi).  The probe halves the bracket in value (the midpoint of its two floats)
// while that shrinks the count inside by at least a quarter, else in key order: on score rows
// the value midpoint needs about half the passes of key bisection, and the alternation bounds
// rows whose values span many binades.  Once at most TKW_LIST keys (with the anchor tiles) lie
// at or above lo, they move with their tile numbers into an LDS list in tile order, and
// everything after runs on the list alone: every key >= lo is in it, so its counts are the
// row's counts.  Once at most 64 keys lie inside the bracket they are gathered one per lane
// and ordered by a bitonic network, which yields T.  The output is then one pass over the
// list: keys above T, the lowest-index keys equal to T (k in all), and the anchor tiles, in
// tile order.  Rows whose budget is too large for the list bisect the full row to T and emit
// from the registers the same way.  Rows that take nothing from the top k (k <= 0) or every
// tile (k >= Tk) need no search.
//
// Scores are compared as floats: float order equals key order for every non-NaN value (-0 ==
// +0 as the keys fold them, -inf lowest).  Padding slots and NaN scores fail every comparison,
// so top-k never takes them (anchor tiles are taken whatever their score).
constexpr int TKW_WAVES = 4;            // rows per workgroup
constexpr int TKW_LIST = 512;           // list entries per row

// Wave-wide minimum and maximum through DPP (quad swaps, row mirrors, row broadcasts), read
// from the last lane: a value in a scalar register.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_min(uint32_t v) {
    return min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_min_uniform(uint32_t v) {
    v = dpp_min<0xB1, 0xF>(v);          // quad_perm [1,0,3,2]
    v = dpp_min<0x4E, 0xF>(v);          // quad_perm [2,3,0,1]
    v = dpp_min<0x141, 0xF>(v);         // row_half_mirror
    v = dpp_min<0x140, 0xF>(v);         // row_mirror: every lane holds its row's minimum
    v = dpp_min<0x142, 0xA>(v);         // row_bcast:15 into rows 1 and 3
    v = dpp_min<0x143, 0xC>(v);         // row_bcast:31 into rows 2 and 3
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_max_uniform(uint32_t v) {
    v = dpp_max<0xB1, 0xF>(v);
    v = dpp_max<0x4E, 0xF>(v);
    v = dpp_max<0x141, 0xF>(v);
    v = dpp_max<0x140, 0xF>(v);
    v = dpp_max<0x142, 0xA>(v);
    v = dpp_max<0x143, 0xC>(v);
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Bitonic sort of one key per lane into descending lane order.  Lane pairs (l, l ^ stride)
// exchange through DPP quad permutes (strides 1, 2), ds_swizzle (4, 8, 16) or a lane permute
// (32); the lane that keeps the larger key in each step is fixed by (size, stride).
constexpr uint64_t bitonic_max_lanes(int size, int stride) {
    uint64_t m = 0;
    for (int l = 0; l < 64; ++l)
        if (((l & stride) == 0) == ((l & size) == 0)) m |= 1ull << l;
    return m;
}
template <int STRIDE>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    if constexpr (STRIDE == 1)
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    else if constexpr (STRIDE == 2)
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    else if constexpr (STRIDE < 32)
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (STRIDE << 10));    // lane ^ STRIDE in 32
    else
        return (uint32_t)__shfl_xor((int)v, STRIDE);
}
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint32_t bitonic_merge(uint32_t v) {
    constexpr uint64_t take_max = bitonic_max_lanes(SIZE, STRIDE);
    const uint32_t o = lane_xor<STRIDE>(v);
    v = __builtin_amdgcn_inverse_ballot_w64(take_max) ? max(v, o) : min(v, o);
    if constexpr (STRIDE > 1) return bitonic_merge<SIZE, STRIDE / 2>(v);
    else return v;
}
template <int SIZE>
__device__ __forceinline__ uint32_t bitonic_sort_desc(uint32_t v) {
    v = bitonic_merge<SIZE, SIZE / 2>(v);
    if constexpr (SIZE < 64) return bitonic_sort_desc<SIZE * 2>(v);
    else return v;
}

// The bisection state of one row (every field wave-uniform).
struct Bracket {
    uint32_t lo, hi;        // key bracket of T
    int c_lo, c_hi;         // c_lo >= count(key >= lo) (exact once lo moved), c_hi = count(key > hi)
    bool by_key;            // the next probe halves in key order
    __device__ __forceinline__ void uniform() {
        lo = __builtin_amdgcn_readfirstlane(lo);
        hi = __builtin_amdgcn_readfirstlane(hi);
        c_lo = __builtin_amdgcn_readfirstlane(c_lo);
        c_hi = __builtin_amdgcn_readfirstlane(c_hi);
    }
    __device__ __forceinline__ uint32_t probe() const {
        uint32_t mid = lo + (uint32_t)(((uint64_t)hi - lo + 1) >> 1);
        if (!by_key) {
            const float fl = key_float(lo), fh = key_float(hi);
            if (__builtin_isfinite(fl) && __builtin_isfinite(fh))
                mid = min(max(order_key(0.5f * fl + 0.5f * fh), lo + 1), hi);
        }
        return mid;                                 // in [lo + 1, hi]: every step shrinks
    }
    // c = count(key >= mid)
    __device__ __forceinline__ void update(uint32_t mid, int c, int k) {
        const int before = c_lo - c_hi;
        if (c >= k) {
            lo = mid;
            c_lo = c;
        } else {
            hi = mid - 1;
            c_hi = c;
        }
        by_key = !by_key && 4 * (c_lo - c_hi) > 3 * before;
    }
};

// Emit the selection of one row from NV slots of (score, tile) per lane, in tile order across
// (slot, lane): keys > Tf, the first need_eq keys == Tf, and tiles in [a0, a0 + na).  Slots
// with valid false take nothing.  Returns the selected count (stores stop at kmax).
template <int NV, typename Get>
__device__ __forceinline__ int emit_selection(Get get, int nslots, float Tf, int need_eq, int a0, int na,
                                              int32_t* out, int kmax) {
    int base = 0, ties = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (i >= nslots) break;                     // uniform
        float v;
        int t;
        bool valid;
        get(i, v, t, valid);
        const bool eq = v == Tf;
        const uint64_t em = __ballot(eq);
        const bool sel = v > Tf || (eq && ties + lanes_below(em) < need_eq) ||
                         (valid && (uint32_t)(t - a0) < (uint32_t)na);
        ties += __popcll(em);
        const uint64_t sm = __ballot(sel);
        const int pos = base + lanes_below(sm);
        if (sel && pos < kmax) out[pos] = t;
        base += __popcll(sm);
    }
    return base;
}

template <int NS, bool FULL>
__global__ __launch_bounds__(64 * TKW_WAVES) void k_select_topk_wave(const float* __restrict__ scores, int Tk,
                                                                     int Tq, int rows, KBudget kb, int tpf,
                                                                     int anchor, int32_t* __restrict__ idx,
                                                                     int32_t* __restrict__ cnt, int kmax) {
    // per row: the list (values and tiles at a fixed distance, so one address serves both).
    // Once the values sit in registers, the value half takes the gathered bracket (64
    // entries, then one dump slot per lane).
    struct List {
        float v[TKW_LIST + 64];         // TKW_LIST entries, then one dump slot per lane
        int32_t t[TKW_LIST + 64];
    };
    __shared__ List s_list[TKW_WAVES];
    // the row is wave-uniform: in a scalar register, its buffer resource needs no lane loop
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = blockIdx.x * TKW_WAVES + wave;
    if (row >= rows) return;                        // whole wave leaves together
    const int k = kb.k[row / Tq];
    int32_t* out = idx + (size_t)row * kmax;
    const int a0 = anchor >= 0 ? anchor * tpf : 0, a1 = anchor >= 0 ? min(a0 + tpf, Tk) : 0, na = a1 - a0;
    auto finish = [&](int n) {
        for (int q = n + lane; q < kmax; q += 64) out[q] = -1;
        if (lane == 0) cnt[row] = min(n, kmax);
    };
    if (k <= 0 || k >= Tk) {
        // only the anchor frame, or every tile (the anchor frame among them)
        const int n = k <= 0 ? na : Tk, first = k <= 0 ? a0 : 0;
        for (int q = lane; q < min(n, kmax); q += 64) out[q] = first + q;
        finish(n);
        return;
    }
    // the row through a buffer resource: slots past Tk read zeros (and are masked below)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(scores) + (size_t)row * Tk, 0, Tk * 4, tl::BUF_RSRC_WORD3);
    float x[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)                    // all loads in flight at once
        x[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane + 256 * s, 0, 0));
    if (!FULL) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (64 * s + lane >= Tk) x[s] = __builtin_nanf("");
    }
    float mn = INFINITY, mx = -INFINITY;            // NaN is ignored by min / max
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        mn = fminf(mn, x[s]);
        mx = fmaxf(mx, x[s]);
    }
    Bracket b{wave_min_uniform(order_key(mn)), wave_max_uniform(order_key(mx)), Tk, 0, false};
    if (b.lo > b.hi) {                              // no score that is not NaN: the anchor frame only
        emit_selection<NS>([&](int s, float& v, int& t, bool& valid) { v = x[s]; t = 64 * s + lane; valid = t < Tk; },
                           NS, INFINITY, 0, a0, na, out, kmax);
        finish(na);
        return;
    }
    // bisect the full row while the keys at or above lo overflow the list
    for (;;) {
        b.uniform();
        if (b.lo == b.hi || b.c_lo <= TKW_LIST) break;
        const uint32_t mid = b.probe();
        const float tf = key_float(mid);
        int c = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s) c += __popcll(__ballot(x[s] >= tf));
        b.update(mid, c, k);
    }
    if (b.c_lo > TKW_LIST) {
        // converged on the full row with more keys >= T than the list holds
        const float Tf = key_float(b.lo);
        int greater = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s) greater += __popcll(__ballot(x[s] > Tf));
        const int n = emit_selection<NS>(
            [&](int s, float& v, int& t, bool& valid) { v = x[s]; t = 64 * s + lane; valid = t < Tk; },
            NS, Tf, k - greater, a0, na, out, kmax);
        finish(n);
        return;
    }
    // the list: every key >= lo, in tile order.  c_lo >= count(key >= lo), so at most c_lo <=
    // TKW_LIST entries are written and every write stays inside.  Every lane writes, the ones
    // without a key for the list to their dump slot, so the writes need no exec mask.
    float* s_v = s_list[wave].v;
    int32_t* s_t = s_list[wave].t;
    int n = 0;
    {
        const float flo = key_float(b.lo);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint64_t m = __ballot(x[s] >= flo);
            int p = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)n));
            asm volatile("" : "+v"(p));             // in every lane, so the choice below is a select
            p = __builtin_amdgcn_inverse_ballot_w64(m) ? p : TKW_LIST + lane;
            s_v[p] = x[s];
            s_t[p] = 64 * s + lane;
            n += __popcll(m);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int NL = TKW_LIST / 64;
    float lv[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) lv[i] = 64 * i + lane < n ? s_v[64 * i + lane] : __builtin_nanf("");
    // bisect on the list while more than 64 keys lie inside the bracket
    for (;;) {
        b.uniform();
        if (b.lo == b.hi || b.c_lo - b.c_hi <= 64) break;
        const uint32_t mid = b.probe();
        const float tf = key_float(mid);
        int c = 0;
#pragma unroll
        for (int i = 0; i < NL; ++i) c += __popcll(__ballot(lv[i] >= tf));
        b.update(mid, c, k);
    }
    if (b.lo != b.hi) {
        // gather the keys inside [lo, hi] (at most 64: c_hi is exact and c_lo bounds count(key
        // >= lo)), one per lane, and rank them: T has rank k - c_hi among them.  The upper bound
        // as "below key hi + 1" (hi stays below the key of NaN, so no wrap), since key_float
        // maps the unused key just below +0 to -0.
        const float glo = key_float(b.lo), gup = key_float(b.hi + 1);
        float* s_g = s_v;                           // the list values are in lv[] now
        int ng = 0;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const uint64_t m = __ballot(lv[i] >= glo) & ~__ballot(lv[i] >= gup);
            s_g[__builtin_amdgcn_inverse_ballot_w64(m) ? ng + lanes_below(m) : 64 + lane] = lv[i];
            ng += __popcll(m);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint32_t v = bitonic_sort_desc<2>(lane < ng ? order_key(s_g[lane]) : 0u);   // pads rank lowest
        b.lo = __builtin_amdgcn_readfirstlane((uint32_t)__shfl((int)v, k - b.c_hi - 1));
    }
    // Emit: S = the keys > T and the first k - count(key > T) keys == T, all in the list.  In
    // the sorted output the anchor frame A = [a0, a1) is one run starting after the members of
    // S below a0, and members of S after A move by the anchor tiles S does not hold.
    const float Tf = key_float(b.lo);
    int greater = 0;
#pragma unroll
    for (int i = 0; i < NL; ++i) greater += __popcll(__ballot(lv[i] > Tf));
    const int need_eq = k - greater;
    uint64_t sm[NL];
    int ties = 0, before_a = 0, in_a = 0;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const bool eq = lv[i] == Tf;
        const uint64_t em = __ballot(eq);
        const bool sel = lv[i] > Tf || (eq && ties + lanes_below(em) < need_eq);
        ties += __popcll(em);
        sm[i] = __ballot(sel);
        const int t = s_t[64 * i + lane];           // read past n: stale, and not selected
        before_a += __popcll(__ballot(sel && t < a0));
        in_a += __popcll(__ballot(sel && t >= a0 && t < a1));
    }
    const int shift = na - in_a;                    // anchor tiles S does not hold
    int base = 0;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int t = s_t[64 * i + lane];
        const int pos = base + lanes_below(sm[i]) + (t >= a1 ? shift : 0);
        if (__builtin_amdgcn_inverse_ballot_w64(sm[i]) && (uint32_t)(t - a0) >= (uint32_t)na && pos < kmax)
            out[pos] = t;
        base += __popcll(sm[i]);
    }
    for (int q = lane; q < na; q += 64)
        if (before_a + q < kmax) out[before_a + q] = a0 + q;
    finish(base + shift);
}

template <int NS>
static void launch_wave(bool full, dim3 grid, dim3 block, hipStream_t st, const float* scores, int tk, int tq,
                        int rows, const KBudget& kb, int tpf, int anchor, int32_t* ix, int32_t* cn, int kmax) {
    if (full)
        hipLaunchKernelGGL((k_select_topk_wave<NS, true>), grid, block, 0, st, scores, tk, tq, rows, kb, tpf, anchor,
                           ix, cn, kmax);
    else
        hipLaunchKernelGGL((k_select_topk_wave<NS, false>), grid, block, 0, st, scores, tk, tq, rows, kb, tpf,
                           anchor, ix, cn, kmax);
}

hipError_t launch_select_topk(const float* scores, int heads, int tq, int tk, const int32_t* k_heads,
                              int tpf, int anchor, int32_t* idx, int32_t* cnt, int kmax, hipStream_t st) {
    const size_t shm = (size_t)tk * sizeof(uint32_t);
    for (int h0 = 0; h0 < heads; h0 += TK_HEAD_CHUNK) {
        const int nh = std::min(TK_HEAD_CHUNK, heads - h0);
        KBudget kb{};
        for (int i = 0; i < nh; ++i) kb.k[i] = k_heads[h0 + i];
        const size_t r0 = (size_t)h0 * tq;
        const int rows = nh * tq;
        int32_t* ix = kmax > 0 ? idx + r0 * kmax : idx;
        const dim3 wgrid((unsigned)((rows + TKW_WAVES - 1) / TKW_WAVES)), wblock(64 * TKW_WAVES);
        const float* sc = scores + r0 * tk;
        // one wave per row while the scores fit 96 registers per lane (NS slots of 64 tiles, the
        // fewest of these that hold the row); otherwise a workgroup per row
        const int ns = (tk + 63) / 64;
        int32_t* cn = cnt + r0;
#define S3D_WAVE(N) launch_wave<N>(tk == 64 * (N), wgrid, wblock, st, sc, tk, tq, rows, kb, tpf, anchor, ix, cn, kmax)
        if (ns <= 8) S3D_WAVE(8);
        else if (ns <= 16) S3D_WAVE(16);
        else if (ns <= 32) S3D_WAVE(32);
        else if (ns <= 44) S3D_WAVE(44);
        else if (ns <= 64) S3D_WAVE(64);
        else if (ns <= 88) S3D_WAVE(88);
        else if (ns <= 96) S3D_WAVE(96);
        else
            hipLaunchKernelGGL(k_select_topk, dim3((unsigned)rows), dim3(TK_THREADS), shm, st,
                               sc, tk, tq, kb, tpf, anchor, ix, cn, kmax);
#undef S3D_WAVE
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace s3d
