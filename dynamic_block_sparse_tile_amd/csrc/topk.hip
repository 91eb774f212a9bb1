// Per-row top-k tile selection united with the anchor frame (SAF3R abstract: keep
// only the most promising interactions for this input; Zebra3D abstract: tile-sparse
// attention).  One workgroup per (head, query tile) row of the score matrix.
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

// The same selection with one wave per score row (rows of at most 256 G tiles): the keys stay
// in registers, lane l holding the four consecutive tiles 256 g + 4 l .. + 3 of each group g
// (one 16-byte load per group), and every count is a ballot and a scalar popcount, so a row
// needs no histogram and no barrier.  The k-th largest key T is bracketed by bisection,
// keeping count(key >= lo) >= k > count(key > hi).  Once at most 256 keys lie inside the
// bracket they are compacted into LDS, four per lane, and the bisection continues on them
// alone (count(key >= t) = count(key > hi at that moment) + candidates >= t); once at most
// 64 remain they are gathered one per lane and ordered by a bitonic network across the
// lanes, which yields T directly.  Selection and compaction then run over the groups in
// tile order, positions from ballots and lane prefix counts (v_mbcnt): keys above T, the
// lowest-index ties, and the anchor tiles.  When exactly k keys are >= T (the bracket
// counts tell) there is no tie to rank and every key >= T is taken.
constexpr int TKW_WAVES = 4;            // rows per workgroup
constexpr int TKW_CAND = 256;           // bracket size at which the candidates move to LDS
// FULL: the row fills every slot (Tk = 256 G), so no slot needs a range check.  Rows start
// 16-byte aligned (Tk a multiple of 4 and an aligned matrix; the launcher checks).
template <int G, bool FULL>
__global__ __launch_bounds__(64 * TKW_WAVES) void k_select_topk_wave(const float* __restrict__ scores, int Tk,
                                                                     int Tq, int rows, KBudget kb, int tpf,
                                                                     int anchor, int32_t* __restrict__ idx,
                                                                     int32_t* __restrict__ cnt, int kmax) {
    // TKW_CAND candidate slots, then one dump slot per lane for lanes that have nothing to write
    __shared__ uint32_t s_cand[TKW_WAVES][TKW_CAND + 64];
    // the row is wave-uniform: in a scalar register, its buffer resource needs no lane loop
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = blockIdx.x * TKW_WAVES + wave;
    if (row >= rows) return;                        // whole wave leaves together
    const int k = kb.k[row / Tq];
    // the row through a buffer resource: slots past Tk read zeros (and are masked below)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(scores) + (size_t)row * Tk, 0, Tk * 4, tl::BUF_RSRC_WORD3);
    // the raw scores: float order equals key order for every non-NaN value (-0 == +0 as
    // the keys fold them, -inf lowest); padding slots hold NaN, which no comparison takes
    float x[G][4];
    {
        typedef float f32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int g = 0; g < G; ++g) {               // all loads in flight at once
            const f32x4v v = __builtin_bit_cast(f32x4v, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, 1024 * g, 0));
            x[g][0] = v[0];
            x[g][1] = v[1];
            x[g][2] = v[2];
            x[g][3] = v[3];
        }
    }
    if (!FULL) {
        const int lim = Tk - 4 * lane;              // slot (g, j) holds a tile iff 256 g + j < lim
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (256 * g + j >= lim) x[g][j] = __builtin_nanf("");
    }
    // count(key >= t) for a key t (its float: the keys' order on non-NaN values)
    auto count_ge = [&](uint32_t t) {
        const float tf = key_float(t);
        int c = 0;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) c += __popcll(__ballot(x[g][j] >= tf));
        return c;
    };
    // b + the number of lanes below this one whose bit in m is set
    auto below_from = [&](uint64_t m, int b) {
        return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)b));
    };
    auto lanes_below = [&](uint64_t m) { return below_from(m, 0); };
    // mode: 0 = nothing from top-k, 1 = every tile, 2 = threshold T with ties
    const int mode = k <= 0 ? 0 : (k >= Tk ? 1 : 2);
    uint32_t T = 0;
    int greater = 0;
    bool take_ge = false;                           // exactly k keys are >= T: no tie to break
    if (mode == 2) {
        float mn = INFINITY, mx = -INFINITY;        // NaN padding is ignored by min / max
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mn = fminf(mn, x[g][j]);
                mx = fmaxf(mx, x[g][j]);
            }
        // readfirstlane: the reductions end in lane shuffles, and a bracket the compiler
        // sees as per-lane would put the whole bisection under exec masks
        uint32_t lo = __builtin_amdgcn_readfirstlane(wave_min(order_key(mn)));
        uint32_t hi = __builtin_amdgcn_readfirstlane(wave_max(order_key(mx)));
        int c_lo = Tk, c_hi = 0;                    // count(key >= lo), count(key > hi)
        // candidates in LDS: cand[j] = candidate 4 lane + j (valid when below ncand);
        // c_base = count(key > bracket top) when they were taken
        int ncand = -1, c_base = 0;
        float cand[4] = {0.f, 0.f, 0.f, 0.f};
        float* s_c = reinterpret_cast<float*>(s_cand[wave]);
        // The probe halves the bracket in value (the midpoint of the two floats) while that
        // keeps shrinking the candidate count by at least a quarter, else in key order: on
        // score rows the value midpoint needs about half the passes of key bisection, and
        // the alternation bounds rows whose values span many binades.
        bool by_key = false;
        for (;;) {
            // every loop-carried value is wave-uniform; saying so keeps the loop's branches
            // scalar (the compiler cannot prove it through the LDS and lane-shuffle steps)
            lo = __builtin_amdgcn_readfirstlane(lo);
            hi = __builtin_amdgcn_readfirstlane(hi);
            c_lo = __builtin_amdgcn_readfirstlane(c_lo);
            c_hi = __builtin_amdgcn_readfirstlane(c_hi);
            ncand = __builtin_amdgcn_readfirstlane(ncand);
            c_base = __builtin_amdgcn_readfirstlane(c_base);
            if (lo == hi) break;
            const int inside = c_lo - c_hi;
            if (inside <= 64 || (ncand < 0 && inside <= TKW_CAND)) {
                // compact the values inside [lo, hi] into LDS (at most 256 of them); the upper
                // bound as "below key hi + 1" (hi stays below the key of NaN, so no wrap), since
                // key_float maps the unused key just below +0 to -0.  The same comparisons gave
                // c_hi = count(key > hi) exactly and c_lo >= count(key >= lo), so at most
                // inside <= TKW_CAND values pass and every write index stays inside s_c.
                const float flo = key_float(lo), fup = key_float(hi + 1);
                int base = 0;
                if (ncand < 0) {
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            // one ballot per comparison, combined on the scalar unit; every
                            // lane writes (outside the bracket to its dump slot), so the
                            // store needs no exec mask
                            const uint64_t m = __ballot(x[g][j] >= flo) & ~__ballot(x[g][j] >= fup);
                            s_c[__builtin_amdgcn_inverse_ballot_w64(m) ? below_from(m, base) : TKW_CAND + lane] = x[g][j];
                            base += __popcll(m);
                        }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool in = 4 * lane + j < ncand && cand[j] >= flo && !(cand[j] >= fup);
                        const uint64_t m = __ballot(in);
                        if (in) s_c[below_from(m, base)] = cand[j];
                        base += __popcll(m);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (inside > 64) {
                    // continue the bisection on the candidates alone
#pragma unroll
                    for (int j = 0; j < 4; ++j) cand[j] = 4 * lane + j < base ? s_c[4 * lane + j] : 0.f;
                    ncand = base;
                    c_base = c_hi;
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();         // read before a later gather overwrites
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    continue;
                }
                // at most 64 left: rank their keys across the lanes (pad lanes rank lowest)
                uint32_t v = lane < base ? order_key(s_c[lane]) : 0u;
#pragma unroll
                for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
                    for (int stride = size >> 1; stride > 0; stride >>= 1) {
                        const uint32_t o = (uint32_t)__shfl_xor((int)v, stride);
                        const bool desc = (lane & size) == 0, lower = (lane & stride) == 0;
                        v = (lower == desc) ? max(v, o) : min(v, o);
                    }
                }
                // rank k - c_hi among the candidates (one lane's key, the same in every lane)
                lo = __builtin_amdgcn_readfirstlane((uint32_t)__shfl((int)v, k - c_hi - 1));
                hi = lo;
                take_ge = c_hi + __popcll(__ballot(lane < base && v >= lo)) == k;
                break;
            }
            uint32_t mid = lo + (uint32_t)(((uint64_t)hi - lo + 1) >> 1);
            if (!by_key) {
                const float fl = key_float(lo), fh = key_float(hi);
                if (__builtin_isfinite(fl) && __builtin_isfinite(fh))
                    mid = min(max(order_key(0.5f * fl + 0.5f * fh), lo + 1), hi);
            }
            const int before = inside;
            int c;
            if (ncand < 0) {
                c = count_ge(mid);
            } else {
                const float tf = key_float(mid);
                c = c_base;
#pragma unroll
                for (int j = 0; j < 4; ++j) c += __popcll(__ballot(4 * lane + j < ncand && cand[j] >= tf));
            }
            if (c >= k) {
                lo = mid;
                c_lo = c;
            } else {
                hi = mid - 1;
                c_hi = c;
            }
            by_key = !by_key && 4 * (c_lo - c_hi) > 3 * before;
            if (lo == hi) take_ge = c_lo == k;      // converged: c_lo = count(key >= T)
        }
        T = lo;
        if (!take_ge) {
            const float tf = key_float(T);
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int j = 0; j < 4; ++j) greater += __popcll(__ballot(x[g][j] > tf));
        }
    }
    const float Tf = key_float(T);
    const int a0 = anchor >= 0 ? anchor * tpf : 0, a1 = anchor >= 0 ? min(a0 + tpf, Tk) : 0;
    int32_t* out = idx + (size_t)row * kmax;
    int base = 0;
    if (mode == 2 && take_ge) {
        // No tie to rank: the row takes every key >= T (exactly k of them) and the anchor
        // tiles.  The selection stays in 64-bit lane masks (scalar registers), turned back
        // into lane predicates where a store needs them; a lane's first slot of a group goes
        // after every selected slot of the lower lanes.  Stores go through a buffer
        // resource of min(kmax, Tk) entries, which drops anything past kmax.
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(out, 0, min(kmax, Tk) * 4,
                                                                            tl::BUF_RSRC_WORD3);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t0 = 256 * g + 4 * lane;
            uint64_t m[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = __ballot(x[g][j] >= Tf);
            if (a0 < 256 * g + 256 && a1 > 256 * g) {   // the group meets the anchor frame
#pragma unroll
                for (int j = 0; j < 4; ++j) m[j] |= __ballot(t0 + j >= a0 && t0 + j < a1);
            }
            uint32_t off = 4u * (uint32_t)below_from(m[3], below_from(m[2], below_from(m[1], below_from(m[0], base))));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (__builtin_amdgcn_inverse_ballot_w64(m[j])) {
                    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(t0 + j), ro, (int)off, 0, 0);
                    off += 4u;
                }
            base += __popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) + __popcll(m[3]);
        }
        for (int q = base + lane; q < kmax; q += 64) out[q] = -1;
        if (lane == 0) cnt[row] = min(base, kmax);
        return;
    }
    int ties_before = 0;                            // keys == T in earlier groups
    const int need_eq = mode == 2 ? k - greater : 0;   // ties to take, lowest index first
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int t0 = 256 * g + 4 * lane;
        bool sel[4], eq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // padding holds NaN, which fails every comparison below; only "every tile" and
            // the anchor range need the bound
            sel[j] = t0 + j >= a0 && t0 + j < a1;
            eq[j] = false;
            if (mode == 1) sel[j] = FULL || t0 + j < Tk;
            else if (mode == 2 && take_ge) sel[j] = sel[j] || x[g][j] >= Tf;
            else if (mode == 2) {
                sel[j] = sel[j] || x[g][j] > Tf;
                eq[j] = x[g][j] == Tf;
            }
        }
        if (mode == 2 && !take_ge) {
            // tie ranks in tile order: earlier groups, lower lanes, then this lane's lower j
            int run = ties_before, tot = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint64_t em = __ballot(eq[j]);
                run += lanes_below(em);
                tot += __popcll(em);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (eq[j]) {
                    sel[j] = sel[j] || run < need_eq;
                    ++run;
                }
            ties_before += tot;
        }
        int pos = base, tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint64_t sm = __ballot(sel[j]);
            pos += lanes_below(sm);
            tot += __popcll(sm);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (sel[j]) {
                if (pos < kmax) out[pos] = t0 + j;
                ++pos;
            }
        base += tot;
    }
    for (int q = base + lane; q < kmax; q += 64) out[q] = -1;
    if (lane == 0) cnt[row] = min(base, kmax);
}

template <int G>
static void launch_wave(bool full, dim3 grid, dim3 block, hipStream_t st, const float* scores, int tk, int tq,
                        int rows, const KBudget& kb, int tpf, int anchor, int32_t* ix, int32_t* cn, int kmax) {
    if (full)
        hipLaunchKernelGGL((k_select_topk_wave<G, true>), grid, block, 0, st, scores, tk, tq, rows, kb, tpf, anchor,
                           ix, cn, kmax);
    else
        hipLaunchKernelGGL((k_select_topk_wave<G, false>), grid, block, 0, st, scores, tk, tq, rows, kb, tpf,
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
        // one wave per row while the keys fit 96 registers per lane (G groups of 256 tiles, the
        // smallest that holds the row) and the rows allow 16-byte loads; otherwise a
        // workgroup per row
        const bool vec = tk % 4 == 0 && reinterpret_cast<uintptr_t>(sc) % 16 == 0;
        const int g = (tk + 255) / 256;
        int32_t* cn = cnt + r0;
#define S3D_WAVE(GG) launch_wave<GG>(tk == 256 * (GG), wgrid, wblock, st, sc, tk, tq, rows, kb, tpf, anchor, ix, cn, kmax)
        if (vec && g <= 2) S3D_WAVE(2);
        else if (vec && g <= 4) S3D_WAVE(4);
        else if (vec && g <= 8) S3D_WAVE(8);
        else if (vec && g <= 11) S3D_WAVE(11);
        else if (vec && g <= 16) S3D_WAVE(16);
        else if (vec && g <= 22) S3D_WAVE(22);
        else if (vec && g <= 24) S3D_WAVE(24);
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
