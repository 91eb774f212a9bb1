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

// The same selection with one wave per score row (rows of at most 64 * E tiles): the keys
// stay in registers (tile i * 64 + lane in slot i) and every count is a ballot and a scalar
// popcount, so a row needs no LDS histogram and no barrier.  The k-th largest key T is
// bracketed by bisection, keeping count(key >= lo) >= k > count(key > hi); once at most 64
// keys remain inside the bracket they are gathered, one per lane, and ordered by a bitonic
// network across the lanes, which yields T directly.
// Selection and compaction then run over the slots in tile order with ballot prefix
// counts, exactly as in the workgroup kernel (keys above T, the lowest-index ties, the
// anchor frame); when exactly k keys are >= T (the bracket counts tell) there is no tie to
// rank and every key >= T is taken.
constexpr int TKW_WAVES = 4;            // rows per workgroup
// FULL: the row fills every slot (Tk = 64 E), so no slot needs a range check.
template <int E, bool FULL>
__global__ __launch_bounds__(64 * TKW_WAVES) void k_select_topk_wave(const float* __restrict__ scores, int Tk,
                                                                     int Tq, int rows, KBudget kb, int tpf,
                                                                     int anchor, int32_t* __restrict__ idx,
                                                                     int32_t* __restrict__ cnt, int kmax) {
    __shared__ uint32_t s_cand[TKW_WAVES][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * TKW_WAVES + wave;
    if (row >= rows) return;                        // whole wave leaves together
    const int k = kb.k[row / Tq];
    const float* src = scores + (size_t)row * Tk;
    uint32_t key[E];
    float f[E];
#pragma unroll
    for (int i = 0; i < E; ++i) f[i] = src[min(i * 64 + lane, Tk - 1)];   // all loads in flight at once
#pragma unroll
    for (int i = 0; i < E; ++i) key[i] = FULL || i * 64 + lane < Tk ? order_key(f[i]) : 0u;   // pad slots rank lowest
    auto count_ge = [&](uint32_t t) {
        int c = 0;
#pragma unroll
        for (int i = 0; i < E; ++i) c += __popcll(__ballot(key[i] >= t));
        return c;
    };
    // mode: 0 = nothing from top-k, 1 = every tile, 2 = threshold T with ties
    const int mode = k <= 0 ? 0 : (k >= Tk ? 1 : 2);
    uint32_t T = 0;
    int greater = 0;
    bool take_ge = false;                           // exactly k keys are >= T: no tie to break
    if (mode == 2) {
        uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            if (FULL || i * 64 + lane < Tk) {
                lo = min(lo, key[i]);
                hi = max(hi, key[i]);
            }
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        int c_lo = Tk, c_hi = 0;                    // count(key >= lo), count(key > hi)
        // The probe halves the bracket in value (the midpoint of the two floats) while that
        // keeps shrinking the candidate count by at least a quarter, else in key order: on
        // score rows the value midpoint needs about half the passes of key bisection, and
        // the alternation bounds rows whose values span many binades.
        bool by_key = false;
        while (lo != hi) {
            if (c_lo - c_hi <= 64) {
                // gather the keys inside [lo, hi] and rank them across the lanes
                int base = 0;
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    const bool in = (FULL || i * 64 + lane < Tk) && key[i] >= lo && key[i] <= hi;
                    const uint64_t m = __ballot(in);
                    const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    if (in) s_cand[wave][pos] = key[i];
                    base += __popcll(m);
                }
                __builtin_amdgcn_wave_barrier();
                uint32_t v = lane < base ? s_cand[wave][lane] : 0u;
#pragma unroll
                for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
                    for (int stride = size >> 1; stride > 0; stride >>= 1) {
                        const uint32_t o = (uint32_t)__shfl_xor((int)v, stride);
                        const bool desc = (lane & size) == 0, lower = (lane & stride) == 0;
                        v = (lower == desc) ? max(v, o) : min(v, o);
                    }
                }
                lo = (uint32_t)__shfl((int)v, k - c_hi - 1);   // rank k - c_hi among the candidates
                hi = lo;
                take_ge = c_hi + __popcll(__ballot(v >= lo)) == k;   // pad lanes hold 0 < lo
                break;
            }
            uint32_t mid = lo + (uint32_t)(((uint64_t)hi - lo + 1) >> 1);
            if (!by_key) {
                const float fl = key_float(lo), fh = key_float(hi);
                if (__builtin_isfinite(fl) && __builtin_isfinite(fh))
                    mid = min(max(order_key(0.5f * fl + 0.5f * fh), lo + 1), hi);
            }
            const int before = c_lo - c_hi;
            const int c = count_ge(mid);
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
#pragma unroll
            for (int i = 0; i < E; ++i) greater += __popcll(__ballot((FULL || i * 64 + lane < Tk) && key[i] > T));
        }
    }
    int ties_before = 0;                            // keys == T in earlier slots
    const int need_eq = mode == 2 ? k - greater : 0;   // ties to take, lowest index first
    const int a0 = anchor >= 0 ? anchor * tpf : 0, a1 = anchor >= 0 ? a0 + tpf : 0;
    int32_t* out = idx + (size_t)row * kmax;
    int base = 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int t = i * 64 + lane;
        const bool valid = FULL || t < Tk;
        bool sel = valid && t >= a0 && t < a1;
        if (mode == 1) sel = valid;
        else if (mode == 2 && take_ge) {
            sel = sel || (valid && key[i] >= T);
        } else if (mode == 2) {
            const uint64_t eqm = __ballot(valid && key[i] == T);
            const int eq_rank = ties_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(eqm >> 32),
                                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)eqm, 0u));
            ties_before += __popcll(eqm);
            if (valid && key[i] > T) sel = true;
            else if (valid && key[i] == T && eq_rank < need_eq) sel = true;
        }
        const uint64_t sm = __ballot(sel);
        const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sm >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
        if (sel && pos < kmax) out[pos] = t;
        base += __popcll(sm);
    }
    for (int q = base + lane; q < kmax; q += 64) out[q] = -1;
    if (lane == 0) cnt[row] = min(base, kmax);
}

template <int E>
static void launch_wave(bool full, dim3 grid, dim3 block, hipStream_t st, const float* scores, int tk, int tq,
                        int rows, const KBudget& kb, int tpf, int anchor, int32_t* ix, int32_t* cn, int kmax) {
    if (full)
        hipLaunchKernelGGL((k_select_topk_wave<E, true>), grid, block, 0, st, scores, tk, tq, rows, kb, tpf, anchor, ix,
                           cn, kmax);
    else
        hipLaunchKernelGGL((k_select_topk_wave<E, false>), grid, block, 0, st, scores, tk, tq, rows, kb, tpf, anchor, ix,
                           cn, kmax);
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
        // one wave per row while the keys fit 48 registers per lane; longer rows (fewer per
        // launch, and each would hold too many registers) use a workgroup per row
        if (tk <= 64 * 16)
            launch_wave<16>(tk == 64 * 16, wgrid, wblock, st, scores + r0 * tk, tk, tq, rows, kb, tpf, anchor, ix,
                           cnt + r0, kmax);
        else if (tk <= 64 * 32)
            launch_wave<32>(tk == 64 * 32, wgrid, wblock, st, scores + r0 * tk, tk, tq, rows, kb, tpf, anchor, ix,
                           cnt + r0, kmax);
        else if (tk <= 64 * 44)
            launch_wave<44>(tk == 64 * 44, wgrid, wblock, st, scores + r0 * tk, tk, tq, rows, kb, tpf, anchor, ix,
                           cnt + r0, kmax);
        else if (tk <= 64 * 48)
            launch_wave<48>(tk == 64 * 48, wgrid, wblock, st, scores + r0 * tk, tk, tq, rows, kb, tpf, anchor, ix,
                           cnt + r0, kmax);
        else
            hipLaunchKernelGGL(k_select_topk, dim3((unsigned)rows), dim3(TK_THREADS), shm, st,
                               scores + r0 * tk, tk, tq, kb, tpf, anchor, ix, cnt + r0, kmax);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace s3d
