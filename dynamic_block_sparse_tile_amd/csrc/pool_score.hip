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

// scores[h, tq, tk] = scale * qbar[h,tq] . kbar[h,tk] (-inf if either tile is empty).
// 64x64 output block per workgroup of 256 threads, 4x4 outputs per thread; both
// operand blocks are staged transposed in LDS so each inner step is two float4 reads.
// The dot product is one fp32 FMA chain over d = 0..63, a fixed order.
constexpr int SC_LD = 68;

__global__ __launch_bounds__(256) void k_tile_scores(const float* __restrict__ qbar,
                                                     const float* __restrict__ kbar, int Tq, int Tk,
                                                     Lay ql, Lay kl, float scale,
                                                     float* __restrict__ scores) {
    __shared__ __align__(16) float qs[HD * SC_LD];
    __shared__ __align__(16) float ks[HD * SC_LD];
    const int tid = threadIdx.x;
    const int tk0 = blockIdx.x * 64, tq0 = blockIdx.y * 64, h = blockIdx.z;
    const float* qb = qbar + (size_t)h * Tq * HD;
    const float* kb = kbar + (size_t)h * Tk * HD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tid / 16 + 16 * i, d4 = tid % 16;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (tq0 + r < Tq) a = *reinterpret_cast<const float4*>(qb + (size_t)(tq0 + r) * HD + d4 * 4);
        if (tk0 + r < Tk) b = *reinterpret_cast<const float4*>(kb + (size_t)(tk0 + r) * HD + d4 * 4);
        qs[(d4 * 4 + 0) * SC_LD + r] = a.x;
        qs[(d4 * 4 + 1) * SC_LD + r] = a.y;
        qs[(d4 * 4 + 2) * SC_LD + r] = a.z;
        qs[(d4 * 4 + 3) * SC_LD + r] = a.w;
        ks[(d4 * 4 + 0) * SC_LD + r] = b.x;
        ks[(d4 * 4 + 1) * SC_LD + r] = b.y;
        ks[(d4 * 4 + 2) * SC_LD + r] = b.z;
        ks[(d4 * 4 + 3) * SC_LD + r] = b.w;
    }
    __syncthreads();
    const int ty = tid / 16, tx = tid % 16;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
#pragma unroll 8
    for (int d = 0; d < HD; ++d) {
        const float4 a = *reinterpret_cast<const float4*>(qs + d * SC_LD + ty * 4);
        const float4 b = *reinterpret_cast<const float4*>(ks + d * SC_LD + tx * 4);
        const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    int kl_lo[4], kl_hi[4];
    bool kempty[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tk0 + tx * 4 + j;
        member_range(kl, c < Tk ? c : 0, kl_lo[j], kl_hi[j]);
        kempty[j] = kl_hi[j] <= kl_lo[j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tq0 + ty * 4 + i;
        if (r >= Tq) continue;
        const bool qempty = valid_rows(ql, r) == 0;
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = (qempty || kempty[j]) ? -INFINITY : acc[i][j] * scale;
        float* dst = scores + ((size_t)h * Tq + r) * Tk + tk0 + tx * 4;
        if ((Tk & 3) == 0 && tk0 + tx * 4 + 3 < Tk) {
            *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (tk0 + tx * 4 + j < Tk) dst[j] = o[j];
        }
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
    const dim3 grid((Tk + 63) / 64, (Tq + 63) / 64, heads), block(256);
    hipLaunchKernelGGL(k_tile_scores, grid, block, 0, st, qbar, kbar, Tq, Tk,
                       Lay{ql.S, ql.N, ql.P, ql.nsp}, Lay{kl.S, kl.N, kl.P, kl.nsp}, scale, scores);
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
