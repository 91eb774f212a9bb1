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

// Tile scores: a 128 x 128 block of scores per workgroup of 256 threads, 8 x 8 per thread
// in fp32 FMAs (four 16-byte LDS reads per 64 FMAs), the 64 dims of the pooled means
// staged in two transposed halves of 32.  sigma = scale * qbar . kbar, -inf where either
// tile has no rows; the block's stores are whole 32-byte row segments.
constexpr int SC2_T = 128;              // queries x keys per workgroup
constexpr int SC2_LD = SC2_T + 4;       // padded row of the transposed halves
__global__ __launch_bounds__(256) void k_tile_scores8(const float* __restrict__ qbar,
                                                      const float* __restrict__ kbar, int Tq, int Tk,
                                                      Lay ql, Lay kl, float scale,
                                                      float* __restrict__ scores) {
    __shared__ __align__(16) float qs[32 * SC2_LD];
    __shared__ __align__(16) float ks[32 * SC2_LD];
    const int tid = threadIdx.x;
    const int tk0 = blockIdx.x * SC2_T, tq0 = blockIdx.y * SC2_T, h = blockIdx.z;
    const float* qb = qbar + (size_t)h * Tq * HD;
    const float* kb = kbar + (size_t)h * Tk * HD;
    const int ty = tid / 16, tx = tid % 16;
    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    for (int half = 0; half < 2; ++half) {
        if (half) __syncthreads();
        // 128 rows x 32 dims of each side: 8 float4 per row, 1024 float4 per side
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int e = tid + 256 * it;
            const int r = e / 8, d4 = e % 8;
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
            if (tq0 + r < Tq) a = *reinterpret_cast<const float4*>(qb + (size_t)(tq0 + r) * HD + 32 * half + 4 * d4);
            if (tk0 + r < Tk) b = *reinterpret_cast<const float4*>(kb + (size_t)(tk0 + r) * HD + 32 * half + 4 * d4);
            qs[(4 * d4 + 0) * SC2_LD + r] = a.x;
            qs[(4 * d4 + 1) * SC2_LD + r] = a.y;
            qs[(4 * d4 + 2) * SC2_LD + r] = a.z;
            qs[(4 * d4 + 3) * SC2_LD + r] = a.w;
            ks[(4 * d4 + 0) * SC2_LD + r] = b.x;
            ks[(4 * d4 + 1) * SC2_LD + r] = b.y;
            ks[(4 * d4 + 2) * SC2_LD + r] = b.z;
            ks[(4 * d4 + 3) * SC2_LD + r] = b.w;
        }
        __syncthreads();
#pragma unroll 4
        for (int d = 0; d < 32; ++d) {
            const float4 a0 = *reinterpret_cast<const float4*>(qs + d * SC2_LD + ty * 8);
            const float4 a1 = *reinterpret_cast<const float4*>(qs + d * SC2_LD + ty * 8 + 4);
            const float4 b0 = *reinterpret_cast<const float4*>(ks + d * SC2_LD + tx * 8);
            const float4 b1 = *reinterpret_cast<const float4*>(ks + d * SC2_LD + tx * 8 + 4);
            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
    }
    bool kempty[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = tk0 + tx * 8 + j;
        int lo, hi;
        member_range(kl, c < Tk ? c : 0, lo, hi);
        kempty[j] = hi <= lo;
    }
    const int c0 = tk0 + tx * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = tq0 + ty * 8 + i;
        if (r >= Tq) continue;
        const bool qempty = valid_rows(ql, r) == 0;
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (qempty || kempty[j]) ? -INFINITY : acc[i][j] * scale;
        float* dst = scores + ((size_t)h * Tq + r) * Tk + c0;
        if ((Tk & 3) == 0 && c0 + 7 < Tk) {
            *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + j < Tk) dst[j] = o[j];
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
    const Lay lq{ql.S, ql.N, ql.P, ql.nsp}, lk{kl.S, kl.N, kl.P, kl.nsp};
    const dim3 grid((Tk + SC2_T - 1) / SC2_T, (Tq + SC2_T - 1) / SC2_T, heads), block(256);
    hipLaunchKernelGGL(k_tile_scores8, grid, block, 0, st, qbar, kbar, Tq, Tk, lq, lk, scale, scores);
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
