// AVGGT grid subsample of keys and values (technical summary, section 2B.2): every
// frame keeps its special tokens and, of its grid_h x grid_w patch grid, the top-left
// patch of each window x window cell (row-major); queries are not touched.  A plain
// gather: one thread per 16-byte chunk of an output row, pad rows written as zeros.
#include "device.h"
#include "launch.h"

namespace s3d {

template <typename Chunk>
__global__ __launch_bounds__(256) void k_grid_subsample(const Chunk* __restrict__ k,
                                                        const Chunk* __restrict__ v, int H, Lay in,
                                                        Lay out, int grid_w, int window,
                                                        Chunk* __restrict__ ko, Chunk* __restrict__ vo,
                                                        int chunks_per_row) {
    const size_t total = (size_t)H * out.S * out.P * chunks_per_row;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int ch = (int)(i % chunks_per_row);
    const size_t rowg = i / chunks_per_row;             // h * Lout + r
    const int Lout = out.S * out.P;
    const int h = (int)(rowg / Lout), r = (int)(rowg % Lout);
    const int s = r / out.P, j = r % out.P;
    Chunk zk{}, zv{};
    if (j < out.N) {
        int src;
        if (j < out.nsp) {
            src = j;
        } else {
            const int kw = (grid_w + window - 1) / window;
            const int pidx = j - out.nsp;
            const int y = (pidx / kw) * window, x = (pidx % kw) * window;
            src = in.nsp + y * grid_w + x;
        }
        const size_t si = ((size_t)h * in.S * in.P + (size_t)s * in.P + src) * chunks_per_row + ch;
        zk = k[si];
        zv = v[si];
    }
    ko[i] = zk;
    vo[i] = zv;
}

hipError_t launch_grid_subsample(const void* k, const void* v, int dtype, int heads, LayH lay,
                                 int grid_w, int window, LayH out_lay, void* k_out, void* v_out,
                                 hipStream_t st) {
    const int cpr = dtype == SPARSE3D_BF16 ? HD * 2 / 16 : HD * 4 / 16;
    const size_t total = (size_t)heads * out_lay.S * out_lay.P * cpr;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    const Lay in{lay.S, lay.N, lay.P, lay.nsp}, ol{out_lay.S, out_lay.N, out_lay.P, out_lay.nsp};
    hipLaunchKernelGGL(k_grid_subsample<uint4>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const uint4*>(k), static_cast<const uint4*>(v), heads, in, ol,
                       grid_w, window, static_cast<uint4*>(k_out), static_cast<uint4*>(v_out), cpr);
    return hipGetLastError();
}

// Mean key and value of the dropped patch rows, per head (the pair standing in for the
// dropped columns).  Block (h, c8) owns head h and dims 8*c8 .. +8; every thread walks a
// fixed stride of patch rows of all frames, skips the kept ones and sums in fp32; the
// block then adds the per-thread sums in a fixed tree, so the result is deterministic.
constexpr int DM_THREADS = 512;

template <bool F32IN>
__global__ __launch_bounds__(DM_THREADS) void k_discarded_mean(const void* __restrict__ k,
                                                               const void* __restrict__ v, Lay lay,
                                                               int grid_w, int window, int npatch,
                                                               float inv_count, float* __restrict__ kmean,
                                                               float* __restrict__ vmean) {
    __shared__ float s_acc[DM_THREADS][17];          // 8 key + 8 value sums (+1: bank spread)
    const int h = blockIdx.x, c8 = blockIdx.y, tid = threadIdx.x;
    const size_t hb = (size_t)h * lay.S * lay.P;
    float ak[8] = {}, av[8] = {};
    const int total = lay.S * npatch;
    for (int u = tid; u < total; u += DM_THREADS) {
        const int s = u / npatch, pidx = u - s * npatch;
        const int y = pidx / grid_w, x = pidx - y * grid_w;
        if ((y % window) == 0 && (x % window) == 0) continue;     // kept by the subsample
        const size_t off = (hb + (size_t)s * lay.P + lay.nsp + pidx) * HD + 8 * c8;
        if (F32IN) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(k) + off + 4 * hf);
                const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(v) + off + 4 * hf);
                ak[4 * hf] += a.x; ak[4 * hf + 1] += a.y; ak[4 * hf + 2] += a.z; ak[4 * hf + 3] += a.w;
                av[4 * hf] += b.x; av[4 * hf + 1] += b.y; av[4 * hf + 2] += b.z; av[4 * hf + 3] += b.w;
            }
        } else {
            const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k) + off);
            const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(v) + off);
            const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ak[2 * i] += __uint_as_float(wa[i] << 16);
                ak[2 * i + 1] += __uint_as_float(wa[i] & 0xffff0000u);
                av[2 * i] += __uint_as_float(wb[i] << 16);
                av[2 * i + 1] += __uint_as_float(wb[i] & 0xffff0000u);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        s_acc[tid][i] = ak[i];
        s_acc[tid][8 + i] = av[i];
    }
    __syncthreads();
    for (int stride = DM_THREADS / 2; stride > 0; stride >>= 1) {
        if (tid < stride) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s_acc[tid][i] += s_acc[tid + stride][i];
        }
        __syncthreads();
    }
    if (tid < 16) {
        const float r = s_acc[0][tid] * inv_count;
        (tid < 8 ? kmean : vmean)[(size_t)h * HD + 8 * c8 + (tid & 7)] = r;
    }
}

hipError_t launch_discarded_mean(const void* k, const void* v, int dtype, int heads, LayH lay,
                                 int grid_h, int grid_w, int window, int64_t count, float* kmean,
                                 float* vmean, hipStream_t st) {
    const Lay L{lay.S, lay.N, lay.P, lay.nsp};
    const float inv = count > 0 ? 1.0f / (float)count : 0.f;
    const dim3 grid((unsigned)heads, HD / 8);
    if (dtype == SPARSE3D_F32)
        hipLaunchKernelGGL(k_discarded_mean<true>, grid, dim3(DM_THREADS), 0, st, k, v, L, grid_w, window,
                           grid_h * grid_w, inv, kmean, vmean);
    else
        hipLaunchKernelGGL(k_discarded_mean<false>, grid, dim3(DM_THREADS), 0, st, k, v, L, grid_w, window,
                           grid_h * grid_w, inv, kmean, vmean);
    return hipGetLastError();
}

}  // namespace s3d
