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

}  // namespace s3d
