// Kernel launchers (host functions, one per kernel family).  Arguments are
// already validated by the entry points; each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sparse3d.h"

namespace s3d {

struct LayH {
    int S, N, P, nsp;
};
inline LayH to_lay(const sparse3d_layout& l) { return {l.frames, l.tokens, l.stride, l.specials}; }

hipError_t launch_tile_pool(const void* x, int dtype, int heads, LayH lay, bool key_rows, float* out,
                            void* out_op, hipStream_t st);
hipError_t launch_tile_scores(const float* qbar, const float* kbar, int heads, LayH ql, LayH kl,
                              float scale, float* scores, hipStream_t st);
// k_heads: host array of one budget per head
hipError_t launch_select_topk(const float* scores, int heads, int tq, int tk, const int32_t* k_heads, int tpf,
                              int anchor, int32_t* idx, int32_t* cnt, int kmax, hipStream_t st);

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    int dtype, out_dtype;
    int heads;
    LayH ql, kl;
    bool dense;
    bool frame;         // dense over the query's own frame only (needs dense)
    const int32_t* idx;
    const int32_t* cnt;
    int kmax;
    const void* kbar;   // landmark means in the operand dtype; landmarks on iff non-null
    const void* vbar;
    float landmark_bias;
    float scale;
    const sparse3d_sga* sga;   // subsample completion, or NULL
    void* out;
    float* lse;
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);

// Backward of the sparse attention (bf16 operands; fp32 gradients)
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    int heads;
    LayH ql, kl;
    const int32_t* idx;
    const int32_t* cnt;
    int kmax;
    const int32_t* t_end;
    const int32_t* t_list;
    const void* kbar;   // landmark means (bf16); landmarks on iff non-null
    const void* vbar;
    float landmark_bias;
    float scale;
    float* dq;
    float* dk;
    float* dv;
    float* delta;
    float* dkbar;       // gradients of the means (landmarks only)
    float* dvbar;
};
hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t st);
hipError_t launch_selection_transpose(const int32_t* idx, const int32_t* cnt, int heads, int tq, int tk,
                                      int kmax, int32_t* t_end, int32_t* t_list, hipStream_t st);

hipError_t launch_cast(const float* src, int64_t n, int dtype, void* dst, hipStream_t st);

hipError_t launch_discarded_mean(const void* k, const void* v, int dtype, int heads, LayH lay,
                                 int grid_h, int grid_w, int window, int64_t count, float* kmean,
                                 float* vmean, hipStream_t st);

hipError_t launch_grid_subsample(const void* k, const void* v, int dtype, int heads, LayH lay,
                                 int grid_w, int window, LayH out_lay, void* k_out, void* v_out,
                                 hipStream_t st);

}  // namespace s3d
