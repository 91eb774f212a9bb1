// The extern "C" entry points declared in include/sparse3d.h: validate on the host
// (validate.cpp, no HIP), then enqueue the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "launch.h"
#include "sparse3d.h"
#include "validate.h"

using namespace s3d;

#define S3D_HIP(expr)                                       \
    do {                                                    \
        if ((expr) != hipSuccess) return SPARSE3D_ERR_HIP;   \
    } while (0)

extern "C" {

int sparse3d_abi_version(void) { return SPARSE3D_ABI_VERSION; }

const char* sparse3d_status_string(int status) {
    switch (status) {
        case SPARSE3D_OK: return "ok";
        case SPARSE3D_ERR_NULL: return "a required pointer is NULL";
        case SPARSE3D_ERR_SHAPE: return "inconsistent sizes or layout";
        case SPARSE3D_ERR_UNSUPPORTED: return "unsupported size, dtype or option";
        case SPARSE3D_ERR_HIP: return "HIP runtime error at launch";
        case SPARSE3D_ERR_ALIAS: return "an output overlaps an input";
        default: return "unknown status";
    }
}

int sparse3d_tile_scores(const void* q, const void* k, const void* v, sparse3d_dtype dtype,
                         int32_t heads, int32_t head_dim, int32_t tile,
                         const sparse3d_layout* qlay, const sparse3d_layout* klay, float scale,
                         float* qbar, float* kbar, float* vbar, float* scores, void* kbar_op,
                         void* vbar_op, void* stream) {
    const int st = validate_tile_scores(q, k, v, dtype, heads, head_dim, tile, qlay, klay, qbar,
                                        kbar, vbar, scores, kbar_op, vbar_op);
    if (st != SPARSE3D_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const LayH ql = to_lay(*qlay), kl = to_lay(*klay);
    S3D_HIP(launch_tile_pool(q, dtype, heads, ql, false, qbar, nullptr, s));
    S3D_HIP(launch_tile_pool(k, dtype, heads, kl, true, kbar, kbar_op, s));
    if (v) S3D_HIP(launch_tile_pool(v, dtype, heads, kl, true, vbar, vbar_op, s));
    S3D_HIP(launch_tile_scores(qbar, kbar, heads, ql, kl, scale, scores, s));
    return SPARSE3D_OK;
}

int sparse3d_select_topk(const float* scores, int32_t heads, int32_t q_tiles, int32_t k_tiles,
                         int32_t k, int32_t tiles_per_frame, int32_t anchor_frame, int32_t* idx,
                         int32_t* cnt, int32_t kmax, void* stream) {
    const int st = validate_select_topk(scores, heads, q_tiles, k_tiles, k, tiles_per_frame,
                                        anchor_frame, idx, cnt, kmax);
    if (st != SPARSE3D_OK) return st;
    const std::vector<int32_t> ks(size_t(heads), k);
    S3D_HIP(launch_select_topk(scores, heads, q_tiles, k_tiles, ks.data(), tiles_per_frame, anchor_frame,
                               idx, cnt, kmax, static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

int sparse3d_select_topk_per_head(const float* scores, int32_t heads, int32_t q_tiles, int32_t k_tiles,
                                  const int32_t* k_heads, int32_t tiles_per_frame, int32_t anchor_frame,
                                  int32_t* idx, int32_t* cnt, int32_t kmax, void* stream) {
    if (!k_heads) return SPARSE3D_ERR_NULL;
    if (heads < 1) return SPARSE3D_ERR_SHAPE;
    int32_t kbig = 0;
    for (int32_t h = 0; h < heads; ++h) {
        if (k_heads[h] < 0) return SPARSE3D_ERR_SHAPE;
        kbig = std::max(kbig, k_heads[h]);
    }
    const int st = validate_select_topk(scores, heads, q_tiles, k_tiles, kbig, tiles_per_frame,
                                        anchor_frame, idx, cnt, kmax);
    if (st != SPARSE3D_OK) return st;
    S3D_HIP(launch_select_topk(scores, heads, q_tiles, k_tiles, k_heads, tiles_per_frame, anchor_frame,
                               idx, cnt, kmax, static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

int sparse3d_sparse_attn_fwd(const void* q, const void* k, const void* v, sparse3d_dtype dtype,
                             int32_t heads, int32_t head_dim, int32_t tile,
                             const sparse3d_layout* qlay, const sparse3d_layout* klay,
                             const int32_t* idx, const int32_t* cnt, int32_t kmax,
                             const void* kbar, const void* vbar, float landmark_bias,
                             float scale, const sparse3d_sga* sga, void* out, sparse3d_dtype out_dtype,
                             float* lse, void* stream) {
    const int st = validate_attn(true, q, k, v, dtype, heads, head_dim, tile, qlay, klay, idx, cnt,
                                 kmax, kbar, vbar, out, out_dtype, lse);
    if (st != SPARSE3D_OK) return st;
    const int sp = check_logit_params(scale, kbar ? landmark_bias : 0.f);
    if (sp != SPARSE3D_OK) return sp;
    const int sg = validate_sga(sga, dtype, heads, head_dim, qlay, klay, out, out_dtype, lse);
    if (sg != SPARSE3D_OK) return sg;
    AttnArgs a{q, k, v, dtype, out_dtype, heads, to_lay(*qlay), to_lay(*klay), false, false, idx, cnt,
               kmax, kbar, vbar, landmark_bias, scale, sga, out, lse};
    S3D_HIP(launch_attn(a, static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

int sparse3d_cast(const float* src, int64_t n, sparse3d_dtype dtype, void* dst, void* stream) {
    const int st = validate_cast(src, n, dtype, dst);
    if (st != SPARSE3D_OK) return st;
    if (n == 0) return SPARSE3D_OK;
    S3D_HIP(launch_cast(src, n, dtype, dst, static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

int sparse3d_dense_attn_fwd(const void* q, const void* k, const void* v, sparse3d_dtype dtype,
                            int32_t heads, int32_t head_dim, const sparse3d_layout* qlay,
                            const sparse3d_layout* klay, float scale, const sparse3d_sga* sga,
                            void* out, sparse3d_dtype out_dtype, float* lse, void* stream) {
    const int st = validate_attn(false, q, k, v, dtype, heads, head_dim, kTile, qlay, klay, nullptr,
                                 nullptr, 0, nullptr, nullptr, out, out_dtype, lse);
    if (st != SPARSE3D_OK) return st;
    const int sp = check_logit_params(scale, 0.f);
    if (sp != SPARSE3D_OK) return sp;
    const int sg = validate_sga(sga, dtype, heads, head_dim, qlay, klay, out, out_dtype, lse);
    if (sg != SPARSE3D_OK) return sg;
    AttnArgs a{q, k, v, dtype, out_dtype, heads, to_lay(*qlay), to_lay(*klay), true, false, nullptr,
               nullptr, 0, nullptr, nullptr, 0.f, scale, sga, out, lse};
    S3D_HIP(launch_attn(a, static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

int sparse3d_frame_attn_fwd(const void* q, const void* k, const void* v, sparse3d_dtype dtype,
                            int32_t heads, int32_t head_dim, const sparse3d_layout* qlay,
                            const sparse3d_layout* klay, float scale, void* out,
                            sparse3d_dtype out_dtype, float* lse, void* stream) {
    const int st = validate_attn(false, q, k, v, dtype, heads, head_dim, kTile, qlay, klay, nullptr,
                                 nullptr, 0, nullptr, nullptr, out, out_dtype, lse);
    if (st != SPARSE3D_OK) return st;
    const int sp = check_logit_params(scale, 0.f);
    if (sp != SPARSE3D_OK) return sp;
    AttnArgs a{q, k, v, dtype, out_dtype, heads, to_lay(*qlay), to_lay(*klay), true, true, nullptr,
               nullptr, 0, nullptr, nullptr, 0.f, scale, nullptr, out, lse};
    S3D_HIP(launch_attn(a, static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

int sparse3d_discarded_mean(const void* k, const void* v, sparse3d_dtype dtype, int32_t heads,
                            int32_t head_dim, const sparse3d_layout* lay, int32_t grid_h,
                            int32_t grid_w, int32_t window, float* kmean, float* vmean, void* stream) {
    const int st = validate_discarded_mean(k, v, dtype, heads, head_dim, lay, grid_h, grid_w, window,
                                           kmean, vmean);
    if (st != SPARSE3D_OK) return st;
    const int64_t count = int64_t(lay->frames) * dropped_per_frame(grid_h, grid_w, window);
    S3D_HIP(launch_discarded_mean(k, v, dtype, heads, to_lay(*lay), grid_h, grid_w, window, count, kmean,
                                  vmean, static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

int sparse3d_selection_transpose(const int32_t* idx, const int32_t* cnt, int32_t heads, int32_t q_tiles,
                                 int32_t k_tiles, int32_t kmax, int32_t* t_end, int32_t* t_list,
                                 void* stream) {
    const int st = validate_selection_transpose(idx, cnt, heads, q_tiles, k_tiles, kmax, t_end, t_list);
    if (st != SPARSE3D_OK) return st;
    S3D_HIP(launch_selection_transpose(idx, cnt, heads, q_tiles, k_tiles, kmax, t_end, t_list,
                                       static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

int sparse3d_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, sparse3d_dtype dtype, int32_t heads, int32_t head_dim,
                             int32_t tile, const sparse3d_layout* qlay, const sparse3d_layout* klay,
                             const int32_t* idx, const int32_t* cnt, int32_t kmax, const int32_t* t_end,
                             const int32_t* t_list, const void* kbar, const void* vbar, float landmark_bias,
                             float scale, float* dq, float* dk, float* dv, float* delta, float* dkbar,
                             float* dvbar, void* stream) {
    const int st = validate_attn_bwd(q, k, v, out, dout, lse, dtype, heads, head_dim, tile, qlay, klay, idx,
                                     cnt, kmax, t_end, t_list, kbar, vbar, landmark_bias, scale, dq, dk, dv,
                                     delta, dkbar, dvbar);
    if (st != SPARSE3D_OK) return st;
    BwdArgs a{q,      k,     v,    out,  dout,          lse,   heads, to_lay(*qlay), to_lay(*klay),
              idx,    cnt,   kmax, t_end, t_list,       kbar,  vbar,  landmark_bias, scale,
              dq,     dk,    dv,   delta, kbar ? dkbar : nullptr, kbar ? dvbar : nullptr};
    S3D_HIP(launch_attn_bwd(a, static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

int sparse3d_subsample_layout(const sparse3d_layout* lay, int32_t grid_h, int32_t grid_w,
                              int32_t window, int32_t tile, sparse3d_layout* out_lay) {
    return subsample_layout(lay, grid_h, grid_w, window, tile, out_lay);
}

int sparse3d_grid_subsample_kv(const void* k, const void* v, sparse3d_dtype dtype, int32_t heads,
                               int32_t head_dim, const sparse3d_layout* lay, int32_t grid_h,
                               int32_t grid_w, int32_t window, void* k_out, void* v_out,
                               const sparse3d_layout* out_lay, void* stream) {
    const int st = validate_subsample(k, v, dtype, heads, head_dim, lay, grid_h, grid_w, window,
                                      k_out, v_out, out_lay);
    if (st != SPARSE3D_OK) return st;
    S3D_HIP(launch_grid_subsample(k, v, dtype, heads, to_lay(*lay), grid_w, window,
                                  to_lay(*out_lay), k_out, v_out, static_cast<hipStream_t>(stream)));
    return SPARSE3D_OK;
}

}  // extern "C"
