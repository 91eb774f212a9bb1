// Host-side argument checks for every entry point.  Plain C++ with no HIP
// dependency: each function returns a sparse3d_status and touches nothing.
#pragma once

#include <cstddef>
#include <cstdint>

#include "sparse3d.h"

namespace s3d {

constexpr int kTile = 64;
constexpr int kHeadDim = 64;
constexpr int kMaxTopkTiles = 12288;   // row keys live in LDS (48 KiB)
// Rows per head of any attention operand: one head of bf16 rows (128 bytes each) must stay
// below the 2^31-byte offset at which the kernels place masked rows.
constexpr int64_t kMaxAttnRows = int64_t(1) << 24;
// Tile scores: query tiles up to 65535 grid rows of 128, key tiles so that 64 score rows
// (64 * Tk * 4 bytes) stay within 2^31.
constexpr int64_t kMaxScoreQTiles = int64_t(65535) * 128;
constexpr int64_t kMaxScoreKTiles = int64_t(1) << 23;

inline int64_t lay_rows(const sparse3d_layout& l) { return int64_t(l.frames) * l.stride; }
inline int64_t lay_tiles(const sparse3d_layout& l) { return lay_rows(l) / kTile; }
inline size_t dtype_bytes(sparse3d_dtype d) { return d == SPARSE3D_BF16 ? 2 : 4; }

int check_layout(const sparse3d_layout* l);
int check_dtype(int dt);
int check_heads_dims(int32_t heads, int32_t head_dim, int32_t tile);
// Softmax scale finite and > 0, landmark bias finite: masked logits are -inf, and only a
// positive finite scale keeps them at -inf (exp -> 0) rather than NaN.
int check_logit_params(float scale, float landmark_bias);
// Byte ranges [a, a+na) and [b, b+nb) overlap (both non-empty).
bool overlaps(const void* a, size_t na, const void* b, size_t nb);

int validate_tile_scores(const void* q, const void* k, const void* v, int dtype, int32_t heads,
                         int32_t head_dim, int32_t tile, const sparse3d_layout* qlay,
                         const sparse3d_layout* klay, const float* qbar, const float* kbar,
                         const float* vbar, const float* scores, const void* kbar_op = nullptr,
                         const void* vbar_op = nullptr);

int validate_select_topk(const float* scores, int32_t heads, int32_t q_tiles, int32_t k_tiles,
                         int32_t k, int32_t tiles_per_frame, int32_t anchor_frame,
                         const int32_t* idx, const int32_t* cnt, int32_t kmax);

int validate_attn(bool sparse, const void* q, const void* k, const void* v, int dtype,
                  int32_t heads, int32_t head_dim, int32_t tile, const sparse3d_layout* qlay,
                  const sparse3d_layout* klay, const int32_t* idx, const int32_t* cnt,
                  int32_t kmax, const void* kbar, const void* vbar, const void* out,
                  int out_dtype, const float* lse);

int validate_cast(const float* src, int64_t n, int dtype, const void* dst);

// The subsample completion of an attention call (sga may be NULL: nothing to check).
int validate_sga(const sparse3d_sga* sga, int dtype, int32_t heads, int32_t head_dim,
                 const sparse3d_layout* qlay, const sparse3d_layout* klay, const void* out,
                 int out_dtype, const float* lse);

int validate_discarded_mean(const void* k, const void* v, int dtype, int32_t heads, int32_t head_dim,
                            const sparse3d_layout* lay, int32_t grid_h, int32_t grid_w,
                            int32_t window, const float* kmean, const float* vmean);
int validate_selection_transpose(const int32_t* idx, const int32_t* cnt, int32_t heads, int32_t q_tiles,
                                 int32_t k_tiles, int32_t kmax, const int32_t* t_end, const int32_t* t_list);

int validate_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, int dtype, int32_t heads, int32_t head_dim, int32_t tile,
                      const sparse3d_layout* qlay, const sparse3d_layout* klay, const int32_t* idx,
                      const int32_t* cnt, int32_t kmax, const int32_t* t_end, const int32_t* t_list,
                      const void* kbar, const void* vbar, float landmark_bias, float scale,
                      const float* dq, const float* dk, const float* dv, const float* delta,
                      const float* dkbar, const float* dvbar);

// Longest tile list the backward's dQ kernel stages in LDS (32 KiB of tile buffers beside
// it); with landmarks the landmark bitmap (at most kMaxTopkTiles / 8 bytes) shares that
// room, so the list is shorter.
constexpr int kMaxBwdList = 8000;
constexpr int kMaxBwdListLm = 7800;
// Most query tiles the selection transpose sorts per key tile (LDS bitonic sort).
constexpr int kMaxTransposeQ = 16384;

// Dropped patch rows per frame of the subsample (grid_h, grid_w, window).
int64_t dropped_per_frame(int32_t grid_h, int32_t grid_w, int32_t window);

int subsample_layout(const sparse3d_layout* lay, int32_t grid_h, int32_t grid_w, int32_t window,
                     int32_t tile, sparse3d_layout* out);

int validate_subsample(const void* k, const void* v, int dtype, int32_t heads, int32_t head_dim,
                       const sparse3d_layout* lay, int32_t grid_h, int32_t grid_w, int32_t window,
                       const void* k_out, const void* v_out, const sparse3d_layout* out_lay);

}  // namespace s3d
