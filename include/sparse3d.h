/*
 * sparse3d.h -- C ABI of the dynamic tile-sparse global-attention library (gfx950).
 *
 * The problem these calls solve: a feed-forward 3-D reconstruction transformer runs
 * global attention across all S views x N tokens, and that quadratic step is the cost
 * to cut (SAF3R abstract; Zebra3D abstract).  Zebra3D (abstract) answers it with
 * tile-sparse attention plus landmark summaries of the tiles left out; SAF3R (abstract)
 * keeps, per input, only the most promising interactions; the EPFL page "(Full)
 * Attention is More Than You Need" (figure "Full vs sparse global attention") states
 * the target, O((SN)^2) work cut to O(SNK) with K << SN.  The library computes one such
 * layer in three calls -- tile scores from pooled summaries, per-row top-k with the
 * anchor frame always kept, exact softmax over the selected tiles -- plus a dense call
 * as the reference it is measured against, and the AVGGT 2-D key/value grid subsample
 * (AVGGT technical summary, section 2B.2).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are row-major, contiguous, [heads, frames*stride, head_dim]; a batch folds
 *    into heads.  Row r is in frame r / stride at in-frame position j = r % stride.
 *    A row is a valid query iff j < tokens, a member key of its 64-row tile iff
 *    specials <= j < tokens, a special key iff j < specials.  Pad rows (j >= tokens)
 *    may hold anything, NaN included: kernels select by index and never read them as data.
 *  - Every tensor pointer is DEVICE memory owned by the caller.  No call allocates,
 *    frees, synchronises, or keeps a pointer after it returns.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as void*;
 *    NULL means the default stream).  Calls on one stream run in order.
 *  - Every argument is validated on the host before anything is launched.  On a
 *    nonzero status nothing was launched and no output was written.
 *  - head_dim and tile are 64 (other values return SPARSE3D_ERR_UNSUPPORTED).
 *  - The library has no global mutable state; calls on different streams may overlap.
 */
#ifndef SPARSE3D_H
#define SPARSE3D_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE3D_ABI_VERSION 5

typedef enum { SPARSE3D_F32 = 0, SPARSE3D_BF16 = 1 } sparse3d_dtype;

typedef enum {
    SPARSE3D_OK = 0,
    SPARSE3D_ERR_NULL = 1,        /* a required pointer is NULL */
    SPARSE3D_ERR_SHAPE = 2,       /* sizes or layouts are inconsistent */
    SPARSE3D_ERR_UNSUPPORTED = 3, /* valid request this build does not implement */
    SPARSE3D_ERR_HIP = 4,         /* the HIP runtime reported a launch error */
    SPARSE3D_ERR_ALIAS = 5        /* an output overlaps an input */
} sparse3d_status;

/* One token sequence: `frames` views of `tokens` valid rows each (the first `specials`
 * of them camera/register tokens), every frame padded to `stride` rows. */
/*
 * Completion of the AVGGT key/value subsample (technical summary, section 2B.2): each
 * query keeps its own key when the subsample dropped its position (the diagonal), and
 * the dropped columns are stood in for by one mean key/value pair.  Passed to the
 * attention calls when klay is the layout sparse3d_grid_subsample_kv produced from qlay
 * with (grid_h, grid_w, window); NULL there means neither term.
 *   - own key: k_full/v_full are K and V BEFORE the subsample, in layout qlay and the
 *     operand dtype.  A valid query row i whose in-frame position is a dropped patch gets
 *     one more logit scale * q_i . k_full[i] with value v_full[i].  NULL = no such term.
 *   - mean pair: kmean/vmean [heads, 64] fp32 (sparse3d_discarded_mean).  Every valid
 *     query gets one more logit scale * q_i . kmean[h] + mean_bias with value vmean[h];
 *     mean_bias = ln |D| (|D| = dropped rows of all frames) makes the one pair stand for
 *     all dropped columns.  NULL = no such term.
 */
typedef struct {
    const void* k_full;
    const void* v_full;
    int32_t grid_h, grid_w, window;
    const float* kmean;
    const float* vmean;
    float mean_bias;
} sparse3d_sga;

typedef struct {
    int32_t frames;
    int32_t tokens;
    int32_t stride;   /* multiple of the tile size, >= tokens */
    int32_t specials; /* 0 <= specials < tokens */
} sparse3d_layout;

/* SPARSE3D_ABI_VERSION of the built library. */
int sparse3d_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* sparse3d_status_string(int status);

/*
 * Tile summaries and pooled tile scores (Zebra3D abstract: tile-sparse attention chosen
 * per input; SAF3R abstract: input-dependent selection).
 *
 *   qbar[h,t,:]  = mean of q over the valid query rows of query tile t
 *   kbar[h,t,:]  = mean of k over the member key rows of key tile t
 *   vbar[h,t,:]  = mean of v over the same rows (only when v and vbar are non-NULL;
 *                  these are the landmark values of the sparse call)
 *   scores[h,tq,tk] = scale * qbar[h,tq] . kbar[h,tk], or -inf when either tile has
 *                  no rows to average.  A tile with no rows gets a zero summary.
 *
 * q: [heads, qlay.frames*qlay.stride, 64]; k, v: [heads, klay.frames*klay.stride, 64],
 * element type `dtype`.  qbar: float [heads, Tq, 64]; kbar, vbar: float [heads, Tk, 64];
 * scores: float [heads, Tq, Tk], with Tq = qlay.frames*qlay.stride/tile and
 * Tk = klay.frames*klay.stride/tile.  Sums accumulate in fp32 in a fixed order, so
 * repeated calls are bit-identical.  The score products run on the bf16 matrix cores with
 * each fp32 mean split into two bf16 terms and all four cross products accumulated in
 * fp32, within about 1e-6 (relative) of the fp32 dot product.  v and vbar must be both
 * NULL or both non-NULL.
 *
 * kbar_op, vbar_op (optional, NULL to skip; vbar_op needs v): the key and value means again,
 * in the operand dtype ([heads, Tk, 64] of `dtype`; for BF16 rounded to nearest even, the
 * same values sparse3d_cast gives).  These are the landmark means the attention calls take,
 * written by the same pooling pass, so a bf16 landmark layer needs no separate cast.
 */
int sparse3d_tile_scores(const void* q, const void* k, const void* v, sparse3d_dtype dtype,
                         int32_t heads, int32_t head_dim, int32_t tile,
                         const sparse3d_layout* qlay, const sparse3d_layout* klay, float scale,
                         float* qbar, float* kbar, float* vbar, float* scores, void* kbar_op,
                         void* vbar_op, void* stream);

/*
 * Per query tile: the k key tiles with the largest score (larger first; equal scores,
 * compared as float values so -0 == +0, go to the lower tile index), united with every
 * tile of frame `anchor_frame` (-1: no anchor), written in ascending tile order.
 *
 * scores: float [heads, q_tiles, k_tiles] (NaN is not allowed).  idx: int32
 * [heads, q_tiles, kmax], entries past the count are -1; cnt: int32 [heads, q_tiles].
 * k_tiles must be a multiple of tiles_per_frame (key tiles per frame);
 * kmax >= min(k_tiles, k + (anchor_frame >= 0 ? tiles_per_frame : 0)).  k_tiles is at
 * most 12288 (SPARSE3D_ERR_UNSUPPORTED beyond).  The result depends only on the score values (bit-exact, deterministic).
 */
int sparse3d_select_topk(const float* scores, int32_t heads, int32_t q_tiles, int32_t k_tiles,
                         int32_t k, int32_t tiles_per_frame, int32_t anchor_frame,
                         int32_t* idx, int32_t* cnt, int32_t kmax, void* stream);

/*
 * sparse3d_select_topk with one budget per head: head h keeps its k_heads[h] best tiles
 * (SAF3R abstract: attention patterns differ across heads, so their budgets may too).
 * k_heads is a HOST array of `heads` values >= 0 (read during the call, not kept);
 * kmax must be >= min(Tk, max_h k_heads[h] + anchor tiles).  Everything else as above.
 */
int sparse3d_select_topk_per_head(const float* scores, int32_t heads, int32_t q_tiles, int32_t k_tiles,
                                  const int32_t* k_heads, int32_t tiles_per_frame, int32_t anchor_frame,
                                  int32_t* idx, int32_t* cnt, int32_t kmax, void* stream);

/*
 * Exact softmax attention of each query tile over its selected tiles (Zebra3D abstract:
 * tile-sparse attention with landmark summaries of unselected context; EPFL figure
 * "Full vs sparse global attention": O(SNK) work).
 *
 * For a valid query row i of query tile tq, the attended set is every special key row of
 * every frame plus the member rows of the tiles idx[h,tq,0:cnt[h,tq]]; the logit of key
 * j is scale * q_i . k_j.  With landmarks on (kbar, vbar non-NULL), every key tile that
 * is not selected and has member rows adds one more logit scale * q_i . kbar[h,t] +
 * landmark_bias with value vbar[h,t].  kbar and vbar are the key/value tile means
 * [heads, Tk, 64] in the operand dtype: for F32 the fp32 means sparse3d_tile_scores
 * writes, for BF16 those means rounded to bf16 (the kbar_op/vbar_op outputs of
 * sparse3d_tile_scores, or sparse3d_cast of the fp32 means), which is the precision the
 * matrix cores take them in.
 *   out[h,i,:] = sum_j softmax_j * value_j   (fp32 statistics and accumulation)
 *   lse[h,i]   = natural-log log-sum-exp of the logits (optional, float [heads, Lq])
 * Rows that are not valid queries get out = 0 and lse = 0; a valid query with nothing
 * to attend gets out = 0 and lse = -inf.  idx entries outside [0, Tk) are skipped and
 * cnt is clamped to kmax.  out: [heads, Lq, 64] of `out_dtype` (results rounded to
 * nearest even); it must not overlap q, k or v.  Operands are bf16 (bf16 matrix cores,
 * fp32 accumulation) or fp32 (fp32 matrix cores).  scale must be finite and > 0 and,
 * with landmarks on, landmark_bias finite (SPARSE3D_ERR_UNSUPPORTED otherwise).
 */
int sparse3d_sparse_attn_fwd(const void* q, const void* k, const void* v, sparse3d_dtype dtype,
                             int32_t heads, int32_t head_dim, int32_t tile,
                             const sparse3d_layout* qlay, const sparse3d_layout* klay,
                             const int32_t* idx, const int32_t* cnt, int32_t kmax,
                             const void* kbar, const void* vbar, float landmark_bias,
                             float scale, const sparse3d_sga* sga, void* out, sparse3d_dtype out_dtype,
                             float* lse, void* stream);

/*
 * Dense global attention, the quadratic operation the sparse call replaces (SAF3R
 * abstract; AVGGT technical summary, section 1): every valid query attends every valid
 * key row (specials in place, pad excluded).  Same tensor conventions, outputs and
 * numerics as sparse3d_sparse_attn_fwd; it is the library's own dense baseline.
 */
int sparse3d_dense_attn_fwd(const void* q, const void* k, const void* v, sparse3d_dtype dtype,
                            int32_t heads, int32_t head_dim,
                            const sparse3d_layout* qlay, const sparse3d_layout* klay,
                            float scale, const sparse3d_sga* sga, void* out, sparse3d_dtype out_dtype,
                            float* lse, void* stream);

/*
 * The selection transposed, for the backward pass: for each head h and key tile t, the
 * query tiles whose list (idx/cnt as written by sparse3d_select_topk) holds t, ascending.
 * CSR with end offsets: the list of (h, t) is t_list[h, b .. e) with e = t_end[h, t] and
 * b = t_end[h, t-1] (0 for t = 0).  t_end: int32 [heads, k_tiles]; t_list: int32
 * [heads, q_tiles * kmax] (the first sum-of-counts entries of each head are written).
 * q_tiles <= 16384.  Deterministic (each list is sorted).
 */
int sparse3d_selection_transpose(const int32_t* idx, const int32_t* cnt, int32_t heads, int32_t q_tiles,
                                 int32_t k_tiles, int32_t kmax, int32_t* t_end, int32_t* t_list,
                                 void* stream);

/*
 * Backward of sparse3d_sparse_attn_fwd, for training through the sparse layer (Zebra3D
 * abstract: landmark summaries, post-conversion training; EPFL "(Full) Attention is More
 * Than You Need": sparse training).  The selection is held fixed (top-k is piecewise
 * constant, no gradient flows into the scores).  Inputs: q, k, v, the forward's out and the
 * output cotangent dout (all bf16, layouts as in the forward), the forward's lse, the
 * selection idx/cnt and its transpose t_end/t_list (sparse3d_selection_transpose).  With P
 * the softmax weights and D = rowsum(dout * out):
 *   dS = P * (dout V^T - D),  dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dout
 * (special keys are attended by every query, member keys by the query tiles that selected
 * their tile).  Outputs, fp32 and fully overwritten: dq [heads, Lq, 64] (0 on rows that
 * are not valid queries), dk and dv [heads, Lk, 64] (0 on pad rows and on keys nobody
 * attends), delta [heads, Lq] = D (0 on invalid rows).
 *
 * Landmarks (kbar and vbar non-NULL, as passed to the forward, with its landmark_bias):
 * each tile t with member rows that a query tile did not select is one more key of its
 * rows, kbar[h,t] with value vbar[h,t] and the logit bias.  dkbar and dvbar [heads, Tk, 64]
 * fp32 (required then, fully overwritten) receive the gradients with respect to the means,
 *   dkbar[t] = scale sum_i dS_it q_i,  dvbar[t] = sum_i P_it dout_i
 * (0 for tiles without member rows), and since the forward's means are the averages of
 * K and V over the tile's member rows M(t), dk and dv of every member row also receive
 * dkbar[t] / |M(t)| and dvbar[t] / |M(t)|: dk and dv are then the gradients with respect
 * to K and V through both routes.  dkbar/dvbar NULL with landmarks on: SPARSE3D_ERR_NULL.
 *
 * bf16 operands only (SPARSE3D_ERR_UNSUPPORTED for F32), kmax <= 8000 (7800 with
 * landmarks), Tq <= 16384.  Deterministic: every output element has one writer and a
 * fixed summation order.
 */
int sparse3d_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, sparse3d_dtype dtype, int32_t heads, int32_t head_dim,
                             int32_t tile, const sparse3d_layout* qlay, const sparse3d_layout* klay,
                             const int32_t* idx, const int32_t* cnt, int32_t kmax, const int32_t* t_end,
                             const int32_t* t_list, const void* kbar, const void* vbar, float landmark_bias,
                             float scale, float* dq, float* dk, float* dv, float* delta, float* dkbar,
                             float* dvbar, void* stream);

/*
 * The mean key and mean value of every patch row the grid subsample (grid_h, grid_w,
 * window) drops, over all frames, per head (the pair that stands in for the dropped
 * columns, AVGGT technical summary, section 2B.2): kmean/vmean [heads, 64] fp32,
 * accumulated in fp32 in a fixed order (deterministic).  Zero when nothing is dropped.
 * Requires lay->tokens == lay->specials + grid_h*grid_w.
 */
int sparse3d_discarded_mean(const void* k, const void* v, sparse3d_dtype dtype, int32_t heads,
                            int32_t head_dim, const sparse3d_layout* lay, int32_t grid_h,
                            int32_t grid_w, int32_t window, float* kmean, float* vmean, void* stream);

/*
 * Frame attention: every valid query attends the valid key rows (specials in place) of its
 * OWN frame only, the per-view attention that replaces the early global layers (AVGGT
 * technical summary, section 2B.1: those layers exchange nothing between views, so the
 * O((NL)^2) cost drops to O(NL^2)).  qlay and klay must have the same number of frames
 * (keys may use another layout, e.g. the subsampled one).  Same tensor conventions,
 * outputs, numerics and errors as sparse3d_dense_attn_fwd.
 */
int sparse3d_frame_attn_fwd(const void* q, const void* k, const void* v, sparse3d_dtype dtype,
                            int32_t heads, int32_t head_dim,
                            const sparse3d_layout* qlay, const sparse3d_layout* klay,
                            float scale, void* out, sparse3d_dtype out_dtype, float* lse,
                            void* stream);

/*
 * Elementwise conversion of n fp32 values to `dtype`, rounded to nearest even (F32 is a
 * plain copy).  Used to hand the landmark means to the bf16 attention in the precision
 * its matrix cores read.  n >= 0; dst must not overlap src.
 */
int sparse3d_cast(const float* src, int64_t n, sparse3d_dtype dtype, void* dst, void* stream);

/*
 * Key/value layout after the AVGGT grid subsample (technical summary, section 2B.2):
 * the specials are kept, and of the grid_h x grid_w patch grid only the top-left patch
 * of every window x window cell; the result is padded to a multiple of `tile`.
 * Requires lay->tokens == lay->specials + grid_h*grid_w.  Host-only; writes *out_lay.
 */
int sparse3d_subsample_layout(const sparse3d_layout* lay, int32_t grid_h, int32_t grid_w,
                              int32_t window, int32_t tile, sparse3d_layout* out_lay);

/*
 * Gather the kept key and value rows of every frame (AVGGT technical summary, section
 * 2B.2: keys/values thinned on the 2-D grid, all queries and special tokens kept).
 * k, v: [heads, lay.frames*lay.stride, 64]; k_out, v_out: [heads, out.frames*out.stride,
 * 64], where *out_lay must equal what sparse3d_subsample_layout returns.  Pad rows of
 * the outputs are written as zeros.  Outputs must not overlap inputs.
 */
int sparse3d_grid_subsample_kv(const void* k, const void* v, sparse3d_dtype dtype,
                               int32_t heads, int32_t head_dim, const sparse3d_layout* lay,
                               int32_t grid_h, int32_t grid_w, int32_t window,
                               void* k_out, void* v_out, const sparse3d_layout* out_lay,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE3D_H */
