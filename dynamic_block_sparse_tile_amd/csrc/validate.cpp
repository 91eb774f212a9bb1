// Host-side argument checks (no HIP).  Every entry point runs these before it
// launches anything, so a rejected call has no side effects.
#include "validate.h"

#include <algorithm>
#include <cmath>
#include <cstdint>

namespace s3d {

int check_layout(const sparse3d_layout* l) {
    if (!l) return SPARSE3D_ERR_NULL;
    if (l->frames < 1 || l->tokens < 1 || l->stride < 1) return SPARSE3D_ERR_SHAPE;
    if (l->tokens > l->stride) return SPARSE3D_ERR_SHAPE;
    if (l->specials < 0 || l->specials >= l->tokens) return SPARSE3D_ERR_SHAPE;
    if (l->stride % kTile != 0) return SPARSE3D_ERR_SHAPE;
    // row indices are int32 inside the kernels
    if (lay_rows(*l) > (int64_t(1) << 30)) return SPARSE3D_ERR_UNSUPPORTED;
    return SPARSE3D_OK;
}

int check_dtype(int dt) {
    return (dt == SPARSE3D_F32 || dt == SPARSE3D_BF16) ? SPARSE3D_OK : SPARSE3D_ERR_UNSUPPORTED;
}

int check_heads_dims(int32_t heads, int32_t head_dim, int32_t tile) {
    if (heads < 1 || head_dim < 1 || tile < 1) return SPARSE3D_ERR_SHAPE;
    if (head_dim != kHeadDim || tile != kTile) return SPARSE3D_ERR_UNSUPPORTED;
    if (heads > 65535) return SPARSE3D_ERR_UNSUPPORTED;
    return SPARSE3D_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

#define S3D_TRY(expr)                      \
    do {                                   \
        int _st = (expr);                  \
        if (_st != SPARSE3D_OK) return _st; \
    } while (0)

int check_logit_params(float scale, float landmark_bias) {
    if (!(std::isfinite(scale) && scale > 0.f) || !std::isfinite(landmark_bias))
        return SPARSE3D_ERR_UNSUPPORTED;
    return SPARSE3D_OK;
}

int validate_tile_scores(const void* q, const void* k, const void* v, int dtype, int32_t heads,
                         int32_t head_dim, int32_t tile, const sparse3d_layout* qlay,
                         const sparse3d_layout* klay, const float* qbar, const float* kbar,
                         const float* vbar, const float* scores, const void* kbar_op, const void* vbar_op) {
    if (!q || !k || !qbar || !kbar || !scores) return SPARSE3D_ERR_NULL;
    if ((v == nullptr) != (vbar == nullptr)) return SPARSE3D_ERR_NULL;
    if (vbar_op && !v) return SPARSE3D_ERR_NULL;         // value means need the values
    S3D_TRY(check_dtype(dtype));
    S3D_TRY(check_heads_dims(heads, head_dim, tile));
    S3D_TRY(check_layout(qlay));
    S3D_TRY(check_layout(klay));
    if (qlay->frames != klay->frames) return SPARSE3D_ERR_SHAPE;
    // the score kernel takes 128 query tiles per grid row (at most 65535 rows) and addresses
    // 64 score rows per wave with 32-bit offsets (64 * Tk * 4 bytes)
    if (lay_tiles(*qlay) > kMaxScoreQTiles || lay_tiles(*klay) > kMaxScoreKTiles) return SPARSE3D_ERR_UNSUPPORTED;
    const size_t eb = dtype_bytes(sparse3d_dtype(dtype));
    const size_t qb = size_t(heads) * lay_rows(*qlay) * head_dim * eb;
    const size_t kb = size_t(heads) * lay_rows(*klay) * head_dim * eb;
    const size_t Tq = lay_tiles(*qlay), Tk = lay_tiles(*klay);
    const size_t qbar_b = size_t(heads) * Tq * head_dim * 4;
    const size_t kbar_b = size_t(heads) * Tk * head_dim * 4;
    const size_t op_b = size_t(heads) * Tk * head_dim * eb;   // means in the operand dtype
    const size_t sc_b = size_t(heads) * Tq * Tk * 4;
    constexpr int NO = 6;
    const void* outs[NO] = {qbar, kbar, vbar, scores, kbar_op, vbar_op};
    const size_t outn[NO] = {qbar_b, kbar_b, vbar ? kbar_b : 0, sc_b, op_b, op_b};
    for (int i = 0; i < NO; ++i) {
        if (overlaps(outs[i], outn[i], q, qb) || overlaps(outs[i], outn[i], k, kb) ||
            overlaps(outs[i], outn[i], v, kb))
            return SPARSE3D_ERR_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlaps(outs[i], outn[i], outs[j], outn[j])) return SPARSE3D_ERR_ALIAS;
    }
    return SPARSE3D_OK;
}

int validate_select_topk(const float* scores, int32_t heads, int32_t q_tiles, int32_t k_tiles,
                         int32_t k, int32_t tiles_per_frame, int32_t anchor_frame,
                         const int32_t* idx, const int32_t* cnt, int32_t kmax) {
    if (!scores || !cnt) return SPARSE3D_ERR_NULL;
    if (kmax > 0 && !idx) return SPARSE3D_ERR_NULL;
    if (heads < 1 || q_tiles < 1 || k_tiles < 1 || k < 0 || tiles_per_frame < 1 || kmax < 0)
        return SPARSE3D_ERR_SHAPE;
    if (k_tiles % tiles_per_frame != 0) return SPARSE3D_ERR_SHAPE;
    if (anchor_frame < -1 || anchor_frame >= k_tiles / tiles_per_frame) return SPARSE3D_ERR_SHAPE;
    const int64_t need = std::min<int64_t>(
        k_tiles, int64_t(k) + (anchor_frame >= 0 ? tiles_per_frame : 0));
    if (kmax < need) return SPARSE3D_ERR_SHAPE;
    if (k_tiles > kMaxTopkTiles) return SPARSE3D_ERR_UNSUPPORTED;
    if (heads > 65535) return SPARSE3D_ERR_UNSUPPORTED;
    const size_t sb = size_t(heads) * q_tiles * k_tiles * 4;
    const size_t ib = size_t(heads) * q_tiles * kmax * 4;
    const size_t cb = size_t(heads) * q_tiles * 4;
    if (overlaps(idx, ib, scores, sb) || overlaps(cnt, cb, scores, sb) || overlaps(idx, ib, cnt, cb))
        return SPARSE3D_ERR_ALIAS;
    return SPARSE3D_OK;
}

int validate_attn(bool sparse, const void* q, const void* k, const void* v, int dtype,
                  int32_t heads, int32_t head_dim, int32_t tile, const sparse3d_layout* qlay,
                  const sparse3d_layout* klay, const int32_t* idx, const int32_t* cnt,
                  int32_t kmax, const void* kbar, const void* vbar, const void* out,
                  int out_dtype, const float* lse) {
    if (!q || !k || !v || !out) return SPARSE3D_ERR_NULL;
    if (sparse) {
        if (!cnt) return SPARSE3D_ERR_NULL;
        if (kmax > 0 && !idx) return SPARSE3D_ERR_NULL;
        if (kmax < 0) return SPARSE3D_ERR_SHAPE;
        if ((kbar == nullptr) != (vbar == nullptr)) return SPARSE3D_ERR_NULL;
    }
    S3D_TRY(check_dtype(dtype));
    S3D_TRY(check_dtype(out_dtype));
    S3D_TRY(check_heads_dims(heads, head_dim, tile));
    S3D_TRY(check_layout(qlay));
    S3D_TRY(check_layout(klay));
    if (qlay->frames != klay->frames) return SPARSE3D_ERR_SHAPE;
    if (sparse && lay_tiles(*klay) > kMaxTopkTiles) return SPARSE3D_ERR_UNSUPPORTED;
    // the bf16 kernels address one head of K/V (and, in the backward, Q) through a buffer
    // resource with 32-bit offsets, masked rows at an offset of 2^31 past its start
    if (lay_rows(*qlay) > kMaxAttnRows || lay_rows(*klay) > kMaxAttnRows) return SPARSE3D_ERR_UNSUPPORTED;
    if (int64_t(heads) * lay_tiles(*qlay) > (int64_t(1) << 31) - 1) return SPARSE3D_ERR_UNSUPPORTED;
    const size_t eb = dtype_bytes(sparse3d_dtype(dtype));
    const size_t qb = size_t(heads) * lay_rows(*qlay) * head_dim * eb;
    const size_t kb = size_t(heads) * lay_rows(*klay) * head_dim * eb;
    const size_t ob = size_t(heads) * lay_rows(*qlay) * head_dim * dtype_bytes(sparse3d_dtype(out_dtype));
    const size_t lb = size_t(heads) * lay_rows(*qlay) * 4;
    if (overlaps(out, ob, q, qb) || overlaps(out, ob, k, kb) || overlaps(out, ob, v, kb))
        return SPARSE3D_ERR_ALIAS;
    if (overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) ||
        overlaps(lse, lb, out, ob))
        return SPARSE3D_ERR_ALIAS;
    if (sparse && kbar) {
        const size_t mb = size_t(heads) * lay_tiles(*klay) * head_dim * eb;   // landmark means
        if (overlaps(out, ob, kbar, mb) || overlaps(out, ob, vbar, mb) || overlaps(lse, lb, kbar, mb) ||
            overlaps(lse, lb, vbar, mb))
            return SPARSE3D_ERR_ALIAS;
    }
    return SPARSE3D_OK;
}

int64_t dropped_per_frame(int32_t grid_h, int32_t grid_w, int32_t window) {
    const int64_t kh = (grid_h + window - 1) / window, kw = (grid_w + window - 1) / window;
    return int64_t(grid_h) * grid_w - kh * kw;
}

int validate_sga(const sparse3d_sga* sga, int dtype, int32_t heads, int32_t head_dim,
                 const sparse3d_layout* qlay, const sparse3d_layout* klay, const void* out,
                 int out_dtype, const float* lse) {
    if (!sga) return SPARSE3D_OK;
    if ((sga->k_full == nullptr) != (sga->v_full == nullptr)) return SPARSE3D_ERR_NULL;
    if ((sga->kmean == nullptr) != (sga->vmean == nullptr)) return SPARSE3D_ERR_NULL;
    // klay must be exactly the subsample of qlay
    sparse3d_layout want;
    S3D_TRY(subsample_layout(qlay, sga->grid_h, sga->grid_w, sga->window, kTile, &want));
    if (klay->frames != want.frames || klay->tokens != want.tokens || klay->stride != want.stride ||
        klay->specials != want.specials)
        return SPARSE3D_ERR_SHAPE;
    if (sga->kmean && !std::isfinite(sga->mean_bias)) return SPARSE3D_ERR_UNSUPPORTED;
    const size_t eb = dtype_bytes(sparse3d_dtype(dtype));
    const size_t fb = size_t(heads) * lay_rows(*qlay) * head_dim * eb;       // k_full / v_full
    const size_t mb = size_t(heads) * head_dim * 4;                          // kmean / vmean
    const size_t ob = size_t(heads) * lay_rows(*qlay) * head_dim * dtype_bytes(sparse3d_dtype(out_dtype));
    const size_t lb = size_t(heads) * lay_rows(*qlay) * 4;
    const void* ins[4] = {sga->k_full, sga->v_full, sga->kmean, sga->vmean};
    const size_t inb[4] = {fb, fb, mb, mb};
    for (int i = 0; i < 4; ++i)
        if (overlaps(out, ob, ins[i], inb[i]) || overlaps(lse, lb, ins[i], inb[i])) return SPARSE3D_ERR_ALIAS;
    return SPARSE3D_OK;
}

int validate_discarded_mean(const void* k, const void* v, int dtype, int32_t heads, int32_t head_dim,
                            const sparse3d_layout* lay, int32_t grid_h, int32_t grid_w,
                            int32_t window, const float* kmean, const float* vmean) {
    if (!k || !v || !kmean || !vmean) return SPARSE3D_ERR_NULL;
    S3D_TRY(check_dtype(dtype));
    S3D_TRY(check_heads_dims(heads, head_dim, kTile));
    sparse3d_layout sub;
    S3D_TRY(subsample_layout(lay, grid_h, grid_w, window, kTile, &sub));
    const size_t ib = size_t(heads) * lay_rows(*lay) * head_dim * dtype_bytes(sparse3d_dtype(dtype));
    const size_t mb = size_t(heads) * head_dim * 4;
    if (overlaps(kmean, mb, k, ib) || overlaps(kmean, mb, v, ib) || overlaps(vmean, mb, k, ib) ||
        overlaps(vmean, mb, v, ib) || overlaps(kmean, mb, vmean, mb))
        return SPARSE3D_ERR_ALIAS;
    return SPARSE3D_OK;
}

namespace {
// any two of n byte ranges overlap
bool any_overlap(const void* const* p, const size_t* n, int count) {
    for (int i = 0; i < count; ++i)
        for (int j = i + 1; j < count; ++j)
            if (overlaps(p[i], n[i], p[j], n[j])) return true;
    return false;
}
}  // namespace

int validate_selection_transpose(const int32_t* idx, const int32_t* cnt, int32_t heads, int32_t q_tiles,
                                 int32_t k_tiles, int32_t kmax, const int32_t* t_end, const int32_t* t_list) {
    if (!cnt || !t_end) return SPARSE3D_ERR_NULL;
    if (kmax > 0 && (!idx || !t_list)) return SPARSE3D_ERR_NULL;
    if (heads < 1 || q_tiles < 1 || k_tiles < 1 || kmax < 0) return SPARSE3D_ERR_SHAPE;
    if (q_tiles > kMaxTransposeQ || k_tiles > kMaxTopkTiles) return SPARSE3D_ERR_UNSUPPORTED;
    const size_t ib = size_t(heads) * q_tiles * kmax * 4, cb = size_t(heads) * q_tiles * 4;
    const size_t eb = size_t(heads) * k_tiles * 4;
    const void* p[4] = {idx, cnt, t_end, t_list};
    const size_t n[4] = {ib, cb, eb, ib};
    if (any_overlap(p, n, 4)) return SPARSE3D_ERR_ALIAS;
    return SPARSE3D_OK;
}

int validate_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, int dtype, int32_t heads, int32_t head_dim, int32_t tile,
                      const sparse3d_layout* qlay, const sparse3d_layout* klay, const int32_t* idx,
                      const int32_t* cnt, int32_t kmax, const int32_t* t_end, const int32_t* t_list,
                      const void* kbar, const void* vbar, float landmark_bias, float scale,
                      const float* dq, const float* dk, const float* dv, const float* delta,
                      const float* dkbar, const float* dvbar) {
    if (!out || !dout || !lse || !t_end || !dq || !dk || !dv || !delta) return SPARSE3D_ERR_NULL;
    if (kmax > 0 && !t_list) return SPARSE3D_ERR_NULL;
    const bool lm = kbar != nullptr;
    if (lm && (!dkbar || !dvbar)) return SPARSE3D_ERR_NULL;
    S3D_TRY(validate_attn(true, q, k, v, dtype, heads, head_dim, tile, qlay, klay, idx, cnt, kmax,
                          kbar, vbar, dq, SPARSE3D_F32, nullptr));
    if (dtype != SPARSE3D_BF16) return SPARSE3D_ERR_UNSUPPORTED;
    if (kmax > (lm ? kMaxBwdListLm : kMaxBwdList) || lay_tiles(*qlay) > kMaxTransposeQ)
        return SPARSE3D_ERR_UNSUPPORTED;
    S3D_TRY(check_logit_params(scale, lm ? landmark_bias : 0.f));
    const size_t qb = size_t(heads) * lay_rows(*qlay) * head_dim;     // elements
    const size_t kb = size_t(heads) * lay_rows(*klay) * head_dim;
    const size_t mb = lm ? size_t(heads) * lay_tiles(*klay) * head_dim : 0;
    const size_t lb = size_t(heads) * lay_rows(*qlay) * 4;
    const size_t ib = size_t(heads) * lay_tiles(*qlay) * kmax * 4;
    const size_t cb = size_t(heads) * lay_tiles(*qlay) * 4, eb = size_t(heads) * lay_tiles(*klay) * 4;
    // inputs first, then the outputs
    constexpr int NIN = 12, NP = 18;
    const void* p[NP] = {q,  k,  v,  out,  dout,  lse,   idx,   cnt,   t_end,  t_list,
                         kbar, vbar, dq, dk, dv, delta, lm ? dkbar : nullptr, lm ? dvbar : nullptr};
    const size_t n[NP] = {qb * 2, kb * 2, kb * 2, qb * 2, qb * 2, lb,     ib,     cb, eb,
                          ib,     mb * 2, mb * 2, qb * 4, kb * 4, kb * 4, lb, mb * 4, mb * 4};
    // every output against everything else; inputs may share memory (q may equal k)
    for (int i = NIN; i < NP; ++i)
        for (int j = 0; j < NP; ++j)
            if (j != i && overlaps(p[i], n[i], p[j], n[j])) return SPARSE3D_ERR_ALIAS;
    return SPARSE3D_OK;
}

int validate_cast(const float* src, int64_t n, int dtype, const void* dst) {
    if (n < 0) return SPARSE3D_ERR_SHAPE;
    S3D_TRY(check_dtype(dtype));
    if (n == 0) return SPARSE3D_OK;
    if (!src || !dst) return SPARSE3D_ERR_NULL;
    if (overlaps(dst, size_t(n) * dtype_bytes(sparse3d_dtype(dtype)), src, size_t(n) * 4))
        return SPARSE3D_ERR_ALIAS;
    return SPARSE3D_OK;
}

int subsample_layout(const sparse3d_layout* lay, int32_t grid_h, int32_t grid_w, int32_t window,
                     int32_t tile, sparse3d_layout* out) {
    if (!lay || !out) return SPARSE3D_ERR_NULL;
    S3D_TRY(check_layout(lay));
    if (grid_h < 1 || grid_w < 1 || window < 1 || tile < 1) return SPARSE3D_ERR_SHAPE;
    if (tile != kTile) return SPARSE3D_ERR_UNSUPPORTED;
    if (int64_t(lay->specials) + int64_t(grid_h) * grid_w != lay->tokens) return SPARSE3D_ERR_SHAPE;
    const int32_t kh = (grid_h + window - 1) / window, kw = (grid_w + window - 1) / window;
    const int32_t tokens = lay->specials + kh * kw;
    out->frames = lay->frames;
    out->tokens = tokens;
    out->stride = (tokens + tile - 1) / tile * tile;
    out->specials = lay->specials;
    return SPARSE3D_OK;
}

int validate_subsample(const void* k, const void* v, int dtype, int32_t heads, int32_t head_dim,
                       const sparse3d_layout* lay, int32_t grid_h, int32_t grid_w, int32_t window,
                       const void* k_out, const void* v_out, const sparse3d_layout* out_lay) {
    if (!k || !v || !k_out || !v_out || !out_lay) return SPARSE3D_ERR_NULL;
    S3D_TRY(check_dtype(dtype));
    S3D_TRY(check_heads_dims(heads, head_dim, kTile));
    sparse3d_layout want;
    S3D_TRY(subsample_layout(lay, grid_h, grid_w, window, kTile, &want));
    if (out_lay->frames != want.frames || out_lay->tokens != want.tokens ||
        out_lay->stride != want.stride || out_lay->specials != want.specials)
        return SPARSE3D_ERR_SHAPE;
    const size_t eb = dtype_bytes(sparse3d_dtype(dtype));
    const size_t ib = size_t(heads) * lay_rows(*lay) * head_dim * eb;
    const size_t ob = size_t(heads) * lay_rows(want) * head_dim * eb;
    if (overlaps(k_out, ob, k, ib) || overlaps(k_out, ob, v, ib) || overlaps(v_out, ob, k, ib) ||
        overlaps(v_out, ob, v, ib) || overlaps(k_out, ob, v_out, ob))
        return SPARSE3D_ERR_ALIAS;
    return SPARSE3D_OK;
}

}  // namespace s3d
