"""fp64 CPU oracle for dynamic tile-sparse global (cross-frame) attention.

TEST INFRASTRUCTURE.  Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The library's
product path never does; it shares no code, tables or helpers with the HIP
kernels, and imports nothing from the package.

Plain, slow, obviously correct numpy float64.  Every input array is upcast to
float64 before any arithmetic; the values themselves are whatever the caller
hands in (the seeded generator already rounds them to the workload dtype).

What is computed, and the passages it follows
---------------------------------------------
* Global attention over all S*N tokens of S views is the quadratic cost these
  methods attack (SAF3R abstract; Zebra3D abstract; EPFL "(Full) Attention is
  More Than You Need", figure "Full vs sparse global attention").  ``dense_attend``
  is that operation: exact softmax attention of every valid query over every
  valid key.
* Zebra3D (abstract) replaces it in sensitive stages by tile-sparse attention
  and keeps "landmark summaries" of the tiles that were not selected; SAF3R
  (abstract) selects the most promising interactions per input.  The steps
  below are the plainest reading of that family:
    1. ``tile_pool``: mean of the rows of each 64-row tile (query tiles over
       their valid rows, key tiles over their member rows);
    2. ``tile_scores``: sigma[tq, tk] = scale * qbar[tq] . kbar[tk], -inf when a
       tile has no rows to average;
    3. ``select_tiles``: the k key tiles with the largest sigma (ties to the lower
       tile index), united with every tile of the anchor frame, in ascending
       tile order;
    4. ``sparse_attend``: exact softmax over the special (camera/register)
       tokens of every frame plus the member keys of the selected tiles; with
       landmarks on, each unselected non-empty tile adds one logit
       scale * q . kbar[t] + ln 64 carrying the value vbar[t].
* AVGGT technical summary, section 2B.2 (subsampled global attention): keys and
  values are thinned on the 2-D patch grid to one token per s_h x s_w window
  while every query and every special token is kept.  ``subsample_keys`` keeps
  the top-left patch of every window.
* The same section completes the subsample with two terms: every token keeps
  its own key (the diagonal of the attention matrix) when the subsample dropped
  it, and the dropped columns are stood in for by a single mean key/value pair.
  ``discarded_mean`` is that pair (means over the dropped patch rows of every
  frame); the attention calls take both terms through ``sga``.  Reading: the
  mean pair stands for all |D| dropped columns at once, so its logit carries
  ln |D| (``sga_mean_bias``), exactly as a landmark carries ln 64 for its tile.
* Zebra3D (abstract) also trains after conversion, and the EPFL page trains
  with sparse attention; both need the gradient of the sparse layer.
  ``sparse_attend_bwd`` is the exact gradient of ``sparse_attend``'s output with
  the selection held fixed (top-k is piecewise constant, so no gradient flows
  through the scores): with P the softmax weights of a row, dP = dO V^T,
  D = rowsum(dO * O), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q,
  dV = P^T dO, summed over every query that attends a key.
* AVGGT technical summary, section 2B.1: the early global layers, which exchange
  no information between views, become attention within each frame.
  ``frame_attend`` is that operation: every valid query over the valid keys of
  its own frame only.
* SAF3R (abstract) finds attention patterns heterogeneous across heads; a
  per-head budget k_h is the knob that follows it (``select_topk`` accepts one
  k per head).

Readings adopted where the pages leave a step open
---------------------------------------------------
Row r lies in frame r // stride at in-frame position j = r % stride.  It is a
valid query iff j < tokens; a member key of its tile iff specials <= j < tokens;
a special key iff j < specials.  Specials are attended at token granularity by
every query and never belong to a tile (so no key is counted twice), pad rows
are never read as data, the landmark bias is ln 64 for every unselected
non-empty tile, rows that are not valid queries get O = 0 and lse = 0, and a
valid query whose key set is empty gets O = 0 and lse = -inf.

Parity: every function here is pinned by the CPU test suite against closed
forms, invariants, library routines or brute force; none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import NamedTuple, Optional, Sequence, Tuple

import numpy as np

LN64 = math.log(64.0)


class Layout(NamedTuple):
    frames: int     # S
    tokens: int     # valid tokens per frame
    stride: int     # padded rows per frame
    specials: int   # leading special tokens per frame

    @property
    def rows(self) -> int:
        return self.frames * self.stride


# ----------------------------------------------------------------------------- row kinds
def _inframe(lay: Layout) -> np.ndarray:
    return np.arange(lay.rows) % lay.stride


def query_rows(lay: Layout) -> np.ndarray:
    """Boolean mask of valid query rows (special and patch tokens, not pad)."""
    return _inframe(lay) < lay.tokens


def member_rows(lay: Layout) -> np.ndarray:
    """Boolean mask of key rows that belong to their tile (patch tokens only)."""
    j = _inframe(lay)
    return (j >= lay.specials) & (j < lay.tokens)


def special_rows(lay: Layout) -> np.ndarray:
    """Boolean mask of special (camera/register) key rows."""
    j = _inframe(lay)
    return j < min(lay.specials, lay.tokens)


def key_rows_dense(lay: Layout) -> np.ndarray:
    """Boolean mask of every valid key row, specials in place (dense attention)."""
    return _inframe(lay) < lay.tokens


# ----------------------------------------------------------------------------- step 1: pool
def tile_pool(X: np.ndarray, lay: Layout, tile: int, rows: str) -> Tuple[np.ndarray, np.ndarray]:
    """Mean of each tile's rows.  ``rows`` is "query" (valid rows) or "key" (member rows).

    X: [H, S*stride, d].  Returns (mean [H, T, d] float64, count [T] int64); a tile
    with no rows gets mean 0 and count 0.
    """
    H, L, d = X.shape
    assert L == lay.rows and lay.stride % tile == 0
    mask = query_rows(lay) if rows == "query" else member_rows(lay)
    T = L // tile
    m = mask.reshape(T, tile)
    count = m.sum(axis=1)
    mean = np.zeros((H, T, d))
    for h in range(H):
        Xh = X[h].astype(np.float64).reshape(T, tile, d)
        Xh = np.where(m[:, :, None], Xh, 0.0)          # pad may hold NaN: select, never multiply
        s = Xh.sum(axis=1)
        nz = count > 0
        mean[h, nz] = s[nz] / count[nz, None]
    return mean, count


# ----------------------------------------------------------------------------- step 2: score
def tile_scores(qbar: np.ndarray, qcount: np.ndarray, kbar: np.ndarray, kcount: np.ndarray,
                scale: float) -> np.ndarray:
    """sigma[h, tq, tk] = scale * qbar[h, tq] . kbar[h, tk]; -inf if either tile is empty."""
    sig = scale * np.matmul(qbar, np.swapaxes(kbar, 1, 2))
    sig[:, qcount == 0, :] = -np.inf
    sig[:, :, kcount == 0] = -np.inf
    return sig


# ----------------------------------------------------------------------------- step 3: select
def select_tiles(row: np.ndarray, k: int, tiles_per_frame: int, anchor: int) -> np.ndarray:
    """Selected key tiles of one query tile, ascending.

    The k largest scores (larger first, equal scores in ascending tile order),
    united with all tiles of frame ``anchor`` (none when anchor < 0).
    """
    Tk = row.shape[0]
    order = np.lexsort((np.arange(Tk), -row))       # primary: -sigma ascending; then index
    top = order[: min(max(k, 0), Tk)]
    forced = (np.arange(anchor * tiles_per_frame, (anchor + 1) * tiles_per_frame)
              if anchor >= 0 else np.empty(0, dtype=np.int64))
    return np.union1d(top, forced).astype(np.int64)


def kmax_for(tk: int, k: int, tiles_per_frame: int, anchor: int) -> int:
    """Largest possible selection size: min(Tk, k + (anchor tiles))."""
    return min(tk, max(k, 0) + (tiles_per_frame if anchor >= 0 else 0))


def select_topk(scores: np.ndarray, k, tiles_per_frame: int, anchor: int,
                kmax: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """All rows of ``select_tiles``: idx [H, Tq, kmax] (ascending, -1 padded), cnt [H, Tq].

    ``k`` is one budget for every head, or a sequence of H budgets (head h keeps k[h]).
    """
    H, Tq, Tk = scores.shape
    ks = [int(k)] * H if np.ndim(k) == 0 else [int(x) for x in k]
    assert len(ks) == H
    if kmax is None:
        kmax = kmax_for(Tk, max(ks), tiles_per_frame, anchor)
    idx = np.full((H, Tq, kmax), -1, dtype=np.int32)
    cnt = np.zeros((H, Tq), dtype=np.int32)
    for h in range(H):
        for t in range(Tq):
            sel = select_tiles(scores[h, t], ks[h], tiles_per_frame, anchor)
            cnt[h, t] = len(sel)
            idx[h, t, : len(sel)] = sel
    return idx, cnt


def select_mask(scores: np.ndarray, k, tiles_per_frame: int, anchor: int) -> np.ndarray:
    """``select_tiles`` of every row at once, as a boolean [H, Tq, Tk] membership mask.

    The same rule written by threshold: with T the k-th largest score of the row, a tile
    is among the k best iff its score exceeds T, or equals T and fewer than k tiles lie
    above T plus the equal ones of lower index; the anchor frame's tiles are added.  Meant
    for large score matrices (one partial sort per head instead of one full sort per row).
    ``k`` is one budget or one per head.
    """
    H, Tq, Tk = scores.shape
    ks = [int(k)] * H if np.ndim(k) == 0 else [int(x) for x in k]
    out = np.zeros((H, Tq, Tk), dtype=bool)
    for h in range(H):
        kh = min(max(ks[h], 0), Tk)
        row = scores[h].astype(np.float64)
        if kh == Tk:
            out[h] = True
        elif kh > 0:
            T = np.partition(row, Tk - kh, axis=1)[:, Tk - kh]          # the k-th largest value
            above = row > T[:, None]
            tie = row == T[:, None]
            room = kh - above.sum(axis=1)                               # how many ties to take
            out[h] = above | (tie & (np.cumsum(tie, axis=1) <= room[:, None]))
        if anchor >= 0:
            out[h, :, anchor * tiles_per_frame:(anchor + 1) * tiles_per_frame] = True
    return out


# ----------------------------------------------------------------------------- step 4: attend
def _softmax_rows(logits: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax-weighted average of ``values`` per row of ``logits``; also log-sum-exp.

    An empty key set (no specials, nothing selected, no landmarks) gives O = 0 and
    lse = -inf: the softmax has no terms, so the weighted sum is empty.
    """
    if logits.shape[1] == 0:
        return np.zeros((logits.shape[0], values.shape[1])), np.full(logits.shape[0], -np.inf)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    den = e.sum(axis=1, keepdims=True)
    out = (e @ values) / den
    return out, (m + np.log(den))[:, 0]


def sparse_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, qlay: Layout, klay: Layout,
                  tile: int, idx: np.ndarray, cnt: np.ndarray, scale: float, *,
                  kbar: Optional[np.ndarray] = None, vbar: Optional[np.ndarray] = None,
                  kcount: Optional[np.ndarray] = None, landmark_bias: float = LN64,
                  query_tiles: Optional[Sequence[int]] = None,
                  heads: Optional[Sequence[int]] = None,
                  sga: Optional[dict] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of each query tile over specials + its selected tiles (+ landmarks).

    Q: [H, Sq*Pq, d], K/V: [H, Sk*Pk, d]; idx/cnt as from ``select_topk``.
    Landmarks are on when ``kbar`` is given (then ``vbar`` and ``kcount`` too).
    Only the listed ``query_tiles`` / ``heads`` are computed; the other rows of the
    returned O [H, Lq, d] and lse [H, Lq] are 0.  ``sga`` adds the subsample completion
    (own key of dropped positions from k_full/v_full, mean pair kmean/vmean + mean_bias;
    keys: grid, window, k_full, v_full, kmean, vmean, mean_bias).
    """
    H, Lq, d = Q.shape
    Tk = klay.rows // tile
    qv = query_rows(qlay)
    mem = member_rows(klay).reshape(Tk, tile)
    spec = np.nonzero(special_rows(klay))[0]
    O = np.zeros((H, Lq, d))
    lse = np.zeros((H, Lq))
    tiles = range(qlay.rows // tile) if query_tiles is None else query_tiles
    for h in (range(H) if heads is None else heads):
        for tq in tiles:
            rows_q = tq * tile + np.nonzero(qv[tq * tile:(tq + 1) * tile])[0]
            if rows_q.size == 0:
                continue
            sel = idx[h, tq, : cnt[h, tq]]
            keys = [spec] + [t * tile + np.nonzero(mem[t])[0] for t in sel]
            J = np.concatenate(keys).astype(np.int64)
            q = Q[h, rows_q].astype(np.float64)
            logits = scale * (q @ K[h, J].astype(np.float64).T)
            values = V[h, J].astype(np.float64)
            if kbar is not None:
                chosen = np.zeros(Tk, dtype=bool)
                chosen[sel] = True
                lm = np.nonzero(~chosen & (kcount > 0))[0]
                logits = np.concatenate([logits, scale * (q @ kbar[h, lm].T) + landmark_bias], axis=1)
                values = np.concatenate([values, vbar[h, lm]], axis=0)
            if sga is not None:
                o, l = _softmax_rows_extra(logits, values, *_sga_extra(h, rows_q, q, qlay, scale, sga))
            else:
                o, l = _softmax_rows(logits, values)
            O[h, rows_q] = o
            lse[h, rows_q] = l
    return O, lse


def sparse_attend_bwd(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, qlay: Layout,
                      klay: Layout, tile: int, idx: np.ndarray, cnt: np.ndarray,
                      scale: float, query_tiles: Optional[Sequence[int]] = None,
                      heads: Optional[Sequence[int]] = None, *,
                      kbar: Optional[np.ndarray] = None, vbar: Optional[np.ndarray] = None,
                      kcount: Optional[np.ndarray] = None, landmark_bias: float = LN64,
                      means: bool = False, magnitudes: bool = False):
    """Gradients of ``sparse_attend`` w.r.t. Q, K, V for the output cotangent dO, selection
    fixed: (dQ [H, Lq, d], dK [H, Lk, d], dV [H, Lk, d], D [H, Lq]) in fp64,
    D = rowsum(dO * O).  Rows that are not valid queries contribute nothing and get
    dQ = 0, D = 0; key rows nobody attends (pad, unselected tiles) get dK = dV = 0.
    With ``query_tiles`` / ``heads`` only those query tiles contribute (dK/dV of a key tile
    are then complete when the list holds every query tile that selected it).

    Landmarks (``kbar``/``vbar``/``kcount`` as in ``sparse_attend``): every unselected
    non-empty tile t is one more key of the row, kbar[t] with logit bias ``landmark_bias``
    and value vbar[t].  Its gradients dkbar[t] = scale sum_i dS_it q_i and
    dvbar[t] = sum_i P_it dO_i flow through the mean pool (kbar[t] is the mean of K over
    the member rows M(t)) into every member row: dK[r] += dkbar[t] / |M(t)|, likewise dV.
    ``means``: also return dkbar, dvbar [H, Tk, d] (zero without landmarks).

    ``magnitudes``: also return a dict of absolute-value sums that bound how rounding of the
    softmax weights and of dS propagates (same shapes as the gradients):
      M_ij = P_ij (|dP_ij - D_i| + A_D_i),  A_D_i = sum_c |dO_ic| (|O_ic| + sum_j P_ij |V_jc|),
      dQ: scale sum_j M_ij |K_j|;  dK: scale sum_i M_ij |Q_i|;  dV: sum_i P_ij |dO_i|;  D: A_D
    (landmark columns chained to member rows like the gradients, and, with landmarks, kept
    per mean as "dkbar" / "dvbar")."""
    H, Lq, d = Q.shape
    Tk = klay.rows // tile
    qv = query_rows(qlay)
    mem = member_rows(klay).reshape(Tk, tile)
    spec = np.nonzero(special_rows(klay))[0]
    dQ = np.zeros((H, Lq, d))
    dK = np.zeros((H, K.shape[1], d))
    dV = np.zeros((H, K.shape[1], d))
    D = np.zeros((H, Lq))
    dkb = np.zeros((H, Tk, d))
    dvb = np.zeros((H, Tk, d))
    if magnitudes:
        mag = {n: np.zeros_like(x) for n, x in (("dQ", dQ), ("dK", dK), ("dV", dV), ("D", D))}
        mkb, mvb = np.zeros((H, Tk, d)), np.zeros((H, Tk, d))
    for h in (range(H) if heads is None else heads):
        for tq in (range(qlay.rows // tile) if query_tiles is None else query_tiles):
            rows_q = tq * tile + np.nonzero(qv[tq * tile:(tq + 1) * tile])[0]
            if rows_q.size == 0:
                continue
            sel = idx[h, tq, : cnt[h, tq]]
            J = np.concatenate([spec] + [t * tile + np.nonzero(mem[t])[0] for t in sel]).astype(np.int64)
            kk = K[h, J].astype(np.float64)
            vv = V[h, J].astype(np.float64)
            bias = np.zeros(J.size)
            lm = np.empty(0, dtype=np.int64)
            if kbar is not None:
                chosen = np.zeros(Tk, dtype=bool)
                chosen[sel] = True
                lm = np.nonzero(~chosen & (kcount > 0))[0]
                kk = np.concatenate([kk, kbar[h, lm]])
                vv = np.concatenate([vv, vbar[h, lm]])
                bias = np.concatenate([bias, np.full(lm.size, landmark_bias)])
            if kk.shape[0] == 0:
                continue
            q = Q[h, rows_q].astype(np.float64)
            g = dO[h, rows_q].astype(np.float64)
            s = scale * (q @ kk.T) + bias
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = p @ vv
            dp = g @ vv.T
            Di = np.sum(g * o, axis=1)
            ds = p * (dp - Di[:, None])
            dQ[h, rows_q] = scale * (ds @ kk)
            gk, gv = scale * (ds.T @ q), p.T @ g          # per attended key, then per landmark
            np.add.at(dK[h], J, gk[:J.size])
            np.add.at(dV[h], J, gv[:J.size])
            dkb[h, lm] += gk[J.size:]
            dvb[h, lm] += gv[J.size:]
            D[h, rows_q] = Di
            if magnitudes:
                AD = np.sum(np.abs(g) * (np.abs(o) + p @ np.abs(vv)), axis=1)
                M = p * (np.abs(dp - Di[:, None]) + AD[:, None])
                mag["dQ"][h, rows_q] = scale * (M @ np.abs(kk))
                ak, av = scale * (M.T @ np.abs(q)), p.T @ np.abs(g)
                np.add.at(mag["dK"][h], J, ak[:J.size])
                np.add.at(mag["dV"][h], J, av[:J.size])
                mkb[h, lm] += ak[J.size:]
                mvb[h, lm] += av[J.size:]
                mag["D"][h, rows_q] = AD
    if kbar is not None:
        # the mean pool: each member row of tile t receives 1/|M(t)| of the mean's gradient
        # (heads that were not processed have no mean gradients)
        rows_t = [t * tile + np.nonzero(mem[t])[0] for t in range(Tk)]
        for h in (range(H) if heads is None else heads):
            for t in range(Tk):
                if kcount[t] > 0:
                    dK[h, rows_t[t]] += dkb[h, t] / kcount[t]
                    dV[h, rows_t[t]] += dvb[h, t] / kcount[t]
                    if magnitudes:
                        mag["dK"][h, rows_t[t]] += mkb[h, t] / kcount[t]
                        mag["dV"][h, rows_t[t]] += mvb[h, t] / kcount[t]
    res = (dQ, dK, dV, D)
    if means:
        res = res + (dkb, dvb)
    if magnitudes:
        mag["dkbar"], mag["dvbar"] = mkb, mvb
        res = res + (mag,)
    return res


def selection_transpose(idx: np.ndarray, cnt: np.ndarray, k_tiles: int) -> list:
    """For each head and key tile, the ascending list of query tiles that selected it."""
    H, Tq, _ = idx.shape
    out = [[[] for _ in range(k_tiles)] for _ in range(H)]
    for h in range(H):
        for tq in range(Tq):
            for t in idx[h, tq, : cnt[h, tq]]:
                out[h][int(t)].append(tq)
    return out


def dense_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, qlay: Layout, klay: Layout,
                 scale: float, heads: Optional[Sequence[int]] = None,
                 query_rows_subset: Optional[np.ndarray] = None,
                 chunk: int = 2048, sga: Optional[dict] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of every valid query over every valid key (specials in place);
    ``sga`` as in ``sparse_attend``."""
    H, Lq, d = Q.shape
    J = np.nonzero(key_rows_dense(klay))[0]
    rows = np.nonzero(query_rows(qlay))[0]
    if query_rows_subset is not None:
        rows = np.intersect1d(rows, query_rows_subset)
    O = np.zeros((H, Lq, d))
    lse = np.zeros((H, Lq))
    for h in (range(H) if heads is None else heads):
        Kh = K[h, J].astype(np.float64)
        Vh = V[h, J].astype(np.float64)
        for c in range(0, rows.size, chunk):
            r = rows[c:c + chunk]
            q = Q[h, r].astype(np.float64)
            if sga is not None:
                o, l = _softmax_rows_extra(scale * (q @ Kh.T), Vh, *_sga_extra(h, r, q, qlay, scale, sga))
            else:
                o, l = _softmax_rows(scale * (q @ Kh.T), Vh)
            O[h, r] = o
            lse[h, r] = l
    return O, lse


def frame_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, qlay: Layout, klay: Layout,
                 scale: float, heads: Optional[Sequence[int]] = None,
                 frames: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of every valid query over the valid keys (specials in
    place) of its own frame; no key of another frame takes part."""
    assert qlay.frames == klay.frames
    H, Lq, d = Q.shape
    O = np.zeros((H, Lq, d))
    lse = np.zeros((H, Lq))
    for h in (range(H) if heads is None else heads):
        for s in (range(qlay.frames) if frames is None else frames):
            r = s * qlay.stride + np.arange(qlay.tokens)
            J = s * klay.stride + np.arange(klay.tokens)
            o, l = _softmax_rows(scale * (Q[h, r].astype(np.float64) @ K[h, J].astype(np.float64).T),
                                 V[h, J].astype(np.float64))
            O[h, r] = o
            lse[h, r] = l
    return O, lse


# ----------------------------------------------------------------------------- K/V subsample
def subsample_positions(specials: int, grid: Tuple[int, int], window: int) -> np.ndarray:
    """In-frame positions kept by the grid subsample: all specials, then the top-left
    patch of every window x window window of the gh x gw patch grid, row-major."""
    gh, gw = grid
    kept = [specials + y * gw + x for y in range(0, gh, window) for x in range(0, gw, window)]
    return np.concatenate([np.arange(specials), np.array(kept, dtype=np.int64)])


def subsample_keys(K: np.ndarray, V: np.ndarray, lay: Layout, grid: Tuple[int, int],
                   window: int, tile: int) -> Tuple[np.ndarray, np.ndarray, Layout]:
    """Keys/values thinned on the patch grid; queries are untouched by this step."""
    assert lay.tokens == lay.specials + grid[0] * grid[1]
    pos = subsample_positions(lay.specials, grid, window)
    n2 = pos.size
    p2 = -(-n2 // tile) * tile
    lay2 = Layout(lay.frames, n2, p2, lay.specials)
    H, _, d = K.shape
    K2 = np.zeros((H, lay.frames * p2, d), dtype=K.dtype)
    V2 = np.zeros((H, lay.frames * p2, d), dtype=V.dtype)
    for s in range(lay.frames):
        K2[:, s * p2: s * p2 + n2] = K[:, s * lay.stride + pos]
        V2[:, s * p2: s * p2 + n2] = V[:, s * lay.stride + pos]
    return K2, V2, lay2


def discarded_positions(specials: int, grid: Tuple[int, int], window: int) -> np.ndarray:
    """In-frame positions of the patches the grid subsample drops, ascending."""
    gh, gw = grid
    return np.array([specials + y * gw + x for y in range(gh) for x in range(gw)
                     if y % window or x % window], dtype=np.int64)


def discarded_mean(K: np.ndarray, V: np.ndarray, lay: Layout, grid: Tuple[int, int],
                   window: int) -> Tuple[np.ndarray, np.ndarray, int]:
    """Mean key and mean value over every dropped patch row of every frame, per head:
    (kmean [H, d], vmean [H, d], |D|).  With nothing dropped the means are 0 and |D| = 0."""
    pos = discarded_positions(lay.specials, grid, window)
    rows = (np.arange(lay.frames)[:, None] * lay.stride + pos[None, :]).ravel()
    H, _, d = K.shape
    if rows.size == 0:
        return np.zeros((H, d)), np.zeros((H, d)), 0
    return (K[:, rows].astype(np.float64).mean(axis=1), V[:, rows].astype(np.float64).mean(axis=1),
            int(rows.size))


def sga_mean_bias(count: int) -> float:
    """Logit offset of the mean pair: it stands for all `count` dropped columns."""
    return math.log(count)


def _sga_extra(h: int, rows_q: np.ndarray, q: np.ndarray, qlay: Layout, scale: float, sga: dict):
    """Per-row extra logits and values of the subsample completion: the row's own key when
    the subsample dropped its position (-inf otherwise), and the mean pair."""
    n, d = q.shape
    dl = np.full(n, -np.inf)
    dv = np.zeros((n, d))
    if sga.get("k_full") is not None:
        drop = np.zeros(qlay.stride, dtype=bool)
        drop[discarded_positions(qlay.specials, sga["grid"], sga["window"])] = True
        own = drop[rows_q % qlay.stride]
        kf = sga["k_full"][h, rows_q].astype(np.float64)
        dl = np.where(own, scale * np.einsum("nd,nd->n", q, np.nan_to_num(kf)), -np.inf)
        dv = np.where(own[:, None], np.nan_to_num(sga["v_full"][h, rows_q].astype(np.float64)), 0.0)
    ml = np.full(n, -np.inf)
    mv = np.zeros(d)
    if sga.get("kmean") is not None:
        ml = scale * (q @ sga["kmean"][h]) + sga["mean_bias"]
        mv = sga["vmean"][h]
    return dl, dv, ml, mv


def _softmax_rows_extra(logits, values, dl, dv, ml, mv):
    """``_softmax_rows`` over the shared keys plus, per row, one own key (logit dl, value
    dv) and the mean pair (logit ml, value mv); -inf logits take no part."""
    n = dl.shape[0]
    m = np.maximum(np.maximum(dl, ml), logits.max(axis=1) if logits.shape[1] else -np.inf)
    out = np.zeros((n, dv.shape[1]))
    lse = np.full(n, -np.inf)
    live = np.isfinite(m)
    if not np.any(live):
        return out, lse
    mm = m[live][:, None]
    e = np.exp(logits[live] - mm)
    ed = np.exp(dl[live] - m[live])
    em = np.exp(ml[live] - m[live])
    den = e.sum(axis=1) + ed + em
    out[live] = (e @ values + ed[:, None] * dv[live] + em[:, None] * mv[None, :]) / den[:, None]
    lse[live] = m[live] + np.log(den)
    return out, lse


# ----------------------------------------------------------------------------- the whole layer
def layer(Q, K, V, qlay: Layout, klay: Layout, tile: int, k: int, anchor: int,
          scale: Optional[float] = None, landmarks: bool = False,
          query_tiles=None, heads=None):
    """pool -> score -> select -> attend (+ landmarks).  Returns a dict of every stage."""
    d = Q.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qbar, qcount = tile_pool(Q, qlay, tile, "query")
    kbar, kcount = tile_pool(K, klay, tile, "key")
    sig = tile_scores(qbar, qcount, kbar, kcount, scale)
    idx, cnt = select_topk(sig, k, klay.stride // tile, anchor)
    kw = {}
    if landmarks:
        vbar, _ = tile_pool(V, klay, tile, "key")
        kw = dict(kbar=kbar, vbar=vbar, kcount=kcount)
    O, lse = sparse_attend(Q, K, V, qlay, klay, tile, idx, cnt, scale,
                           query_tiles=query_tiles, heads=heads, **kw)
    out = dict(qbar=qbar, qcount=qcount, kbar=kbar, kcount=kcount, scores=sig,
               idx=idx, cnt=cnt, O=O, lse=lse)
    if landmarks:
        out["vbar"] = kw["vbar"]
    return out
