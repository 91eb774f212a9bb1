"""The sparse global-attention layer composed from the C-ABI calls, plus host logic.

``sparse_global_attention`` runs the three steps of one layer (pooled tile
scores -> per-row top-k united with the anchor frame -> exact attention over the
selected tiles, optionally with landmark summaries), each step one library call
on the current stream.  The rest is host-side bookkeeping: the number of special
pseudo-tiles, the measured sparsity, calibrating k to a target sparsity, and
the FLOP count of the selected tile pairs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Optional

import torch

from . import sparse3d as S

TILE = S.TILE


def special_tiles(klay) -> int:
    """Ts: 64-row pseudo-tiles holding the special tokens of every frame."""
    frames, _, _, specials = klay
    return (specials * frames + TILE - 1) // TILE


def tiles_per_frame(lay) -> int:
    return lay[2] // TILE


def measured_sparsity(total_cnt: int, rows: int, ts: int, tk: int) -> float:
    """1 - (attended key tiles per query tile) / Tk, averaged over (head, query tile) rows.

    Attended tiles are the special pseudo-tiles plus the selected tiles.
    """
    return 1.0 - (ts + total_cnt / rows) / tk


def calibrate_k(count_fn: Callable[[int], int], rows: int, ts: int, tk: int,
                target: float) -> int:
    """The k whose measured sparsity is closest to ``target`` (ties to higher sparsity).

    ``count_fn(k)`` returns the total selection count over all rows for that k; it
    is monotone non-decreasing in k, so a binary search finds the crossing.
    """
    def sp(k):
        return measured_sparsity(count_fn(k), rows, ts, tk)

    lo, hi = 0, tk                     # sp(lo) >= sp(hi)
    if sp(lo) <= target:
        return lo
    if sp(hi) >= target:
        return hi
    while hi - lo > 1:                 # invariant: sp(lo) > target > sp(hi)
        mid = (lo + hi) // 2
        if sp(mid) > target:
            lo = mid
        else:
            hi = mid
    return lo if abs(sp(lo) - target) <= abs(sp(hi) - target) else hi


def pair_flops(tile: int = TILE, head_dim: int = 64) -> int:
    """FLOPs of one (query tile, key tile) pair: QK^T plus PV, 2 * 2 * B * B * d."""
    return 4 * tile * tile * head_dim


def selected_flops(total_cnt: int, rows: int, ts: int, landmarks: int = 0,
                   tile: int = TILE, head_dim: int = 64) -> int:
    """Algorithmic FLOPs of the sparse attention: every (query tile, attended tile)
    pair, plus 4*d per (query row, landmark) when landmarks are on."""
    return (rows * ts + total_cnt) * pair_flops(tile, head_dim) + landmarks * tile * 4 * head_dim


def valid_pair_flops(idx, cnt, qlay, klay, tile: int = TILE, head_dim: int = 64) -> int:
    """FLOPs of the attended pairs counted over real rows only: valid query rows (in-frame
    position below N) times member keys (patch tokens of a selected tile, special tokens of
    the special pseudo-tiles), 4*d per (query, key).  ``idx``/``cnt`` are host arrays
    [heads, Tq, kmax] / [heads, Tq]."""
    import numpy as np
    S, N, P, nsp = klay
    tpf = P // tile
    j0 = (np.arange(S * tpf) % tpf) * tile
    members = np.clip(np.minimum(tile, N - j0) - np.maximum(0, nsp - j0), 0, None)
    qS, qN, qP, _ = qlay
    qj0 = (np.arange(qS * (qP // tile)) % (qP // tile)) * tile
    vq = np.clip(np.minimum(tile, qN - qj0), 0, None)
    kmax = idx.shape[2]
    live = np.arange(kmax)[None, None, :] < cnt[:, :, None]
    safe = np.where(live, idx, 0)
    keys = (members[safe] * live).sum(axis=2) + nsp * S          # members per row, specials included
    return int((keys * vq[None, :]).sum()) * 4 * head_dim


@dataclass
class LayerResult:
    out: torch.Tensor
    lse: Optional[torch.Tensor]
    qbar: torch.Tensor
    kbar: torch.Tensor
    vbar: Optional[torch.Tensor]
    scores: torch.Tensor
    idx: torch.Tensor
    cnt: torch.Tensor


def sparse_global_attention(q, k, v, qlay, klay=None, *, top_k: int, anchor_frame: int = 0,
                            landmarks: bool = False, scale: Optional[float] = None,
                            landmark_bias: float = S.LN64, out_dtype=None,
                            return_lse: bool = False) -> LayerResult:
    """One dynamic tile-sparse global-attention layer (three library calls)."""
    klay = qlay if klay is None else klay
    scale = 1.0 / math.sqrt(q.shape[2]) if scale is None else scale
    # with landmarks the pooling pass also writes the means in the operand dtype (the
    # precision the attention reads them in)
    sc = S.sparse3d_tile_scores(q, k, qlay, klay, v=v if landmarks else None, scale=scale,
                                operand_means=landmarks)
    qbar, kbar, vbar, scores = sc[:4]
    km, vm = sc[4:] if landmarks else (None, None)
    idx, cnt = S.sparse3d_select_topk(scores, top_k, tiles_per_frame(klay), anchor_frame)
    res = S.sparse3d_sparse_attn_fwd(q, k, v, qlay, klay, idx, cnt,
                                     kbar=km if landmarks else None, vbar=vm if landmarks else None,
                                     landmark_bias=landmark_bias, scale=scale,
                                     out_dtype=out_dtype, return_lse=return_lse)
    out, lse = res if return_lse else (res, None)
    return LayerResult(out, lse, qbar, kbar, vbar, scores, idx, cnt)


def device_count_fn(scores: torch.Tensor, tpf: int, anchor_frame: int) -> Callable[[int], int]:
    """count_fn for ``calibrate_k`` that runs the library's top-k on the device."""
    def f(k: int) -> int:
        _, cnt = S.sparse3d_select_topk(scores, k, tpf, anchor_frame)
        return int(cnt.sum().item())
    return f
