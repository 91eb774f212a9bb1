"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from dynamic_block_sparse_tile_amd import layer as LY
from dynamic_block_sparse_tile_amd import sparse3d as S
from dynamic_block_sparse_tile_amd import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}       # max |O_gpu - O_oracle| under the same selection
MARGIN = 1e-3                            # selections must match where the k/k+1 gap exceeds this


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def tdt(w):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def to_dev(x: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev(), dtype)


def margin_rows(ref_scores: np.ndarray, k: int) -> np.ndarray:
    """Boolean [H, Tq]: the oracle's k-th and (k+1)-th largest scores differ by > MARGIN relative."""
    H, Tq, Tk = ref_scores.shape
    if k <= 0 or k >= Tk:
        return np.ones((H, Tq), dtype=bool)
    a = np.empty((H, Tq))
    b = np.empty((H, Tq))
    for h in range(H):                  # the k-th and (k+1)-th largest by a partial sort
        part = np.partition(ref_scores[h], (Tk - k - 1, Tk - k), axis=1)
        a[h], b[h] = part[:, Tk - k], part[:, Tk - k - 1]
    with np.errstate(invalid="ignore"):
        den = np.maximum(np.abs(a), np.abs(b))
        rel = np.where(np.isfinite(a) & np.isfinite(b),
                       np.abs(a - b) / np.where(den > 0, den, 1.0),
                       np.where(a == b, 0.0, np.inf))
    return rel > MARGIN


def check_selection(g_scores, g_idx, g_cnt, ref_scores, k, tpf, anchor, rows=None):
    """(a) the GPU selection is exactly the oracle's selection rule applied to the GPU's own
    fp32 scores; (b) wherever the oracle's fp64 margin exceeds 1e-3 it equals the oracle's
    selection from its own scores.  ``rows``: optional list of (h, tq) to check."""
    H, Tq, Tk = g_scores.shape
    kmax = g_idx.shape[2]
    ok = margin_rows(ref_scores, k)
    pairs = rows if rows is not None else [(h, t) for h in range(H) for t in range(Tq)]
    n_margin = 0
    for (h, t) in pairs:
        own = oracle.select_tiles(g_scores[h, t].astype(np.float64), k, tpf, anchor)
        got = g_idx[h, t, :g_cnt[h, t]]
        assert g_cnt[h, t] == len(own) and np.array_equal(got, own), (h, t, got, own)
        assert np.all(g_idx[h, t, g_cnt[h, t]:] == -1)
        if ok[h, t]:
            n_margin += 1
            ref = oracle.select_tiles(ref_scores[h, t], k, tpf, anchor)
            assert np.array_equal(got, ref), ("margin row differs", h, t, got, ref)
    return n_margin, len(pairs)


def selection_mask(g_idx, g_cnt, Tk):
    """[H, Tq, Tk] membership of the GPU's lists, after checking their form: ascending,
    in range, -1 after the count."""
    H, Tq, kmax = g_idx.shape
    assert np.all((g_cnt >= 0) & (g_cnt <= kmax))
    live = np.arange(kmax)[None, None, :] < g_cnt[:, :, None]
    assert np.all(g_idx[~live] == -1)
    assert np.all((g_idx[live] >= 0) & (g_idx[live] < Tk))
    if kmax > 1:
        both = live[:, :, 1:]
        assert np.all(np.diff(g_idx, axis=2)[both] > 0)          # strictly ascending
    m = np.zeros((H, Tq, Tk), dtype=bool)
    h, t, e = np.nonzero(live)
    m[h, t, g_idx[h, t, e]] = True
    return m


def check_selection_all_rows(g_scores, g_idx, g_cnt, ref_scores, k, tpf, anchor):
    """``check_selection`` on every (head, query tile) row of a large case, through the
    oracle's whole-matrix form of the selection rule.  Returns (margin rows, rows)."""
    H, Tq, Tk = g_scores.shape
    got = selection_mask(g_idx, g_cnt, Tk)
    n_margin = 0
    for h in range(H):
        own = oracle.select_mask(g_scores[h:h + 1].astype(np.float64), k, tpf, anchor)[0]
        bad = np.nonzero(np.any(got[h] != own, axis=1))[0]
        assert bad.size == 0, ("GPU selection differs from the rule on its own scores", h, bad[:8])
        ok = margin_rows(ref_scores[h:h + 1], k)[0]
        ref = oracle.select_mask(ref_scores[h:h + 1], k, tpf, anchor)[0]
        bad = np.nonzero(ok & np.any(got[h] != ref, axis=1))[0]
        assert bad.size == 0, ("margin row differs from the oracle's selection", h, bad[:8])
        n_margin += int(ok.sum())
    return n_margin, H * Tq


def check_scores(g_qbar, g_kbar, g_scores, ref, atol_bar=2e-5, rtol_sc=2e-5):
    assert np.allclose(g_qbar, ref["qbar"], rtol=0, atol=atol_bar)
    assert np.allclose(g_kbar, ref["kbar"], rtol=0, atol=atol_bar)
    rs = ref["scores"]
    fin = np.isfinite(rs)
    assert np.array_equal(np.isfinite(g_scores), fin)
    assert np.all(g_scores[~fin] == -np.inf)
    err = np.abs(g_scores[fin] - rs[fin])
    lim = rtol_sc * (1.0 + np.abs(rs[fin]))
    assert np.all(err <= lim), float(np.max(err / lim))


def oracle_pool_scores(inp, qlay, klay, K=None, V=None, landmarks=False):
    """Oracle pool + scores (full), with optional subsampled K/V."""
    K = inp.k if K is None else K
    V = inp.v if V is None else V
    qbar, qc = oracle.tile_pool(inp.q, qlay, 64, "query")
    kbar, kc = oracle.tile_pool(K, klay, 64, "key")
    sc = oracle.tile_scores(qbar, qc, kbar, kc, 0.125)
    out = dict(qbar=qbar, qcount=qc, kbar=kbar, kcount=kc, scores=sc)
    if landmarks:
        out["vbar"], _ = oracle.tile_pool(V, klay, 64, "key")
    return out


def sample_tiles(H, Tq, n, seed=0):
    rng = np.random.default_rng(seed)
    pairs = {(int(rng.integers(H)), int(rng.integers(Tq))) for _ in range(n)}
    pairs |= {(0, 0), (H - 1, Tq - 1)}
    return sorted(pairs)


def compare_outputs(g_out, ref_O, pairs, tile=64, tol=2e-2, g_lse=None, ref_lse=None, lse_tol=None):
    worst = 0.0
    for (h, t) in pairs:
        r = slice(t * tile, (t + 1) * tile)
        e = float(np.max(np.abs(g_out[h, r].astype(np.float64) - ref_O[h, r])))
        worst = max(worst, e)
        assert e <= tol, (h, t, e)
        if g_lse is not None:
            a, b = g_lse[h, r].astype(np.float64), ref_lse[h, r]
            fin = np.isfinite(b)
            assert np.array_equal(np.isfinite(a), fin)
            assert np.all(np.abs(a[fin] - b[fin]) <= lse_tol), (h, t)
    return worst
