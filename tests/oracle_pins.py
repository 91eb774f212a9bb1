"""Pins of the fp64 oracle against things other than itself.

Each ``pin_*`` takes an oracle module and raises AssertionError when that
module disagrees with a closed form, an invariant, a library routine or brute
force.  ``test_oracle.py`` runs them on the real oracle; ``test_oracle_mutants.py``
runs them on copies of the oracle with planted mistakes and requires that
every mistake is caught by at least one pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import scipy.special
import torch

from dynamic_block_sparse_tile_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_tiles.json")


def _lay(o, S, N, P, nsp):
    return o.Layout(S, N, P, nsp)


def _rand_inputs(S, N, P, nsp, H=2, d=8, seed=0, pad=np.nan):
    rng = np.random.default_rng(seed)
    L = S * P
    Q = rng.standard_normal((H, L, d))
    K = rng.standard_normal((H, L, d))
    V = rng.standard_normal((H, L, d))
    j = np.arange(L) % P
    for X in (Q, K, V):
        X[:, j >= N] = pad
    return Q, K, V


# --------------------------------------------------------------------------- pool + score
def pin_block_mean_identity(o):
    """sigma[tq, tk] is the mean of the dense logit block over valid queries x member keys.

    By bilinearity mean_{i,j} s*q_i.k_j = s*mean(q).mean(k); the block means are taken
    here from a separately computed dense logit matrix with row sets written out by
    position (valid query: in-frame < N; member key: nsp <= in-frame < N).
    """
    for (S, N, P, nsp, tile) in [(2, 256, 256, 0, 64), (3, 37, 48, 5, 16), (2, 10, 32, 3, 8),
                                 (2, 5, 16, 2, 8)]:
        Q, K, _ = _rand_inputs(S, N, P, nsp, seed=S * 100 + N)
        lay = _lay(o, S, N, P, nsp)
        scale = 0.3
        qbar, qc = o.tile_pool(Q, lay, tile, "query")
        kbar, kc = o.tile_pool(K, lay, tile, "key")
        sig = o.tile_scores(qbar, qc, kbar, kc, scale)
        T = S * P // tile
        for h in range(Q.shape[0]):
            Qz = np.nan_to_num(Q[h])
            Kz = np.nan_to_num(K[h])
            logits = scale * (Qz @ Kz.T)
            for tq in range(T):
                R = [r for r in range(tq * tile, (tq + 1) * tile) if r % P < N]
                for tk in range(T):
                    M = [r for r in range(tk * tile, (tk + 1) * tile) if nsp <= r % P < N]
                    if not R or not M:
                        assert sig[h, tq, tk] == -np.inf
                    else:
                        want = logits[np.ix_(R, M)].mean()
                        assert abs(sig[h, tq, tk] - want) <= 1e-12 * (1 + abs(want)), (tq, tk)


def pin_tile_constant_pool(o):
    """Rows equal to c_t inside every tile pool to exactly c_t (pad holds NaN)."""
    S, N, P, nsp, tile = 2, 50, 64, 4, 16
    lay = _lay(o, S, N, P, nsp)
    T = S * P // tile
    c = np.arange(T * 3, dtype=np.float64).reshape(1, T, 3) * 0.25 - 1.0
    X = np.repeat(c, tile, axis=1)
    j = np.arange(S * P) % P
    X[:, j >= N] = np.nan
    qbar, qc = o.tile_pool(X, lay, tile, "query")
    kbar, kc = o.tile_pool(X, lay, tile, "key")
    for t in range(T):
        rows = np.arange(t * tile, (t + 1) * tile) % P
        nq = int(np.sum(rows < N))
        nk = int(np.sum((rows >= nsp) & (rows < N)))
        assert qc[t] == nq and kc[t] == nk
        if nq:
            assert np.array_equal(qbar[0, t], c[0, t])
        if nk:
            assert np.array_equal(kbar[0, t], c[0, t])


def pin_symmetric_scores(o):
    """With Q = K and no specials or pad, query and key tiles coincide: sigma is symmetric."""
    w = synth.WORKLOADS["tiny_s2"]
    inp = synth.make_inputs(w, seed=3)
    lay = o.Layout(*w.layout)
    qbar, qc = o.tile_pool(inp.q, lay, 64, "query")
    kbar, kc = o.tile_pool(inp.k, lay, 64, "key")
    sig = o.tile_scores(qbar, qc, kbar, kc, 0.125)
    assert np.allclose(sig, np.swapaxes(sig, 1, 2), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- select
def _brute_topk(row, k):
    """argmax over all k-subsets of the score sum; ties to the lexicographically smallest set."""
    best, best_set = None, None
    for comb in itertools.combinations(range(len(row)), k):
        s = float(np.sum(row[list(comb)]))
        if best is None or s > best + 1e-12:
            best, best_set = s, comb
    return np.array(best_set, dtype=np.int64)


def pin_select_brute_force(o):
    rng = np.random.default_rng(7)
    for trial in range(60):
        Tk = int(rng.integers(2, 11))
        # small integers: plenty of exact ties between tiles
        row = rng.integers(-3, 4, size=Tk).astype(np.float64) * 0.5
        k = int(rng.integers(0, Tk + 1))
        tpf = [t for t in (1, 2, Tk) if Tk % t == 0][int(rng.integers(0, 2))]
        anchor = int(rng.integers(-1, Tk // tpf))
        want = set(_brute_topk(row, k).tolist()) if k else set()
        if anchor >= 0:
            want |= set(range(anchor * tpf, (anchor + 1) * tpf))
        got = o.select_tiles(row, k, tpf, anchor)
        assert got.tolist() == sorted(want), (row, k, tpf, anchor, got)


def pin_select_invariants(o):
    rng = np.random.default_rng(11)
    for trial in range(40):
        Tk = int(rng.integers(1, 40))
        row = rng.standard_normal(Tk)
        prev = set()
        for k in range(Tk + 2):
            s = o.select_tiles(row, k, 1, -1)
            assert list(s) == sorted(set(s.tolist()))             # ascending, unique
            assert len(s) == min(k, Tk)
            assert prev <= set(s.tolist())                        # nested in k
            prev = set(s.tolist())
            if k <= Tk and k > 0:                                 # the k largest, by value
                thr = np.sort(row)[::-1][k - 1]
                assert np.all(row[s] >= thr)
        assert o.select_tiles(row, Tk + 5, 1, -1).tolist() == list(range(Tk))
    # an empty tile scores -inf: it is only picked once the finite ones run out (lowest index first)
    row = np.array([-np.inf, 2.0, -np.inf, 1.0, -np.inf])
    assert o.select_tiles(row, 2, 1, -1).tolist() == [1, 3]
    assert o.select_tiles(row, 3, 1, -1).tolist() == [0, 1, 3]
    assert o.select_tiles(row, 4, 1, -1).tolist() == [0, 1, 2, 3]
    # -0.0 and +0.0 are the same score: the lower index wins
    assert o.select_tiles(np.array([0.0, -0.0, 0.0]), 1, 1, -1).tolist() == [0]
    assert o.select_tiles(np.array([-0.0, 0.0]), 1, 1, -1).tolist() == [0]
    # the anchor union and the padded table
    sc = np.array([[[5.0, 4.0, 3.0, 2.0, 1.0, 0.0]]])
    idx, cnt = o.select_topk(sc, 2, 3, 1)
    assert idx.shape == (1, 1, 5) and cnt[0, 0] == 5 and idx[0, 0].tolist() == [0, 1, 3, 4, 5]
    idx, cnt = o.select_topk(sc, 2, 3, 0)
    assert cnt[0, 0] == 3 and idx[0, 0].tolist() == [0, 1, 2, -1, -1]


# --------------------------------------------------------------------------- attend
def _sdpa_dense(Q, K, V, qlay, klay, scale):
    """Dense attention through torch's library routine, fp64 on the CPU, key-padding mask."""
    H, Lq, d = Q.shape
    kvalid = (np.arange(K.shape[1]) % klay.stride) < klay.tokens
    qt = torch.from_numpy(np.nan_to_num(Q)).double()
    kt = torch.from_numpy(np.nan_to_num(K)).double()
    vt = torch.from_numpy(np.nan_to_num(V)).double()
    mask = torch.from_numpy(np.broadcast_to(kvalid, (Lq, K.shape[1])).copy())
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    logits = scale * np.einsum("hqd,hkd->hqk", np.nan_to_num(Q), np.nan_to_num(K))
    lse = scipy.special.logsumexp(np.where(kvalid[None, None, :], logits, -np.inf), axis=2)
    return out.numpy(), lse


def pin_dense_matches_library(o):
    for (S, N, P, nsp) in [(2, 60, 64, 5), (3, 100, 128, 2), (2, 64, 64, 0)]:
        Q, K, V = _rand_inputs(S, N, P, nsp, H=2, d=16, seed=N)
        lay = o.Layout(S, N, P, nsp)
        O, lse = o.dense_attend(Q, K, V, lay, lay, 0.25)
        ref, rlse = _sdpa_dense(Q, K, V, lay, lay, 0.25)
        qv = (np.arange(S * P) % P) < N
        assert np.allclose(O[:, qv], ref[:, qv], rtol=0, atol=1e-12)
        assert np.allclose(lse[:, qv], rlse[:, qv], rtol=0, atol=1e-12)
        assert np.all(O[:, ~qv] == 0) and np.all(lse[:, ~qv] == 0)


def _selection(o, Q, K, lay, tile, k, anchor, scale):
    qbar, qc = o.tile_pool(Q, lay, tile, "query")
    kbar, kc = o.tile_pool(K, lay, tile, "key")
    sig = o.tile_scores(qbar, qc, kbar, kc, scale)
    idx, cnt = o.select_topk(sig, k, lay.stride // tile, anchor)
    return idx, cnt, kbar, kc


def pin_all_tiles_is_dense(o):
    """k >= Tk keeps every tile: specials + all member keys = every valid key."""
    for (S, N, P, nsp, tile) in [(2, 60, 64, 5, 16), (3, 37, 48, 5, 16), (2, 64, 64, 0, 32)]:
        Q, K, V = _rand_inputs(S, N, P, nsp, H=2, d=16, seed=P + N)
        lay = o.Layout(S, N, P, nsp)
        Tk = S * P // tile
        idx, cnt, _, _ = _selection(o, Q, K, lay, tile, Tk, 0, 0.25)
        O, lse = o.sparse_attend(Q, K, V, lay, lay, tile, idx, cnt, 0.25)
        ref, rlse = _sdpa_dense(Q, K, V, lay, lay, 0.25)
        qv = (np.arange(S * P) % P) < N
        assert np.allclose(O[:, qv], ref[:, qv], rtol=0, atol=1e-12)
        assert np.allclose(lse[:, qv], rlse[:, qv], rtol=0, atol=1e-12)


def _explicit_key_set(lay, tile, sel):
    """Key rows attended by a query tile, written out by position."""
    S, N, P, nsp = lay
    J = [s * P + j for s in range(S) for j in range(min(nsp, N))]
    for t in sel:
        J += [r for r in range(t * tile, (t + 1) * tile) if nsp <= r % P < N]
    return J


def pin_closed_forms(o):
    """V = c gives O = c; Q = 0 gives the plain (landmark-weighted) mean; convexity."""
    S, N, P, nsp, tile = 3, 45, 64, 5, 16
    lay = o.Layout(S, N, P, nsp)
    Q, K, V = _rand_inputs(S, N, P, nsp, H=2, d=8, seed=5)
    T = S * P // tile
    qv = (np.arange(S * P) % P) < N
    for k, anchor, lm in [(3, 0, False), (2, -1, False), (1, 2, True), (5, 1, True)]:
        idx, cnt, kbar, kc = _selection(o, Q, K, lay, tile, k, anchor, 0.5)
        vbar, _ = o.tile_pool(V, lay, tile, "key")
        kw = dict(kbar=kbar, vbar=vbar, kcount=kc) if lm else {}
        # constant V
        c = np.array([1.5, -2.25, 0.0, 3.0, 7.0, -1.0, 0.5, 2.0])
        Vc = np.broadcast_to(c, V.shape).copy()
        Vc[:, ~qv] = np.nan
        vbc, _ = o.tile_pool(Vc, lay, tile, "key")
        kwc = dict(kbar=kbar, vbar=vbc, kcount=kc) if lm else {}
        O, _ = o.sparse_attend(Q, K, Vc, lay, lay, tile, idx, cnt, 0.5, **kwc)
        assert np.allclose(O[:, qv], c, rtol=1e-13, atol=1e-13)
        # Q = 0: uniform weights; each landmark stands for 64 keys
        Qz = np.zeros_like(Q)
        O, lse = o.sparse_attend(Qz, K, V, lay, lay, tile, idx, cnt, 0.5, **kw)
        for h in range(2):
            for tq in range(T):
                rows = [r for r in range(tq * tile, (tq + 1) * tile) if r % P < N]
                if not rows:
                    continue
                sel = idx[h, tq, :cnt[h, tq]]
                J = _explicit_key_set(lay, tile, sel)
                num = V[h, J].sum(axis=0)
                den = float(len(J))
                if lm:
                    for t in range(T):
                        if t not in set(sel.tolist()) and kc[t] > 0:
                            num = num + 64.0 * vbar[h, t]
                            den += 64.0
                assert np.allclose(O[h, rows], num / den, rtol=0, atol=1e-12)
                assert np.allclose(lse[h, rows], math.log(den), rtol=0, atol=1e-12)
        # convexity over the attended values
        O, _ = o.sparse_attend(Q, K, V, lay, lay, tile, idx, cnt, 0.5)
        for h in range(2):
            for tq in range(T):
                rows = [r for r in range(tq * tile, (tq + 1) * tile) if r % P < N]
                if not rows:
                    continue
                J = _explicit_key_set(lay, tile, idx[h, tq, :cnt[h, tq]])
                lo, hi = V[h, J].min(axis=0), V[h, J].max(axis=0)
                assert np.all(O[h, rows] >= lo - 1e-12) and np.all(O[h, rows] <= hi + 1e-12)


def pin_frame_permutation(o):
    """Permuting frames (the anchor moves with its frame) permutes the outputs."""
    w = synth.with_frames(synth.WORKLOADS["vggt_s8"], 3, heads=2)
    inp = synth.make_inputs(w, seed=2)
    lay = o.Layout(*w.layout)
    perm = np.array([2, 0, 1])                 # new frame s holds old frame perm[s]
    P = w.stride

    def permute(X):
        return X.reshape(X.shape[0], w.frames, P, -1)[:, perm].reshape(X.shape)

    base = o.layer(inp.q, inp.k, inp.v, lay, lay, 64, 3, anchor=0, landmarks=True)
    new_anchor = int(np.nonzero(perm == 0)[0][0])
    moved = o.layer(permute(inp.q), permute(inp.k), permute(inp.v), lay, lay, 64, 3,
                    anchor=new_anchor, landmarks=True)
    assert np.allclose(moved["O"], permute(base["O"]), rtol=0, atol=1e-12)


def pin_query_tiles_independent(o):
    w = synth.with_frames(synth.WORKLOADS["vggt_s8"], 2, heads=2)
    inp = synth.make_inputs(w, seed=4)
    lay = o.Layout(*w.layout)
    full = o.layer(inp.q, inp.k, inp.v, lay, lay, 64, 4, anchor=0, landmarks=True)
    some = [3, 17, 30]
    part = o.layer(inp.q, inp.k, inp.v, lay, lay, 64, 4, anchor=0, landmarks=True,
                   query_tiles=some, heads=[1])
    for t in some:
        r = slice(t * 64, (t + 1) * 64)
        assert np.array_equal(part["O"][1, r], full["O"][1, r])


def pin_landmarks_exact_on_constant_tiles(o):
    """K, V constant inside every full 64-row tile: a landmark (mean K, mean V, +ln 64)
    carries exactly the softmax mass of its tile, so sparse + landmarks = dense for any
    selection (64 * e^{q.k} = sum over the tile's 64 equal keys)."""
    S, N, P, nsp, tile = 2, 256, 256, 0, 64
    rng = np.random.default_rng(9)
    H, d = 2, 8
    T = S * P // tile
    Q = rng.standard_normal((H, S * P, d))
    K = np.repeat(rng.standard_normal((H, T, d)), tile, axis=1)
    V = np.repeat(rng.standard_normal((H, T, d)), tile, axis=1)
    lay = o.Layout(S, N, P, nsp)
    ref, rlse = _sdpa_dense(Q, K, V, lay, lay, 0.4)
    kbar, kc = o.tile_pool(K, lay, tile, "key")
    vbar, _ = o.tile_pool(V, lay, tile, "key")
    for k, anchor in [(0, -1), (1, -1), (2, 0), (3, 1)]:
        idx, cnt, _, _ = _selection(o, Q, K, lay, tile, k, anchor, 0.4)
        O, lse = o.sparse_attend(Q, K, V, lay, lay, tile, idx, cnt, 0.4,
                                 kbar=kbar, vbar=vbar, kcount=kc)
        assert np.allclose(O, ref, rtol=0, atol=1e-12)
        assert np.allclose(lse, rlse, rtol=0, atol=1e-12)


def pin_landmarks_vanish_when_all_selected(o):
    S, N, P, nsp, tile = 2, 60, 64, 5, 16
    lay = o.Layout(S, N, P, nsp)
    Q, K, V = _rand_inputs(S, N, P, nsp, H=2, d=8, seed=13)
    Tk = S * P // tile
    idx, cnt, kbar, kc = _selection(o, Q, K, lay, tile, Tk, -1, 0.3)
    vbar, _ = o.tile_pool(V, lay, tile, "key")
    a, la = o.sparse_attend(Q, K, V, lay, lay, tile, idx, cnt, 0.3, kbar=kbar, vbar=vbar, kcount=kc)
    b, lb = o.sparse_attend(Q, K, V, lay, lay, tile, idx, cnt, 0.3)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def pin_empty_key_set(o):
    """No specials, k = 0, no anchor: nothing to attend; O = 0, lse = -inf."""
    S, N, P, nsp, tile = 2, 64, 64, 0, 32
    lay = o.Layout(S, N, P, nsp)
    Q, K, V = _rand_inputs(S, N, P, nsp, H=1, d=4, seed=1)
    idx, cnt, _, _ = _selection(o, Q, K, lay, tile, 0, -1, 0.5)
    assert np.all(cnt == 0)
    O, lse = o.sparse_attend(Q, K, V, lay, lay, tile, idx, cnt, 0.5)
    assert np.all(O == 0) and np.all(lse == -np.inf)


# --------------------------------------------------------------------------- subsample
def pin_subsample(o):
    # closed form on a 5x5 grid, window 2, 2 specials: rows/cols 0, 2, 4 of the grid
    pos = o.subsample_positions(2, (5, 5), 2)
    assert pos.tolist() == [0, 1] + [2 + p for p in (0, 2, 4, 10, 12, 14, 20, 22, 24)]
    pos = o.subsample_positions(5, (37, 37), 2)
    assert pos.size == 5 + 19 * 19
    assert pos.tolist()[:8] == [0, 1, 2, 3, 4, 5, 7, 9] and pos[-1] == 5 + 36 * 37 + 36
    pos = o.subsample_positions(1, (4, 3), 3)
    assert pos.tolist() == [0, 1 + 0, 1 + 9]
    # attention over all subsampled tiles is dense attention over exactly the kept keys
    S, gh, gw, nsp, tile = 2, 6, 6, 3, 16
    N, P = nsp + gh * gw, 48
    lay = o.Layout(S, N, P, nsp)
    Q, K, V = _rand_inputs(S, N, P, nsp, H=2, d=8, seed=21)
    K2, V2, lay2 = o.subsample_keys(K, V, lay, (gh, gw), 2, tile)
    assert tuple(lay2) == (S, nsp + 9, 16, nsp)
    Tk = S * lay2.stride // tile
    qbar, qc = o.tile_pool(Q, lay, tile, "query")
    kbar, kc = o.tile_pool(K2, lay2, tile, "key")
    idx, cnt = o.select_topk(o.tile_scores(qbar, qc, kbar, kc, 0.3), Tk, lay2.stride // tile, 0)
    O, _ = o.sparse_attend(Q, K2, V2, lay, lay2, tile, idx, cnt, 0.3)
    kept = [s * P + p for s in range(S) for p in
            list(range(nsp)) + [nsp + y * gw + x for y in (0, 2, 4) for x in (0, 2, 4)]]
    qv = np.nonzero((np.arange(S * P) % P) < N)[0]
    qt = torch.from_numpy(Q[:, qv]).double()
    kt = torch.from_numpy(K[:, kept]).double()
    vt = torch.from_numpy(V[:, kept]).double()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.3).numpy()
    assert np.allclose(O[:, qv], ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- hand-worked cases
def _arr(rows):
    return np.array([[float(x) for x in r] for r in rows])


def pin_hand_worked(o):
    spec = json.load(open(GOLDEN))
    env = {"e": math.e, "ln64": math.log(64.0), "__builtins__": {}}
    for case in spec["cases"]:
        L = case["layout"]
        lay = o.Layout(L["frames"], L["tokens"], L["stride"], L["specials"])
        tile, scale = case["tile"], case["scale"]
        Q = _arr(case["q"])[None]
        V = _arr(case["v"])[None]
        qbar, qc = o.tile_pool(Q, lay, tile, "query")
        kbar, kc = o.tile_pool(Q, lay, tile, "key")
        vbar, _ = o.tile_pool(V, lay, tile, "key")
        sig = o.tile_scores(qbar, qc, kbar, kc, scale)
        assert np.allclose(sig[0], np.array(case["sigma"], dtype=float), rtol=0, atol=1e-15)
        for run in case["runs"]:
            want = np.array([eval(s, env) for s in run["o0"]])
            if run["k"] == "dense":
                O, _ = o.dense_attend(Q, Q, V, lay, lay, scale)
            else:
                idx, cnt = o.select_topk(sig, run["k"], lay.stride // tile, run["anchor"])
                got_sel = [idx[0, t, :cnt[0, t]].tolist() for t in range(idx.shape[1])]
                assert got_sel == run["sel"], (case["name"], run, got_sel)
                kw = dict(kbar=kbar, vbar=vbar, kcount=kc) if run["landmarks"] else {}
                O, _ = o.sparse_attend(Q, Q, V, lay, lay, tile, idx, cnt, scale, **kw)
            assert np.allclose(O[0, :, 0], want, rtol=0, atol=1e-12), (case["name"], run, O[0, :, 0])
            qv = (np.arange(lay.rows) % lay.stride) < lay.tokens
            assert np.allclose(O[0, qv, 1], 1.0, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- per-head budgets
def pin_select_per_head(o):
    """Head h of a per-head selection is the brute-force top-k_h of its rows (plus the
    anchor frame), and the table is sized for the largest budget."""
    rng = np.random.default_rng(23)
    for trial in range(12):
        H, Tq, Tk = int(rng.integers(2, 5)), 3, int(rng.integers(3, 10))
        tpf = [t for t in (1, Tk) if Tk % t == 0][int(rng.integers(0, 2))]
        anchor = int(rng.integers(-1, Tk // tpf))
        sc = rng.integers(-3, 4, size=(H, Tq, Tk)).astype(np.float64) * 0.5
        ks = rng.integers(0, Tk + 1, size=H)
        idx, cnt = o.select_topk(sc, ks, tpf, anchor)
        forced = set(range(anchor * tpf, (anchor + 1) * tpf)) if anchor >= 0 else set()
        assert idx.shape[2] == min(Tk, int(ks.max()) + (tpf if anchor >= 0 else 0))
        for h in range(H):
            for t in range(Tq):
                want = (set(_brute_topk(sc[h, t], int(ks[h])).tolist()) if ks[h] else set()) | forced
                assert idx[h, t, :cnt[h, t]].tolist() == sorted(want), (h, t, ks, anchor)
                assert np.all(idx[h, t, cnt[h, t]:] == -1)


# --------------------------------------------------------------------------- frame attention
def _sdpa_block_diagonal(Q, K, V, qlay, klay, scale):
    """Attention through torch's routine with a mask written out from frame numbers:
    query row r (frame r // Pq) may see key row c iff c is in the same frame and valid."""
    qf = np.arange(Q.shape[1]) // qlay.stride
    kf = np.arange(K.shape[1]) // klay.stride
    kvalid = (np.arange(K.shape[1]) % klay.stride) < klay.tokens
    allow = (qf[:, None] == kf[None, :]) & kvalid[None, :]
    t = lambda x: torch.from_numpy(np.nan_to_num(x)).double()
    out = torch.nn.functional.scaled_dot_product_attention(
        t(Q), t(K), t(V), attn_mask=torch.from_numpy(allow), scale=scale)
    logits = scale * np.einsum("hqd,hkd->hqk", np.nan_to_num(Q), np.nan_to_num(K))
    lse = scipy.special.logsumexp(np.where(allow[None], logits, -np.inf), axis=2)
    return out.numpy(), lse


def pin_frame_attention(o):
    for (S, N, P, nsp, Pk, Nk) in [(3, 60, 64, 5, 64, 60), (2, 100, 128, 2, 64, 50), (4, 10, 16, 3, 16, 10)]:
        Q, _, _ = _rand_inputs(S, N, P, nsp, H=2, d=16, seed=N)
        _, K, V = _rand_inputs(S, Nk, Pk, nsp, H=2, d=16, seed=N + 1)
        qlay, klay = o.Layout(S, N, P, nsp), o.Layout(S, Nk, Pk, nsp)
        O, lse = o.frame_attend(Q, K, V, qlay, klay, 0.25)
        ref, rlse = _sdpa_block_diagonal(Q, K, V, qlay, klay, 0.25)
        qv = (np.arange(S * P) % P) < N
        assert np.allclose(O[:, qv], ref[:, qv], rtol=0, atol=1e-12)
        assert np.allclose(lse[:, qv], rlse[:, qv], rtol=0, atol=1e-12)
        assert np.all(O[:, ~qv] == 0) and np.all(lse[:, ~qv] == 0)
    # one frame: frame attention is dense attention
    Q, K, V = _rand_inputs(1, 50, 64, 4, H=2, d=8, seed=3)
    lay = o.Layout(1, 50, 64, 4)
    a, la = o.frame_attend(Q, K, V, lay, lay, 0.3)
    b, lb = o.dense_attend(Q, K, V, lay, lay, 0.3)
    assert np.allclose(a, b, rtol=0, atol=1e-12) and np.allclose(la, lb, rtol=0, atol=1e-12)
    # another frame's keys and values never matter
    Q, K, V = _rand_inputs(3, 40, 64, 2, H=1, d=8, seed=4)
    lay = o.Layout(3, 40, 64, 2)
    a, _ = o.frame_attend(Q, K, V, lay, lay, 0.3)
    K2, V2 = K.copy(), V.copy()
    K2[:, 64:128] += 5.0
    V2[:, 64:128] -= 3.0
    b, _ = o.frame_attend(Q, K2, V2, lay, lay, 0.3)
    assert np.array_equal(a[:, :64], b[:, :64]) and np.array_equal(a[:, 128:], b[:, 128:])
    assert not np.allclose(a[:, 64:104], b[:, 64:104])


# --------------------------------------------------------------------------- subsample completion
def _sga_setup(o, S=2, nsp=2, grid=(4, 4), window=2, tile=16, H=2, d=8, seed=0):
    N = nsp + grid[0] * grid[1]
    P = -(-N // tile) * tile
    Q, K, V = _rand_inputs(S, N, P, nsp, H=H, d=d, seed=seed)
    lay = o.Layout(S, N, P, nsp)
    K2, V2, lay2 = o.subsample_keys(K, V, lay, grid, window, tile)
    km, vm, n = o.discarded_mean(K, V, lay, grid, window)
    return Q, K, V, lay, K2, V2, lay2, km, vm, n


def _explicit_sga(Q, K, V, lay, lay2, K2, V2, key_rows2, drop_pos, km, vm, n, scale, diag, mean):
    """Softmax over an explicitly listed key set per query row: the given subsampled key
    rows, the row's own key if its position was dropped, and n copies of the mean pair."""
    H, L, d = Q.shape
    O = np.zeros((H, L, d))
    for h in range(H):
        for r in range(L):
            if r % lay.stride >= lay.tokens:
                continue
            keys = [K2[h, c] for c in key_rows2]
            vals = [V2[h, c] for c in key_rows2]
            if diag and (r % lay.stride) in drop_pos:
                keys.append(K[h, r]); vals.append(V[h, r])
            if mean:
                keys += [km[h]] * n; vals += [vm[h]] * n
            kk, vv = np.array(keys), np.array(vals)
            z = scale * (kk @ Q[h, r])
            w = np.exp(z - z.max())
            O[h, r] = (w @ vv) / w.sum()
    return O


def pin_sga_explicit_key_list(o):
    """The completion terms equal attention over an explicit key list holding the row's own
    key (only where the subsample dropped it) and |D| copies of the mean pair."""
    for (grid, window, nsp) in [((4, 4), 2, 2), ((5, 3), 2, 1), ((4, 6), 3, 2)]:
        Q, K, V, lay, K2, V2, lay2, km, vm, n = _sga_setup(o, grid=grid, window=window, nsp=nsp,
                                                           seed=grid[1])
        drop = set(o.discarded_positions(lay.specials, grid, window).tolist())
        kept = set(o.subsample_positions(lay.specials, grid, window).tolist())
        assert drop.isdisjoint(kept) and drop | kept == set(range(lay.tokens))
        assert n == lay.frames * len(drop) and n > 0
        scale = 0.35
        all2 = np.nonzero((np.arange(lay2.rows) % lay2.stride) < lay2.tokens)[0]
        for diag, mean in [(True, True), (True, False), (False, True)]:
            sga = dict(grid=grid, window=window,
                       k_full=K if diag else None, v_full=V if diag else None,
                       kmean=km if mean else None, vmean=vm, mean_bias=o.sga_mean_bias(n))
            got, _ = o.dense_attend(Q, K2, V2, lay, lay2, scale, sga=sga)
            want = _explicit_sga(Q, K, V, lay, lay2, K2, V2, all2, drop, km, vm, n, scale, diag, mean)
            qv = (np.arange(lay.rows) % lay.stride) < lay.tokens
            assert np.allclose(got[:, qv], want[:, qv], rtol=0, atol=1e-12), (grid, diag, mean)
        # the same terms on the tile-sparse call: specials + the selected tiles' members
        tile = 16
        T2 = lay2.rows // tile
        mem = ((np.arange(lay2.rows) % lay2.stride >= lay2.specials) &
               (np.arange(lay2.rows) % lay2.stride < lay2.tokens))
        spec = np.nonzero((np.arange(lay2.rows) % lay2.stride) < lay2.specials)[0]
        sel = np.array([T2 - 1], dtype=np.int32)
        idx = np.broadcast_to(sel, (2, lay.rows // tile, 1)).copy()
        cnt = np.ones((2, lay.rows // tile), dtype=np.int32)
        sga = dict(grid=grid, window=window, k_full=K, v_full=V, kmean=km, vmean=vm,
                   mean_bias=o.sga_mean_bias(n))
        got, _ = o.sparse_attend(Q, K2, V2, lay, lay2, tile, idx, cnt, scale, sga=sga)
        rows2 = np.concatenate([spec, (T2 - 1) * tile + np.nonzero(mem[(T2 - 1) * tile:T2 * tile])[0]])
        want = _explicit_sga(Q, K, V, lay, lay2, K2, V2, rows2, drop, km, vm, n, scale, True, True)
        qv = (np.arange(lay.rows) % lay.stride) < lay.tokens
        assert np.allclose(got[:, qv], want[:, qv], rtol=0, atol=1e-12)


def pin_sga_constant_dropped_is_dense(o):
    """If every dropped key and value equals one constant pair, the mean pair with ln |D|
    restores dense attention exactly (|D| e^{q.k} is the dropped columns' total)."""
    Q, K, V, lay, _, _, _, _, _, _ = _sga_setup(o, grid=(6, 4), window=2, nsp=3, seed=9)
    pos = o.discarded_positions(lay.specials, (6, 4), 2)
    rows = (np.arange(lay.frames)[:, None] * lay.stride + pos[None, :]).ravel()
    rng = np.random.default_rng(1)
    for h in range(K.shape[0]):
        K[h, rows] = rng.standard_normal(K.shape[2])
        V[h, rows] = rng.standard_normal(V.shape[2])
    K2, V2, lay2 = o.subsample_keys(K, V, lay, (6, 4), 2, 16)
    km, vm, n = o.discarded_mean(K, V, lay, (6, 4), 2)
    assert np.allclose(km, K[:, rows[0]]) and np.allclose(vm, V[:, rows[0]])
    sga = dict(grid=(6, 4), window=2, k_full=None, v_full=None, kmean=km, vmean=vm,
               mean_bias=o.sga_mean_bias(n))
    got, gl = o.dense_attend(Q, K2, V2, lay, lay2, 0.4, sga=sga)
    want, wl = o.dense_attend(Q, K, V, lay, lay, 0.4)
    qv = (np.arange(lay.rows) % lay.stride) < lay.tokens
    assert np.allclose(got[:, qv], want[:, qv], rtol=0, atol=1e-12)
    assert np.allclose(gl[:, qv], wl[:, qv], rtol=0, atol=1e-12)


def pin_sga_nothing_dropped(o):
    """Window 1 keeps every token: no own-key term applies, |D| = 0, dense attention."""
    Q, K, V, lay, K2, V2, lay2, km, vm, n = _sga_setup(o, grid=(4, 4), window=1, seed=5)
    assert n == 0 and o.discarded_positions(lay.specials, (4, 4), 1).size == 0
    sga = dict(grid=(4, 4), window=1, k_full=K, v_full=V, kmean=None, vmean=None, mean_bias=0.0)
    got, _ = o.dense_attend(Q, K2, V2, lay, lay2, 0.3, sga=sga)
    want, _ = o.dense_attend(Q, K, V, lay, lay, 0.3)
    qv = (np.arange(lay.rows) % lay.stride) < lay.tokens
    assert np.allclose(got[:, qv], want[:, qv], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- backward
def _bwd_case(o, S=2, N=60, P=64, nsp=5, tile=16, k=2, seed=0, H=2, d=8):
    Q, K, V = _rand_inputs(S, N, P, nsp, H=H, d=d, seed=seed)
    lay = o.Layout(S, N, P, nsp)
    idx, cnt, _, _ = _selection(o, Q, K, lay, tile, k, 0, 0.3)
    rng = np.random.default_rng(seed + 1)
    dO = rng.standard_normal(Q.shape)
    return Q, K, V, dO, lay, idx, cnt


def _explicit_mask(lay, tile, idx, cnt, h):
    """[Lq, Lk] boolean: valid query i may attend key j (special, or member of a tile its
    query tile selected), written out from positions."""
    L = lay.rows
    j = np.arange(L) % lay.stride
    qvalid = j < lay.tokens
    special = j < lay.specials
    member = (j >= lay.specials) & (j < lay.tokens)
    M = np.zeros((L, L), dtype=bool)
    for i in np.nonzero(qvalid)[0]:
        tq = i // tile
        allowed = special.copy()
        for t in idx[h, tq, :cnt[h, tq]]:
            allowed[t * tile:(t + 1) * tile] |= member[t * tile:(t + 1) * tile]
        M[i] = allowed
    return M


def pin_backward_autograd(o):
    """The gradient equals torch autograd (fp64, CPU) of masked attention whose mask is
    written out from the selection."""
    for (S, N, P, nsp, tile, k) in [(2, 60, 64, 5, 16, 2), (3, 40, 48, 0, 16, 3), (2, 30, 32, 6, 8, 1)]:
        Q, K, V, dO, lay, idx, cnt = _bwd_case(o, S, N, P, nsp, tile, k, seed=N)
        dQ, dK, dV, D = o.sparse_attend_bwd(Q, K, V, dO, lay, lay, tile, idx, cnt, 0.3)
        qv = (np.arange(lay.rows) % lay.stride) < lay.tokens
        for h in range(Q.shape[0]):
            M = torch.from_numpy(_explicit_mask(lay, tile, idx, cnt, h))
            qt = torch.tensor(np.nan_to_num(Q[h]), requires_grad=True)
            kt = torch.tensor(np.nan_to_num(K[h]), requires_grad=True)
            vt = torch.tensor(np.nan_to_num(V[h]), requires_grad=True)
            logits = (0.3 * qt @ kt.T).masked_fill(~M, float("-inf"))
            rows = torch.from_numpy(qv)
            pr = torch.softmax(logits[rows], dim=1)
            out = pr @ vt
            (out * torch.from_numpy(dO[h][qv])).sum().backward()
            assert np.allclose(dQ[h], qt.grad.numpy(), rtol=0, atol=1e-10)
            assert np.allclose(dK[h], kt.grad.numpy(), rtol=0, atol=1e-10)
            assert np.allclose(dV[h], vt.grad.numpy(), rtol=0, atol=1e-10)
            O, _ = o.sparse_attend(Q, K, V, lay, lay, tile, idx, cnt, 0.3)
            assert np.allclose(D[h, qv], np.sum(dO[h, qv] * O[h, qv], axis=1), rtol=0, atol=1e-12)
            assert np.all(dQ[h, ~qv] == 0) and np.all(D[h, ~qv] == 0)


def pin_backward_finite_difference(o):
    """Central differences of sum(dO * O) through the forward oracle."""
    S, N, P, nsp, tile = 2, 7, 8, 2, 4
    Q, K, V = _rand_inputs(S, N, P, nsp, H=1, d=3, seed=2, pad=0.0)
    lay = o.Layout(S, N, P, nsp)
    idx, cnt, _, _ = _selection(o, Q, K, lay, tile, 1, 0, 0.5)
    dO = np.random.default_rng(3).standard_normal(Q.shape)
    dQ, dK, dV, _ = o.sparse_attend_bwd(Q, K, V, dO, lay, lay, tile, idx, cnt, 0.5)
    f = lambda Q_, K_, V_: float(np.sum(dO * o.sparse_attend(Q_, K_, V_, lay, lay, tile, idx, cnt, 0.5)[0]))
    eps = 1e-6
    for X, G, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        for r in range(X.shape[1]):
            for c in range(X.shape[2]):
                args = [Q.copy(), K.copy(), V.copy()]
                args[which][0, r, c] += eps
                up = f(*args)
                args[which][0, r, c] -= 2 * eps
                dn = f(*args)
                assert abs((up - dn) / (2 * eps) - G[0, r, c]) < 1e-6, (which, r, c)


def _landmark_bwd_case(o, S, N, P, nsp, tile, k, seed):
    Q, K, V, dO, lay, idx, cnt = _bwd_case(o, S, N, P, nsp, tile, k, seed=seed)
    kbar, kc = o.tile_pool(K, lay, tile, "key")
    vbar, _ = o.tile_pool(V, lay, tile, "key")
    return Q, K, V, dO, lay, idx, cnt, kbar, vbar, kc


def pin_backward_landmarks_autograd(o):
    """With landmarks, the gradient equals torch autograd (fp64, CPU) of an explicit
    computation: every query row attends its masked keys plus one pseudo-key per unselected
    tile that has members, whose key and value are the means of the tile's member rows
    taken inside the graph (so the gradient reaches K and V through the mean) and whose
    logit carries the bias; dkbar/dvbar equal the gradients of those means."""
    for (S, N, P, nsp, tile, k, bias) in [(2, 60, 64, 5, 16, 2, math.log(64.0)), (3, 40, 48, 0, 16, 1, 0.7),
                                          (2, 30, 32, 6, 8, 2, 2.0)]:
        Q, K, V, dO, lay, idx, cnt, kbar, vbar, kc = _landmark_bwd_case(o, S, N, P, nsp, tile, k, seed=N + 1)
        dQ, dK, dV, D, dkb, dvb = o.sparse_attend_bwd(Q, K, V, dO, lay, lay, tile, idx, cnt, 0.3, kbar=kbar,
                                                      vbar=vbar, kcount=kc, landmark_bias=bias, means=True)
        L = lay.rows
        j = np.arange(L) % lay.stride
        qv = j < lay.tokens
        member = (j >= lay.specials) & (j < lay.tokens)
        Tk = L // tile
        for h in range(Q.shape[0]):
            M = torch.from_numpy(_explicit_mask(lay, tile, idx, cnt, h))
            qt = torch.tensor(np.nan_to_num(Q[h]), requires_grad=True)
            kt = torch.tensor(np.nan_to_num(K[h]), requires_grad=True)
            vt = torch.tensor(np.nan_to_num(V[h]), requires_grad=True)
            kms, vms = [], []
            for t in range(Tk):
                rows = [r for r in range(t * tile, (t + 1) * tile) if member[r]]
                kms.append(kt[rows].mean(0) if rows else torch.zeros(kt.shape[1], dtype=kt.dtype))
                vms.append(vt[rows].mean(0) if rows else torch.zeros(vt.shape[1], dtype=vt.dtype))
            km, vm = torch.stack(kms), torch.stack(vms)
            km.retain_grad()
            vm.retain_grad()
            # landmark mask [L, Tk]: query row i gets tile t iff its query tile did not select t
            # and t has members
            LMm = np.zeros((L, Tk), dtype=bool)
            has = np.array([member[t * tile:(t + 1) * tile].any() for t in range(Tk)])
            for i in np.nonzero(qv)[0]:
                sel = set(idx[h, i // tile, :cnt[h, i // tile]].tolist())
                LMm[i] = has & np.array([t not in sel for t in range(Tk)])
            logits = torch.cat([(0.3 * qt @ kt.T).masked_fill(~M, float("-inf")),
                                (0.3 * qt @ km.T + bias).masked_fill(~torch.from_numpy(LMm), float("-inf"))], 1)
            rows = torch.from_numpy(qv)
            pr = torch.softmax(logits[rows], dim=1)
            out = pr @ torch.cat([vt, vm])
            (out * torch.from_numpy(dO[h][qv])).sum().backward()
            assert np.allclose(dQ[h], qt.grad.numpy(), rtol=0, atol=1e-10)
            assert np.allclose(dK[h], kt.grad.numpy(), rtol=0, atol=1e-10)
            assert np.allclose(dV[h], vt.grad.numpy(), rtol=0, atol=1e-10)
            assert np.allclose(dkb[h], km.grad.numpy(), rtol=0, atol=1e-10)
            assert np.allclose(dvb[h], vm.grad.numpy(), rtol=0, atol=1e-10)
            O, _ = o.sparse_attend(Q, K, V, lay, lay, tile, idx, cnt, 0.3, kbar=kbar, vbar=vbar, kcount=kc,
                                   landmark_bias=bias)
            assert np.allclose(D[h, qv], np.sum(dO[h, qv] * O[h, qv], axis=1), rtol=0, atol=1e-12)


def pin_backward_landmarks_finite_difference(o):
    """Central differences of sum(dO * O) through the forward oracle with landmarks, the
    means recomputed from the perturbed K and V by the pool (selection held fixed)."""
    S, N, P, nsp, tile = 2, 7, 8, 2, 4
    Q, K, V = _rand_inputs(S, N, P, nsp, H=1, d=3, seed=4, pad=0.0)
    lay = o.Layout(S, N, P, nsp)
    idx, cnt, _, _ = _selection(o, Q, K, lay, tile, 1, -1, 0.5)
    dO = np.random.default_rng(5).standard_normal(Q.shape)

    def f(Q_, K_, V_):
        kb, kc = o.tile_pool(K_, lay, tile, "key")
        vb, _ = o.tile_pool(V_, lay, tile, "key")
        return float(np.sum(dO * o.sparse_attend(Q_, K_, V_, lay, lay, tile, idx, cnt, 0.5, kbar=kb, vbar=vb,
                                                 kcount=kc)[0]))
    kb, kc = o.tile_pool(K, lay, tile, "key")
    vb, _ = o.tile_pool(V, lay, tile, "key")
    dQ, dK, dV, _ = o.sparse_attend_bwd(Q, K, V, dO, lay, lay, tile, idx, cnt, 0.5, kbar=kb, vbar=vb, kcount=kc)
    assert np.any(cnt[0] < S * P // tile)                      # some tiles are landmarks
    eps = 1e-6
    for X, G, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        for r in range(X.shape[1]):
            for c in range(X.shape[2]):
                args = [Q.copy(), K.copy(), V.copy()]
                args[which][0, r, c] += eps
                up = f(*args)
                args[which][0, r, c] -= 2 * eps
                dn = f(*args)
                assert abs((up - dn) / (2 * eps) - G[0, r, c]) < 1e-6, (which, r, c)


def pin_backward_magnitudes_bound_the_gradients(o):
    """The absolute-value sums returned with ``magnitudes`` bound the gradients by the
    triangle inequality (|dS_ij| = P_ij |dP_ij - D_i| <= M_ij, |D_i| <= A_D_i), with and
    without landmarks; every gradient entry that is nonzero has a nonzero magnitude."""
    for lm in (False, True):
        Q, K, V, dO, lay, idx, cnt, kbar, vbar, kc = _landmark_bwd_case(o, 2, 60, 64, 5, 16, 2, seed=9)
        kw = dict(kbar=kbar, vbar=vbar, kcount=kc) if lm else {}
        *g, mag = o.sparse_attend_bwd(Q, K, V, dO, lay, lay, 16, idx, cnt, 0.3, magnitudes=True, means=True, **kw)
        for x, n in zip(g, ("dQ", "dK", "dV", "D", "dkbar", "dvbar")):
            assert np.all(np.abs(x) <= mag[n] * (1 + 1e-12) + 1e-300), n
            assert np.all(mag[n][x != 0] > 0), n


def pin_backward_gradient_sums(o):
    """Sums fixed by the softmax: each valid row's weights over all its keys (landmark
    means included) add to 1, so the value gradients of all keys add to the sum of the
    cotangents of the valid rows; dS_i sums to P_i . dP_i - D_i = 0 over a row, so the key
    gradients add to 0.  Through the mean pool a mean's gradient reaches its member rows
    divided by their count, so the sums over K and V rows are the same as over the keys."""
    for lm in (False, True):
        for (S, N, P, nsp, tile, k) in [(2, 60, 64, 5, 16, 2), (3, 40, 48, 2, 16, 1)]:
            Q, K, V, dO, lay, idx, cnt, kbar, vbar, kc = _landmark_bwd_case(o, S, N, P, nsp, tile, k, seed=N + 7)
            kw = dict(kbar=kbar, vbar=vbar, kcount=kc) if lm else {}
            dQ, dK, dV, D, dkb, dvb = o.sparse_attend_bwd(Q, K, V, dO, lay, lay, tile, idx, cnt, 0.3, means=True,
                                                          **kw)
            qv = (np.arange(lay.rows) % lay.stride) < lay.tokens
            for h in range(Q.shape[0]):
                assert np.allclose(dV[h].sum(axis=0), dO[h][qv].sum(axis=0), rtol=0, atol=1e-10)
                assert np.allclose(dK[h].sum(axis=0), 0.0, rtol=0, atol=1e-10)


def pin_select_mask_equals_per_row_rule(o):
    """The whole-matrix selection mask equals ``select_tiles`` row by row, on rows full of
    ties (integer scores), signed zeros, -inf entries and constant rows, for budgets from 0
    past Tk, per head, with and without the anchor."""
    rng = np.random.default_rng(41)
    for trial in range(12):
        H, Tq, tpf = 2, int(rng.integers(1, 9)), int(rng.integers(1, 5))
        Tk = tpf * int(rng.integers(1, 6))
        sc = rng.integers(-3, 3, (H, Tq, Tk)).astype(np.float64)
        sc[:, ::3] = rng.standard_normal((H, sc[:, ::3].shape[1], Tk))
        sc[sc == 0] = np.where(rng.random(np.count_nonzero(sc == 0)) < 0.5, -0.0, 0.0)
        sc[rng.random(sc.shape) < 0.1] = -np.inf
        if Tq > 1:
            sc[:, 1] = 2.5
        ks = [int(x) for x in rng.integers(0, Tk + 3, H)]
        for anchor in (-1, 0, Tk // tpf - 1):
            m = o.select_mask(sc, ks, tpf, anchor)
            for h in range(H):
                for t in range(Tq):
                    want = o.select_tiles(sc[h, t], ks[h], tpf, anchor)
                    assert np.array_equal(np.nonzero(m[h, t])[0], want), (trial, h, t, anchor)


def pin_selection_transpose(o):
    rng = np.random.default_rng(31)
    for _ in range(10):
        H, Tq, Tk = 2, int(rng.integers(1, 12)), int(rng.integers(1, 12))
        sc = rng.standard_normal((H, Tq, Tk))
        k = int(rng.integers(0, Tk + 1))
        idx, cnt = o.select_topk(sc, k, 1, -1)
        T = o.selection_transpose(idx, cnt, Tk)
        for h in range(H):
            for t in range(Tk):
                want = [tq for tq in range(Tq) if t in set(idx[h, tq, :cnt[h, tq]].tolist())]
                assert T[h][t] == want


ALL_PINS = [
    pin_backward_gradient_sums,
    pin_block_mean_identity, pin_tile_constant_pool, pin_symmetric_scores,
    pin_select_brute_force, pin_select_invariants,
    pin_dense_matches_library, pin_all_tiles_is_dense, pin_closed_forms,
    pin_frame_permutation, pin_query_tiles_independent,
    pin_landmarks_exact_on_constant_tiles, pin_landmarks_vanish_when_all_selected,
    pin_empty_key_set, pin_subsample, pin_hand_worked,
    pin_select_per_head, pin_frame_attention,
    pin_sga_explicit_key_list, pin_sga_constant_dropped_is_dense, pin_sga_nothing_dropped,
    pin_backward_autograd, pin_backward_finite_difference, pin_selection_transpose,
    pin_backward_landmarks_autograd, pin_backward_landmarks_finite_difference,
    pin_backward_magnitudes_bound_the_gradients, pin_select_mask_equals_per_row_rule,
]
