"""HIP path vs the fp64 oracle, through the C ABI, on seeded inputs (needs an MI355X).

Selections: bit-exact against the oracle's rule applied to the GPU's fp32 scores,
and equal to the oracle's own fp64 selection wherever the k-th/(k+1)-th score gap
exceeds 1e-3 relative.  Outputs, given the GPU's selection: max-abs 1e-4 for fp32
inputs, 2e-2 for bf16.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from dynamic_block_sparse_tile_amd import layer as LY
from dynamic_block_sparse_tile_amd import sparse3d as S
from dynamic_block_sparse_tile_amd import synth
from parity_helpers import (TOL, check_scores, check_selection, check_selection_all_rows,
                            compare_outputs, dev, oracle_pool_scores, sample_tiles, say, tdt, to_dev)

pytestmark = pytest.mark.gpu

# bf16 path: the row sum accumulates the bf16-rounded probabilities (the weights that
# multiply V).  bf16 keeps 8 significant bits, so each is within a relative 2^-8 of the
# exact value and the log-sum-exp is within ln(1 + 2^-8) = 3.9e-3 of the oracle's, plus
# fp32 rounding
LSE_TOL_BF16 = 4e-3


def run_full_case(w, seed=0, k=None, landmarks=None, out_f32=True, pad=0.0):
    """Whole layer on the GPU, everything compared with the oracle (small workloads)."""
    k = w.k if k is None else k
    lm = w.landmarks if landmarks is None else landmarks
    say(f"[case] {w.name} seed={seed} k={k} landmarks={lm} dtype={w.dtype}")
    inp = synth.make_inputs(w, seed=seed, pad_value=pad)
    dt = tdt(w)
    q, v = to_dev(inp.q, dt), to_dev(inp.v, dt)
    lay = w.layout
    res = LY.sparse_global_attention(q, q, v, lay, top_k=k, anchor_frame=w.anchor, landmarks=lm,
                                     out_dtype=torch.float32 if out_f32 else None, return_lse=True)
    torch.cuda.synchronize()
    ol = oracle.Layout(*lay)
    ref = oracle_pool_scores(inp, ol, ol, landmarks=lm)
    g = {n: getattr(res, n).cpu().numpy() for n in ("qbar", "kbar", "scores", "idx", "cnt")}
    check_scores(g["qbar"], g["kbar"], g["scores"], ref)
    tpf = w.stride // 64
    nm, n = check_selection(g["scores"], g["idx"], g["cnt"], ref["scores"], k, tpf, w.anchor)
    kw = dict(kbar=ref["kbar"], vbar=ref["vbar"], kcount=ref["kcount"]) if lm else {}
    O, lse = oracle.sparse_attend(inp.q, inp.k, inp.v, ol, ol, 64, g["idx"], g["cnt"], 0.125, **kw)
    out = res.out.float().cpu().numpy()
    tol = TOL[w.dtype] if out_f32 or w.dtype == "f32" else 2e-2
    H, L, _ = out.shape
    pairs = [(h, t) for h in range(H) for t in range(L // 64)]
    worst = compare_outputs(out, O, pairs, tol=tol, g_lse=res.lse.cpu().numpy(), ref_lse=lse,
                            lse_tol=LSE_TOL_BF16 if w.dtype == "bf16" else 1e-5)
    qv = (np.arange(L) % w.stride) < w.tokens
    assert np.all(out[:, ~qv] == 0)
    say(f"  ok: margin rows {nm}/{n}, max|dO| = {worst:.2e}")
    return res, inp


def test_tiny_fp32_layer():
    run_full_case(synth.WORKLOADS["tiny_s2"])


@pytest.mark.parametrize("seed", [1, 2])
def test_tiny_fp32_seeds_and_k(seed):
    w = synth.WORKLOADS["tiny_s2"]
    for k in (0, 1, 3, 8):
        run_full_case(w, seed=seed, k=k)


def test_tiny_fp32_landmarks():
    run_full_case(synth.WORKLOADS["tiny_s2"], landmarks=True)


def test_tiny_fp32_dense():
    w = synth.WORKLOADS["tiny_s2"]
    inp = synth.make_inputs(w, seed=0)
    q, v = to_dev(inp.q, torch.float32), to_dev(inp.v, torch.float32)
    out, lse = S.sparse3d_dense_attn_fwd(q, q, v, w.layout, return_lse=True)
    torch.cuda.synchronize()
    ol = oracle.Layout(*w.layout)
    O, L = oracle.dense_attend(inp.q, inp.k, inp.v, ol, ol, 0.125)
    assert float(np.max(np.abs(out.cpu().numpy() - O))) <= 1e-4
    assert float(np.max(np.abs(lse.cpu().numpy() - L))) <= 1e-5


def test_vggt_s8_bf16_layer_f32_out():
    run_full_case(synth.WORKLOADS["vggt_s8"])


def test_vggt_s8_bf16_layer_bf16_out():
    run_full_case(synth.WORKLOADS["vggt_s8"], out_f32=False, seed=3)


def test_vggt_s8_landmarks():
    run_full_case(synth.WORKLOADS["vggt_s8"], landmarks=True, seed=4)


def test_vggt_s8_dense_sampled():
    w = synth.WORKLOADS["vggt_s8"]
    inp = synth.make_inputs(w, seed=5)
    q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    out, lse = S.sparse3d_dense_attn_fwd(q, q, v, w.layout, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ol = oracle.Layout(*w.layout)
    rows = np.concatenate([np.arange(0, 200), np.arange(5000, 5400), np.arange(11000, 11264)])
    O, L = oracle.dense_attend(inp.q, inp.k, inp.v, ol, ol, 0.125, query_rows_subset=rows)
    g, gl = out.cpu().numpy(), lse.cpu().numpy()
    qv = rows[(rows % w.stride) < w.tokens]
    assert float(np.max(np.abs(g[:, qv] - O[:, qv]))) <= 2e-2
    assert float(np.max(np.abs(gl[:, qv] - L[:, qv]))) <= LSE_TOL_BF16
    pad = rows[(rows % w.stride) >= w.tokens]
    assert np.all(g[:, pad] == 0) and np.all(gl[:, pad] == 0)


# ------------------------------------------------------------------ edge cases
def _custom(frames, tokens, stride, specials, heads=2, dtype="bf16", k=3, **kw):
    return synth.Workload(name=f"custom_{frames}x{tokens}_{stride}_{specials}", frames=frames,
                          tokens=tokens, stride=stride, specials=specials, heads=heads, dtype=dtype,
                          structure="cyclic1d", bank=max(tokens - specials, 1), k=k, **kw)


def test_ragged_and_empty_tiles():
    # tile 2 of every frame has no valid rows (empty query and key tile, scores -inf)
    run_full_case(_custom(3, 70, 192, 5, k=2))
    run_full_case(_custom(3, 70, 192, 5, k=2, dtype="f32"))


def test_specials_span_tiles():
    # 70 specials per frame: key tile 0 holds only specials (no members) and the
    # special pseudo-tiles run past 64 rows
    run_full_case(_custom(2, 150, 192, 70, k=2))
    run_full_case(_custom(2, 150, 192, 70, k=2), landmarks=True)


@pytest.mark.parametrize("specials", [1, 3, 64, 65])
def test_special_counts(specials):
    # The special pseudo-tiles gather every frame's special tokens in frame order, and each
    # staged row finds its frame as the quotient of its index by the special count: one
    # per frame, a count that leaves pseudo-tile rows unfilled, a frame's worth that fills a
    # pseudo-tile exactly, and one that spills into the next (5 frames: 1 to 6 pseudo-tiles)
    run_full_case(_custom(5, specials + 100, 192, specials, k=2))


def test_rising_logits_move_the_reference():
    # Every frame's tokens scaled by 2^frame (exact in bf16): scores grow by factors of up to
    # 2^(2*3) across frames, spanning ~100 base-2 units, so the sparse kernel's running
    # reference must move many times within a row (its slow path) and every rescale of O
    # and l is exercised; outputs and lse still match the oracle.
    w = _custom(4, 256, 256, 5, k=6)
    inp = synth.make_inputs(w, seed=3)
    S_, P = w.frames, w.stride
    scale = np.repeat(2.0 ** np.arange(S_), P).astype(np.float32)[None, :, None]
    q_np = (inp.q * scale).astype(np.float32)
    assert np.array_equal(torch.from_numpy(q_np).to(torch.bfloat16).float().numpy(), q_np)   # exact
    q, v = to_dev(q_np, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    res = LY.sparse_global_attention(q, q, v, w.layout, top_k=w.k, anchor_frame=w.anchor,
                                     out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ol = oracle.Layout(*w.layout)
    g_idx, g_cnt = res.idx.cpu().numpy(), res.cnt.cpu().numpy()
    O, lse = oracle.sparse_attend(q_np, q_np, inp.v, ol, ol, 64, g_idx, g_cnt, 0.125)
    out = res.out.cpu().numpy()
    H, L, _ = out.shape
    pairs = [(h, t) for h in range(H) for t in range(L // 64)]
    # lse reaches several hundred here; its fp32 accumulation error stays far below 1e-2
    worst = compare_outputs(out, O, pairs, tol=TOL["bf16"], g_lse=res.lse.cpu().numpy(), ref_lse=lse,
                            lse_tol=1e-2)
    say(f"  ok: max|dO| = {worst:.2e}")


def test_select_topk_hard_rows():
    # Score rows built to stress the k-th-largest search: heavy ties, values spread over
    # many binades (with overflow to +inf), masked (-inf) entries, constant rows and signed
    # zeros, at lengths that take each wave width (full rows: 512, 1024, 2048, 2816, 4096,
    # 5632, 6144; the others ragged, and a matrix that starts 4 bytes past an aligned
    # address) and the workgroup kernel (6500: longer than a wave holds).  Budgets up to 138
    # finish on the short list of keys at or above the bracket; larger ones, and the rows of
    # many equal values, bisect the whole row.  Compared with the oracle's rule applied to
    # the same fp32 scores.
    rng = np.random.default_rng(21)
    for Tk in (100, 512, 1000, 1001, 1024, 2000, 2048, 2816, 3000, 3072, 4096, 5000, 5632, 6144, 6500, -1000):
        shifted = Tk < 0
        Tk = abs(Tk)
        tpf = 22 if Tk % 22 == 0 else (20 if Tk % 20 == 0 else (16 if Tk % 16 == 0 else 1))
        rows = [rng.standard_normal(Tk),
                rng.integers(-3, 3, Tk).astype(np.float64),
                np.exp(rng.normal(0.0, 20.0, Tk)),
                rng.standard_normal(Tk) * 10.0 ** rng.integers(-30, 30, Tk),
                np.where(rng.random(Tk) < 0.5, -np.inf, rng.standard_normal(Tk)),
                np.full(Tk, -np.inf),
                np.full(Tk, 2.5)]
        r = rng.standard_normal(Tk)
        r[::7] = 0.0
        r[::11] = -0.0
        rows.append(r)
        with np.errstate(over="ignore"):
            sc = np.stack(rows).astype(np.float32)[None]
        g = to_dev(sc, torch.float32)
        if shifted:                                   # same values, 4 bytes past alignment
            buf = torch.empty(g.numel() + 1, device=g.device, dtype=torch.float32)
            g = buf[1:].view(g.shape)
            g.copy_(to_dev(sc, torch.float32))
            assert g.data_ptr() % 16 == 4
        say(f"[case] select hard rows Tk={Tk}{' (shifted)' if shifted else ''}")
        # anchor frames: none, the first, one whose tiles straddle a 256-tile group boundary
        # (frame 11 of 22-tile frames covers tiles 242..263) where it exists, and the last
        nf = Tk // tpf
        anchors = sorted({a for a in (-1, 0, 11, nf - 1) if a < nf})
        for k in (1, 5, 138, Tk - 1, Tk, Tk + 3):
            for anchor in anchors:
                idx, cnt = S.sparse3d_select_topk(g, k, tpf, anchor)
                gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
                for t in range(sc.shape[1]):
                    ref = oracle.select_tiles(sc[0, t].astype(np.float64), k, tpf, anchor)
                    assert gc[0, t] == len(ref) and np.array_equal(gi[0, t, :gc[0, t]], ref), (Tk, k, anchor, t)
                    assert np.all(gi[0, t, gc[0, t]:] == -1)


def test_long_selection_lists():
    # more than 128 selected tiles per query tile (the staged index list spans several
    # passes of the workgroup) and a landmark bitmap wider than 128 words
    w = _custom(24, 1374, 1408, 5, heads=2, k=300)
    run_full_case(w, seed=5)
    run_full_case(w, seed=6, landmarks=True)


def test_selection_longer_than_lds_list():
    # 8200 one-tile frames, k = 8100: the list is too long to stage in LDS next to the tile
    # buffers, so the launcher takes the generic kernel; sampled query tiles vs the oracle
    w = synth.Workload(name="long_list", frames=8200, tokens=64, stride=64, specials=0, heads=1,
                       structure="cyclic1d", bank=64, grid=(8, 8), k=8100)
    inp = synth.make_inputs(w, seed=3)
    q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    res = LY.sparse_global_attention(q, q, v, w.layout, top_k=8100, anchor_frame=-1,
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    idx, cnt = res.idx.cpu().numpy(), res.cnt.cpu().numpy()
    assert idx.shape[2] == 8100 and np.all(cnt == 8100)
    ol = oracle.Layout(*w.layout)
    tiles = [0, 4100, 8199]
    O, _ = oracle.sparse_attend(inp.q, inp.k, inp.v, ol, ol, 64, idx, cnt, 0.125, query_tiles=tiles)
    compare_outputs(res.out.cpu().numpy(), O, [(0, t) for t in tiles], tol=2e-2)


def test_single_frame_and_anchor_off():
    run_full_case(_custom(1, 100, 128, 3, k=1, anchor=-1))
    run_full_case(_custom(4, 64, 64, 0, k=2, anchor=-1))


def test_k_all_tiles_equals_dense():
    w = synth.with_frames(synth.WORKLOADS["vggt_s8"], 2, heads=2)
    inp = synth.make_inputs(w, seed=7)
    q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    Tk = w.rows // 64
    res = LY.sparse_global_attention(q, q, v, w.layout, top_k=Tk, out_dtype=torch.float32)
    dense = S.sparse3d_dense_attn_fwd(q, q, v, w.layout, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(res.cnt == Tk)
    ol = oracle.Layout(*w.layout)
    O, _ = oracle.dense_attend(inp.q, inp.k, inp.v, ol, ol, 0.125)
    assert float(np.max(np.abs(res.out.cpu().numpy() - O))) <= 2e-2
    assert float(np.max(np.abs(dense.cpu().numpy() - O))) <= 2e-2
    # same keys, different tile order and pseudo-tiles, and the probabilities rounded to
    # bf16 against different references (the sparse kernel's running reference, the dense
    # kernel's tile max): the two agree to about one bf16 rounding of the weights
    assert float((res.out - dense).abs().max()) <= 1e-2


def test_dense_and_frame_with_odd_tiles_per_frame():
    # 3 tiles per frame, 4 frames: with an odd number of tiles per frame the dense and the
    # frame call both take one query tile per workgroup (the two-tile instance needs an even
    # count, so that a pair never straddles a frame)
    w = _custom(4, 150, 192, 5, heads=2)
    inp = synth.make_inputs(w, seed=17)
    q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    ol = oracle.Layout(*w.layout)
    d, dl = S.sparse3d_dense_attn_fwd(q, q, v, w.layout, out_dtype=torch.float32, return_lse=True)
    f, fl = S.sparse3d_frame_attn_fwd(q, q, v, w.layout, w.layout, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    O, L = oracle.dense_attend(inp.q, inp.k, inp.v, ol, ol, 0.125)
    Of, Lf = oracle.frame_attend(inp.q, inp.k, inp.v, ol, ol, 0.125)
    qv = (np.arange(O.shape[1]) % w.stride) < w.tokens
    for g, gl, r, rl in ((d, dl, O, L), (f, fl, Of, Lf)):
        g, gl = g.cpu().numpy(), gl.cpu().numpy()
        assert float(np.max(np.abs(g - r))) <= TOL["bf16"]
        assert float(np.max(np.abs(gl[:, qv] - rl[:, qv]))) <= LSE_TOL_BF16
        assert np.all(g[:, ~qv] == 0)


def test_empty_key_set():
    w = _custom(2, 128, 128, 0, dtype="f32", k=0, anchor=-1)
    inp = synth.make_inputs(w, seed=1)
    q, v = to_dev(inp.q, torch.float32), to_dev(inp.v, torch.float32)
    res = LY.sparse_global_attention(q, q, v, w.layout, top_k=0, anchor_frame=-1, return_lse=True)
    torch.cuda.synchronize()
    assert res.idx.shape[2] == 0 and torch.all(res.cnt == 0)
    assert torch.all(res.out == 0) and torch.all(torch.isneginf(res.lse))


def test_nan_pad_is_never_read():
    w = synth.with_frames(synth.WORKLOADS["vggt_s8"], 3, heads=2, k=5)
    a = synth.make_inputs(w, seed=11, pad_value=0.0)
    b = synth.make_inputs(w, seed=11, pad_value=float("nan"))
    outs = []
    for inp in (a, b):
        q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
        r = LY.sparse_global_attention(q, q, v, w.layout, top_k=5, landmarks=True, return_lse=True)
        d = S.sparse3d_dense_attn_fwd(q, q, v, w.layout)
        torch.cuda.synchronize()
        outs.append((r, d))
    (ra, da), (rb, db) = outs
    for x, y in ((ra.out, rb.out), (ra.lse, rb.lse), (ra.scores, rb.scores), (ra.idx, rb.idx),
                 (ra.kbar, rb.kbar), (ra.vbar, rb.vbar), (da, db)):
        assert torch.equal(x, y)


def test_deterministic():
    w = synth.with_frames(synth.WORKLOADS["vggt_s32"], 6, heads=4, k=12)
    inp = synth.make_inputs(w, seed=2)
    q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    r1 = LY.sparse_global_attention(q, q, v, w.layout, top_k=12, landmarks=True)
    r2 = LY.sparse_global_attention(q, q, v, w.layout, top_k=12, landmarks=True)
    torch.cuda.synchronize()
    for n in ("out", "scores", "idx", "cnt", "qbar", "kbar", "vbar"):
        assert torch.equal(getattr(r1, n), getattr(r2, n)), n


def test_constant_v_and_convexity():
    w = synth.with_frames(synth.WORKLOADS["vggt_s8"], 2, heads=2, k=4)
    inp = synth.make_inputs(w, seed=3)
    q = to_dev(inp.q, torch.bfloat16)
    vc = torch.full_like(q, 1.5)
    r = LY.sparse_global_attention(q, q, vc, w.layout, top_k=4, landmarks=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qv = torch.from_numpy((np.arange(w.rows) % w.stride) < w.tokens).to(q.device)
    o = r.out[:, qv]
    assert float((o - 1.5).abs().max()) <= 1.5 * 2 ** -8
    v = to_dev(inp.v, torch.bfloat16)
    r = LY.sparse_global_attention(q, q, v, w.layout, top_k=4, out_dtype=torch.float32)
    torch.cuda.synchronize()
    vmax = float(v.float().abs().max())
    assert float(r.out.abs().max()) <= vmax * (1 + 2 ** -8)


def _permutation_case(w, k, tol, dtype):
    inp = synth.make_inputs(w, seed=8)
    perm = np.array([2, 0, 3, 1])
    P = w.stride

    def permute(x):
        return np.ascontiguousarray(x.reshape(x.shape[0], w.frames, P, -1)[:, perm].reshape(x.shape))

    outs = []
    for (qq, vv, anchor) in ((inp.q, inp.v, 0),
                             (permute(inp.q), permute(inp.v), int(np.nonzero(perm == 0)[0][0]))):
        q, v = to_dev(qq, dtype), to_dev(vv, dtype)
        r = LY.sparse_global_attention(q, q, v, w.layout, top_k=k, anchor_frame=anchor,
                                       landmarks=True, out_dtype=torch.float32)
        torch.cuda.synchronize()
        outs.append(r.out.cpu().numpy())
    err = float(np.max(np.abs(outs[1] - permute(outs[0]))))
    say(f"  permutation max diff {err:.2e}")
    assert err <= tol


def test_frame_permutation_bf16():
    # the tile order changes with the permutation, so P is rounded to bf16 against a
    # different running max: equal within the bf16 bar, not bitwise
    _permutation_case(synth.with_frames(synth.WORKLOADS["vggt_s32"], 4, heads=2), 10, 2e-2,
                      torch.bfloat16)


def test_frame_permutation_fp32():
    w = synth.Workload(name="perm_f32", frames=4, tokens=256, stride=256, specials=0, heads=2,
                       dtype="f32", structure="cyclic1d", bank=256, grid=(16, 16), k=3)
    _permutation_case(w, 3, 1e-4, torch.float32)


# ------------------------------------------------------------------ full-size workloads
def _full_size(name, n_tiles=48, seed=0):
    w = synth.WORKLOADS[name]
    say(f"[full] {name}: generating inputs")
    inp = synth.make_inputs(w, seed=seed)
    q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    lay, klay = w.layout, w.layout
    K, V = q, v
    if w.kv_window > 1:
        K, V, klay = S.sparse3d_grid_subsample_kv(q, v, lay, w.grid, w.kv_window)
    qbar, kbar, vbar, scores, km, vm = S.sparse3d_tile_scores(q, K, lay, klay, v=V if w.landmarks else None,
                                                              operand_means=True)
    tpf = klay[2] // 64
    Tq, Tk = scores.shape[1], scores.shape[2]
    ts = LY.special_tiles(klay)
    k = LY.calibrate_k(LY.device_count_fn(scores, tpf, w.anchor), w.heads * Tq, ts, Tk,
                       w.target_sparsity)
    idx, cnt = S.sparse3d_select_topk(scores, k, tpf, w.anchor)
    if w.landmarks:                                   # the pooling pass's means equal the cast
        assert torch.equal(km, S.sparse3d_cast(kbar, q.dtype)) and torch.equal(vm, S.sparse3d_cast(vbar, q.dtype))
    else:
        km = vm = None
    out = S.sparse3d_sparse_attn_fwd(q, K, V, lay, klay, idx, cnt, kbar=km, vbar=vm)
    torch.cuda.synchronize()
    sp = LY.measured_sparsity(int(cnt.sum()), w.heads * Tq, ts, Tk)
    say(f"[full] {name}: k={k} sparsity={sp:.4f}")
    assert abs(sp - w.target_sparsity) < 0.01
    ol = oracle.Layout(*lay)
    okl = oracle.Layout(*klay)
    Kn, Vn = inp.k, inp.v
    if w.kv_window > 1:
        Kn, Vn, okl2 = oracle.subsample_keys(inp.k, inp.v, ol, w.grid, w.kv_window, 64)
        assert tuple(okl2) == tuple(klay)
        assert np.array_equal(K.float().cpu().numpy(), Kn) and np.array_equal(V.float().cpu().numpy(), Vn)
    ref = oracle_pool_scores(inp, ol, okl, K=Kn, V=Vn, landmarks=w.landmarks)
    pairs = sample_tiles(w.heads, Tq, n_tiles, seed=seed)
    g_scores = scores.cpu().numpy()
    # pooled summaries and scores everywhere, one head of scores at a time
    for h in range(w.heads):
        check_scores(qbar[h:h + 1].cpu().numpy(), kbar[h:h + 1].cpu().numpy(), g_scores[h:h + 1],
                     dict(qbar=ref["qbar"][h:h + 1], kbar=ref["kbar"][h:h + 1], scores=ref["scores"][h:h + 1]))
    say(f"[full] {name}: scores checked on every row")
    # the selection on every (head, query tile) row: the oracle's rule on the GPU's scores,
    # and the oracle's own fp64 selection wherever the margin exceeds 1e-3
    g_idx, g_cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    nm, n = check_selection_all_rows(g_scores, g_idx, g_cnt, ref["scores"], k, tpf, w.anchor)
    say(f"[full] {name}: selection identical on all {n} rows ({nm} margin rows)")
    kw = dict(kbar=ref["kbar"], vbar=ref["vbar"], kcount=ref["kcount"]) if w.landmarks else {}
    heads = sorted({h for h, _ in pairs})
    O, _ = oracle.sparse_attend(inp.q, Kn, Vn, ol, okl, 64, g_idx, g_cnt, 0.125,
                                query_tiles=sorted({t for _, t in pairs}), heads=heads, **kw)
    worst = compare_outputs(out.float().cpu().numpy(), O, pairs, tol=2e-2)
    say(f"[full] {name}: margin rows {nm}/{n}, max|dO| = {worst:.2e}")


def test_full_vggt_s32():
    _full_size("vggt_s32")


def test_full_vggt_s128():
    _full_size("vggt_s128", n_tiles=32)


def test_full_vggt_s128_90():
    # the 90 % sparsity point of the S = 128 workload (k calibrated to about 251)
    _full_size("vggt_s128_90", n_tiles=32)


def test_full_vggt_s256_landmarks():
    _full_size("vggt_s256_lm", n_tiles=16)


def test_full_vggt_s256_landmarks_subsampled():
    _full_size("vggt_s256_lm_sub2", n_tiles=16)


def _bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even, NaN kept NaN (from the formats'
    definitions: drop the low 16 bits with the usual tie-to-even carry)."""
    b = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    r[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint16)            # quiet NaN, same sign
    return r


@pytest.mark.parametrize("n", [0, 1, 7, 1000003])
def test_cast_bf16_round_to_nearest_even(n):
    say(f"[case] cast n={n}")
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 10.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    if n >= 7:
        # exact ties between neighbouring bf16 values (both parities), zeros, infinities, NaN
        x[:7] = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, np.inf, -np.inf, np.nan,
                          3.0e38], dtype=np.float32)
    g = S.sparse3d_cast(torch.from_numpy(x).to(dev()), torch.bfloat16)
    got = g.view(torch.int16).cpu().numpy().view(np.uint16)
    exp = _bf16_rne_bits(x)
    fin = ~np.isnan(x)
    assert np.array_equal(got[fin], exp[fin])
    assert np.all(np.isnan(g.float().cpu().numpy()[~fin]))
    g32 = S.sparse3d_cast(torch.from_numpy(x).to(dev()), torch.float32)
    assert np.array_equal(g32.cpu().numpy().view(np.uint32)[fin], x.view(np.uint32)[fin])


# --------------------------------------------------------------------------- per-head budgets
def test_per_head_budgets_selection_and_attention():
    w = synth.WORKLOADS["vggt_s8"]
    say("[case] per-head budgets vggt_s8")
    inp = synth.make_inputs(w, seed=3)
    q, v = to_dev(inp.q, tdt(w)), to_dev(inp.v, tdt(w))
    lay = w.layout
    tpf = lay[2] // 64
    ks = [0, 1, 5, 18, 40, 175, 176, 300, 3, 9, 18, 27, 36, 45, 54, 63][: w.heads]
    _, _, _, sc = S.sparse3d_tile_scores(q, q, lay)
    idx, cnt = S.sparse3d_select_topk_per_head(sc, ks, tpf, w.anchor)
    torch.cuda.synchronize()
    ref = oracle_pool_scores(inp, oracle.Layout(*lay), oracle.Layout(*lay))
    g_sc, g_idx, g_cnt = sc.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    Tq = g_sc.shape[1]
    assert g_idx.shape[2] == oracle.kmax_for(g_sc.shape[2], max(ks), tpf, w.anchor)
    for h, kh in enumerate(ks):
        check_selection(g_sc, g_idx, g_cnt, ref["scores"], kh, tpf, w.anchor,
                        rows=[(h, t) for t in range(Tq)])
    # a uniform budget through the per-head entry equals the single-budget entry
    i1, c1 = S.sparse3d_select_topk_per_head(sc, [18] * w.heads, tpf, w.anchor)
    i2, c2 = S.sparse3d_select_topk(sc, 18, tpf, w.anchor)
    assert torch.equal(i1, i2) and torch.equal(c1, c2)
    # attention under the per-head selection
    out, lse = S.sparse3d_sparse_attn_fwd(q, q, v, lay, lay, idx, cnt, out_dtype=torch.float32,
                                          return_lse=True)
    ol = oracle.Layout(*lay)
    pairs = sample_tiles(w.heads, Tq, 40, seed=5)
    rO, rl = oracle.sparse_attend(inp.q, inp.k, inp.v, ol, ol, 64, g_idx, g_cnt, 0.125,
                                  query_tiles=sorted({t for _, t in pairs}))
    compare_outputs(out.cpu().numpy(), rO, pairs, tol=TOL["bf16"], g_lse=lse.cpu().numpy(),
                    ref_lse=rl, lse_tol=LSE_TOL_BF16)


# --------------------------------------------------------------------------- frame attention
def _frame_case(w, seed=0, klay=None, K=None, V=None, frames=None, out_f32=True):
    inp = synth.make_inputs(w, seed=seed)
    dt = tdt(w)
    lay = w.layout
    klay = lay if klay is None else klay
    Kn = inp.k if K is None else K
    Vn = inp.v if V is None else V
    q, k, v = to_dev(inp.q, dt), to_dev(Kn, dt), to_dev(Vn, dt)
    out, lse = S.sparse3d_frame_attn_fwd(q, k, v, lay, klay, return_lse=True,
                                         out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    ref, rl = oracle.frame_attend(inp.q, Kn, Vn, oracle.Layout(*lay), oracle.Layout(*klay), 0.125,
                                  frames=frames)
    return out.float().cpu().numpy(), lse.cpu().numpy(), ref, rl, lay


def _frame_rows(lay, frames):
    S_, N, P, _ = lay
    fs = range(S_) if frames is None else frames
    return np.concatenate([s * P + np.arange(P) for s in fs])


def test_frame_attention_tiny_fp32():
    w = synth.WORKLOADS["tiny_s2"]
    say("[case] frame attention tiny_s2 fp32")
    g, gl, r, rl, lay = _frame_case(w, seed=2)
    assert float(np.max(np.abs(g - r))) <= TOL["f32"]
    qv = (np.arange(g.shape[1]) % lay[2]) < lay[1]
    assert np.allclose(gl[:, qv], rl[:, qv], rtol=0, atol=1e-5)
    assert np.all(g[:, ~qv] == 0)


@pytest.mark.parametrize("out_f32", [True, False])
def test_frame_attention_vggt_s8_bf16(out_f32):
    w = synth.WORKLOADS["vggt_s8"]
    say(f"[case] frame attention vggt_s8 bf16 out_f32={out_f32}")
    g, gl, r, rl, lay = _frame_case(w, seed=1, out_f32=out_f32)
    assert float(np.max(np.abs(g - r))) <= TOL["bf16"]
    qv = (np.arange(g.shape[1]) % lay[2]) < lay[1]
    assert np.all(np.abs(gl[:, qv] - rl[:, qv]) <= LSE_TOL_BF16)
    assert np.all(g[:, ~qv] == 0) and np.all(gl[:, ~qv] == 0)


def test_frame_attention_subsampled_keys():
    w = synth.WORKLOADS["vggt_s8"]
    say("[case] frame attention over 2x2-subsampled keys vggt_s8")
    inp = synth.make_inputs(w, seed=4)
    ol = oracle.Layout(*w.layout)
    K2, V2, kl2 = oracle.subsample_keys(inp.k, inp.v, ol, w.grid, 2, 64)
    g, gl, r, rl, lay = _frame_case(w, seed=4, klay=tuple(kl2), K=K2, V=V2)
    assert float(np.max(np.abs(g - r))) <= TOL["bf16"]


def test_frame_attention_full_s128_sampled_frames():
    w = synth.WORKLOADS["vggt_s128"]
    frames = [0, 1, 63, 127]
    say(f"[case] frame attention vggt_s128 frames {frames}")
    g, gl, r, rl, lay = _frame_case(w, seed=0, frames=frames, out_f32=False)
    rows = _frame_rows(lay, frames)
    assert float(np.max(np.abs(g[:, rows] - r[:, rows]))) <= TOL["bf16"]
    qv = rows[(rows % lay[2]) < lay[1]]
    assert np.all(np.abs(gl[:, qv] - rl[:, qv]) <= LSE_TOL_BF16)


# --------------------------------------------------------------------------- subsample completion
def _sga_inputs(w, seed, window=2):
    inp = synth.make_inputs(w, seed=seed)
    dt = tdt(w)
    q, v = to_dev(inp.q, dt), to_dev(inp.v, dt)
    lay = w.layout
    K2, V2, klay = S.sparse3d_grid_subsample_kv(q, v, lay, w.grid, window)
    ol = oracle.Layout(*lay)
    rK2, rV2, rkl = oracle.subsample_keys(inp.k, inp.v, ol, w.grid, window, 64)
    assert tuple(rkl) == tuple(klay)
    km, vm, n = oracle.discarded_mean(inp.k, inp.v, ol, w.grid, window)
    return inp, q, v, K2, V2, klay, ol, rK2, rV2, (km, vm, n)


@pytest.mark.parametrize("name", ["tiny_s2", "vggt_s8"])
def test_discarded_mean(name):
    w = synth.WORKLOADS[name]
    say(f"[case] discarded mean {name}")
    inp, q, v, *_ , (km, vm, n) = _sga_inputs(w, seed=6)
    gk, gv, gn = S.sparse3d_discarded_mean(q, v, w.layout, w.grid, 2)
    assert gn == n
    assert np.allclose(gk.cpu().numpy(), km, rtol=0, atol=1e-5)
    assert np.allclose(gv.cpu().numpy(), vm, rtol=0, atol=1e-5)
    g2, _, _ = S.sparse3d_discarded_mean(q, v, w.layout, w.grid, 2)
    assert torch.equal(gk, g2)                                  # fixed summation order
    z, _, zn = S.sparse3d_discarded_mean(q, v, w.layout, w.grid, 1)
    assert zn == 0 and torch.count_nonzero(z) == 0             # nothing dropped


@pytest.mark.parametrize("name,diag,mean", [("tiny_s2", True, True), ("vggt_s8", True, True),
                                            ("vggt_s8", True, False), ("vggt_s8", False, True)])
def test_subsample_completion_dense(name, diag, mean):
    w = synth.WORKLOADS[name]
    say(f"[case] subsample completion, dense over kept keys: {name} diag={diag} mean={mean}")
    inp, q, v, K2, V2, klay, ol, rK2, rV2, (km, vm, n) = _sga_inputs(w, seed=7)
    gk, gv, _ = S.sparse3d_discarded_mean(q, v, w.layout, w.grid, 2)
    bias = oracle.sga_mean_bias(n)
    sga = S.Sga(w.grid, 2, k_full=q if diag else None, v_full=v if diag else None,
                kmean=gk if mean else None, vmean=gv if mean else None, mean_bias=bias)
    out, lse = S.sparse3d_dense_attn_fwd(q, K2, V2, w.layout, klay, out_dtype=torch.float32,
                                         return_lse=True, sga=sga)
    rsga = dict(grid=w.grid, window=2, k_full=inp.k if diag else None, v_full=inp.v if diag else None,
                kmean=km if mean else None, vmean=vm, mean_bias=bias)
    rO, rl = oracle.dense_attend(inp.q, rK2, rV2, ol, oracle.Layout(*klay), 0.125, sga=rsga)
    g, gl = out.cpu().numpy(), lse.cpu().numpy()
    qv = oracle.query_rows(ol)
    tol = TOL["f32"] if w.dtype == "f32" else TOL["bf16"]
    ltol = 1e-5 if w.dtype == "f32" else LSE_TOL_BF16
    assert float(np.max(np.abs(g[:, qv] - rO[:, qv]))) <= tol
    assert np.all(np.abs(gl[:, qv] - rl[:, qv]) <= ltol)
    assert np.all(g[:, ~qv] == 0)


def test_subsample_completion_sparse_with_landmarks():
    w = synth.WORKLOADS["vggt_s8"]
    say("[case] subsample completion on the tile-sparse call with landmarks, vggt_s8")
    inp, q, v, K2, V2, klay, ol, rK2, rV2, (km, vm, n) = _sga_inputs(w, seed=8)
    okl = oracle.Layout(*klay)
    _, kbar, vbar, sc = S.sparse3d_tile_scores(q, K2, w.layout, klay, v=V2)
    tpf = klay[2] // 64
    idx, cnt = S.sparse3d_select_topk(sc, 6, tpf, 0)
    gk, gv, _ = S.sparse3d_discarded_mean(q, v, w.layout, w.grid, 2)
    bias = oracle.sga_mean_bias(n)
    sga = S.Sga(w.grid, 2, k_full=q, v_full=v, kmean=gk, vmean=gv, mean_bias=bias)
    out, lse = S.sparse3d_sparse_attn_fwd(q, K2, V2, w.layout, klay, idx, cnt,
                                          kbar=S.sparse3d_cast(kbar, q.dtype),
                                          vbar=S.sparse3d_cast(vbar, q.dtype),
                                          out_dtype=torch.float32, return_lse=True, sga=sga)
    rkbar, kc = oracle.tile_pool(rK2, okl, 64, "key")
    rvbar, _ = oracle.tile_pool(rV2, okl, 64, "key")
    rsga = dict(grid=w.grid, window=2, k_full=inp.k, v_full=inp.v, kmean=km, vmean=vm, mean_bias=bias)
    g_idx, g_cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    rO, rl = oracle.sparse_attend(inp.q, rK2, rV2, ol, okl, 64, g_idx, g_cnt, 0.125, kbar=rkbar,
                                  vbar=rvbar, kcount=kc, sga=rsga)
    g, gl = out.cpu().numpy(), lse.cpu().numpy()
    qv = oracle.query_rows(ol)
    assert float(np.max(np.abs(g[:, qv] - rO[:, qv]))) <= TOL["bf16"]
    assert np.all(np.abs(gl[:, qv] - rl[:, qv]) <= LSE_TOL_BF16)


# --------------------------------------------------------------------------- backward
# Elementwise bound of the backward, derived from where the bf16 path rounds (u = 2^-8 bounds
# one bf16 rounding, relative).  The softmax weights P are recomputed from the forward's lse,
# which its bf16-rounded probabilities move by at most ln(1 + u), and are rounded to bf16 for
# the products: |dP_ij| relative error <= 2u.  D = rowsum(dO * O) reads the stored bf16 O,
# which is within u of the exact output's weights: |dD_i| <= 2u A_D_i.  dS = P (dP - D) is
# rounded to bf16: |d(dS_ij)| <= 3u M_ij with M_ij = P_ij (|dP_ij - D_i| + A_D_i).  The
# products with K, Q, dO take exact bf16 inputs and accumulate in fp32.  Hence
#   |dQ - ref| <= 3u scale sum_j M_ij |K_j|,  |dK - ref| <= 3u scale sum_i M_ij |Q_i|,
#   |dV - ref| <= 2u sum_i P_ij |dO_i|,       |D - ref|  <= 2u A_D_i,
# the sums taken by the oracle in absolute-value arithmetic (``magnitudes``); the test allows
# twice that, plus 1e-6 for fp32 accumulation.  Being worst cases, these bounds can exceed a
# typical gradient, so each tensor must also match in relative Frobenius norm within 2^-5
# (rounding errors of random sign cancel: a simulation of these roundings on the 8-view case
# gives at most 0.0093, while a dropped tile or a missing term moves the norm by several %).
_BWD_U = 2.0 ** -8
_BWD_C = {"dQ": 3.0, "dK": 3.0, "dV": 2.0, "D": 2.0}


def _grad_bound(g, ref, mag, what, rows=None):
    g = g.astype(np.float64)
    if rows is not None:
        g, ref, mag = g[rows], ref[rows], mag[rows]
    name = what if isinstance(what, str) else what[0]
    lim = 2.0 * _BWD_C[name] * _BWD_U * mag + 1e-6
    err = np.abs(g - ref)
    assert np.all(err <= lim), (what, float(np.max(err - lim)), float(np.max(err / lim)))
    nr = float(np.linalg.norm(ref))
    fro = float(np.linalg.norm(g - ref)) / nr if nr > 0 else float(np.linalg.norm(g))
    assert fro <= 2.0 ** -5, (what, fro)
    return float(np.max(err / lim)), fro


def _bwd_setup(w, seed, k=None):
    inp = synth.make_inputs(w, seed=seed)
    q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    lay = w.layout
    tpf = lay[2] // 64
    _, _, _, sc = S.sparse3d_tile_scores(q, q, lay)
    idx, cnt = S.sparse3d_select_topk(sc, w.k if k is None else k, tpf, w.anchor)
    out, lse = S.sparse3d_sparse_attn_fwd(q, q, v, lay, lay, idx, cnt, return_lse=True)
    rng = np.random.default_rng(seed + 100)
    dO = synth.round_bf16(rng.standard_normal(inp.q.shape).astype(np.float32))
    dout = to_dev(dO, torch.bfloat16)
    t_end, t_list = S.sparse3d_selection_transpose(idx, cnt, sc.shape[2])
    dq, dk, dv, delta = S.sparse3d_sparse_attn_bwd(q, q, v, out, dout, lse, lay, lay, idx, cnt, t_end, t_list)
    torch.cuda.synchronize()
    return inp, dO, idx.cpu().numpy(), cnt.cpu().numpy(), t_end, t_list, (dq, dk, dv, delta), out, sc.shape[2]


def test_selection_transpose():
    w = synth.WORKLOADS["vggt_s8"]
    say("[case] selection transpose vggt_s8")
    inp, dO, g_idx, g_cnt, t_end, t_list, *_ , Tk = _bwd_setup(w, seed=11)
    ref = oracle.selection_transpose(g_idx, g_cnt, Tk)
    te, tl = t_end.cpu().numpy(), t_list.cpu().numpy()
    for h in range(g_idx.shape[0]):
        b = 0
        for t in range(Tk):
            e = int(te[h, t])
            assert tl[h, b:e].tolist() == ref[h][t], (h, t)
            b = e


@pytest.mark.parametrize("seed,k", [(12, None), (13, 40), (14, 0)])
def test_backward_vggt_s8(seed, k):
    w = synth.WORKLOADS["vggt_s8"]
    say(f"[case] backward vggt_s8 seed={seed} k={k}")
    inp, dO, g_idx, g_cnt, t_end, t_list, (dq, dk, dv, delta), out, Tk = _bwd_setup(w, seed, k)
    ol = oracle.Layout(*w.layout)
    rdq, rdk, rdv, rD, mag = oracle.sparse_attend_bwd(inp.q, inp.k, inp.v, dO, ol, ol, 64, g_idx, g_cnt,
                                                      0.125, magnitudes=True)
    for n, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv), ("D", delta, rD)):
        worst, fro = _grad_bound(g.cpu().numpy(), r, mag[n], n)
        say(f"  {n}: max err / bound {worst:.3f}, relative Frobenius error {fro:.2e}")
    qv = oracle.query_rows(ol)
    assert np.all(dq.cpu().numpy()[:, ~qv] == 0)
    pad = ~oracle.query_rows(ol)
    assert np.all(dk.cpu().numpy()[:, pad] == 0) and np.all(dv.cpu().numpy()[:, pad] == 0)


def test_backward_nan_pad_and_determinism():
    w = synth.WORKLOADS["vggt_s8"]
    say("[case] backward with NaN pad rows, twice")
    inp = synth.make_inputs(w, seed=15, pad_value=np.nan)
    q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    lay = w.layout
    _, _, _, sc = S.sparse3d_tile_scores(q, q, lay)
    idx, cnt = S.sparse3d_select_topk(sc, 18, lay[2] // 64, 0)
    out, lse = S.sparse3d_sparse_attn_fwd(q, q, v, lay, lay, idx, cnt, return_lse=True)
    dO = np.random.default_rng(16).standard_normal(inp.q.shape).astype(np.float32)
    dO[:, ~oracle.query_rows(oracle.Layout(*lay))] = np.nan           # the cotangent's pad may hold NaN too
    dout = to_dev(dO, torch.bfloat16)
    t_end, t_list = S.sparse3d_selection_transpose(idx, cnt, sc.shape[2])
    r1 = S.sparse3d_sparse_attn_bwd(q, q, v, out, dout, lse, lay, lay, idx, cnt, t_end, t_list)
    r2 = S.sparse3d_sparse_attn_bwd(q, q, v, out, dout, lse, lay, lay, idx, cnt, t_end, t_list)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
        assert not torch.isnan(a).any()


def test_backward_full_s128_sampled():
    w = synth.WORKLOADS["vggt_s128"]
    say("[case] backward vggt_s128 (k=138), sampled query and key tiles")
    inp, dO, g_idx, g_cnt, t_end, t_list, (dq, dk, dv, delta), out, Tk = _bwd_setup(w, seed=0, k=138)
    ol = oracle.Layout(*w.layout)
    H, Tq = g_idx.shape[0], g_idx.shape[1]
    pairs = sample_tiles(H, Tq, 6, seed=3)
    for (h, t) in pairs:                                             # dQ of sampled query tiles
        rdq, _, _, rD, mag = oracle.sparse_attend_bwd(inp.q, inp.k, inp.v, dO, ol, ol, 64, g_idx, g_cnt, 0.125,
                                                      query_tiles=[t], heads=[h], magnitudes=True)
        r = slice(t * 64, (t + 1) * 64)
        if not np.any(oracle.query_rows(ol)[r]):
            continue
        _grad_bound(dq[h, r].cpu().numpy(), rdq[h, r], mag["dQ"][h, r], ("dQ", h, t))
        _grad_bound(delta[h, r].cpu().numpy(), rD[h, r], mag["D"][h, r], ("D", h, t))
    te = t_end.cpu().numpy()
    tl = t_list.cpu().numpy()
    tpf = w.layout[2] // 64
    key_pairs = [(h, t) for (h, t) in sample_tiles(H, Tk, 4, seed=4) if t >= tpf]   # not the anchor frame
    for (h, t) in key_pairs:                                         # dK, dV of sampled key tiles
        b = 0 if t == 0 else int(te[h, t - 1])
        qt = tl[h, b:int(te[h, t])].tolist()
        _, rdk, rdv, _, mag = oracle.sparse_attend_bwd(inp.q, inp.k, inp.v, dO, ol, ol, 64, g_idx, g_cnt, 0.125,
                                                       query_tiles=qt, heads=[h], magnitudes=True)
        j = np.arange(t * 64, (t + 1) * 64)
        mem = j[oracle.member_rows(ol)[j]]
        _grad_bound(dk[h, mem].cpu().numpy(), rdk[h, mem], mag["dK"][h, mem], ("dK", h, t))
        _grad_bound(dv[h, mem].cpu().numpy(), rdv[h, mem], mag["dV"][h, mem], ("dV", h, t))


# ----------------------------------------------------------------- backward with landmarks
# The landmark keys are the tile means kbar/vbar, rounded to bf16 once (the precision the
# matrix cores read) and handed to both sides, so the bound above covers them unchanged: a
# landmark column enters dQ, D and its own gradients exactly like a key, dkbar like dK
# (constant 3) and dvbar like dV (constant 2); the chain into member rows divides by the
# member count in fp32, and the oracle's magnitudes carry the same chain.
_BWD_C.update({"dkbar": 3.0, "dvbar": 2.0})


def _bwd_lm_setup(w, seed, k=None):
    inp = synth.make_inputs(w, seed=seed)
    q, v = to_dev(inp.q, torch.bfloat16), to_dev(inp.v, torch.bfloat16)
    lay = w.layout
    ol = oracle.Layout(*lay)
    tpf = lay[2] // 64
    kb, kc = oracle.tile_pool(inp.k, ol, 64, "key")
    vb, _ = oracle.tile_pool(inp.v, ol, 64, "key")
    kb16 = synth.round_bf16(kb.astype(np.float32))
    vb16 = synth.round_bf16(vb.astype(np.float32))
    kbar, vbar = to_dev(kb16, torch.bfloat16), to_dev(vb16, torch.bfloat16)
    _, _, _, sc = S.sparse3d_tile_scores(q, q, lay)
    idx, cnt = S.sparse3d_select_topk(sc, w.k if k is None else k, tpf, w.anchor)
    out, lse = S.sparse3d_sparse_attn_fwd(q, q, v, lay, lay, idx, cnt, kbar=kbar, vbar=vbar, return_lse=True)
    rng = np.random.default_rng(seed + 100)
    dO = synth.round_bf16(rng.standard_normal(inp.q.shape).astype(np.float32))
    dout = to_dev(dO, torch.bfloat16)
    t_end, t_list = S.sparse3d_selection_transpose(idx, cnt, sc.shape[2])
    grads = S.sparse3d_sparse_attn_bwd(q, q, v, out, dout, lse, lay, lay, idx, cnt, t_end, t_list,
                                       kbar=kbar, vbar=vbar)
    torch.cuda.synchronize()
    means = dict(kbar=kb16.astype(np.float64), vbar=vb16.astype(np.float64), kcount=kc)
    return inp, dO, idx.cpu().numpy(), cnt.cpu().numpy(), t_end, t_list, grads, means, ol


def _sum_invariants(dO, ol, dk, dv):
    """Whole-tensor properties of the gradients that hold at any size (pinned on the oracle):
    every valid row's softmax weights sum to 1, so the value gradients of all keys (landmark
    means included, through the chain into member rows) sum to the cotangents of the valid
    rows, and the rows of dS sum to 0, so the key gradients sum to 0.  Rounding errors of
    random sign stay far below 2^-5 of the norm of what is summed; a key block or the chain
    left out moves the sums by a sizeable fraction of it."""
    qv = oracle.query_rows(ol)
    for h in range(dk.shape[0]):
        g = dO[h][qv].astype(np.float64)
        want_v, got_v = g.sum(axis=0), dv[h].astype(np.float64).sum(axis=0)
        tol_v = 2.0 ** -5 * np.sqrt((g ** 2).sum(axis=0))
        assert np.all(np.abs(got_v - want_v) <= tol_v), (h, float(np.max(np.abs(got_v - want_v) / tol_v)))
        kk = dk[h].astype(np.float64)
        got_k, tol_k = kk.sum(axis=0), 2.0 ** -5 * np.sqrt((kk ** 2).sum(axis=0))
        assert np.all(np.abs(got_k) <= tol_k), (h, float(np.max(np.abs(got_k) / tol_k)))


@pytest.mark.parametrize("seed,k,heads", [(21, None, None), (22, 0, [0, 5]), (23, 60, [3, 9])])
def test_backward_landmarks_vggt_s8(seed, k, heads):
    # heads = None: every head; otherwise those heads, each complete
    w = synth.WORKLOADS["vggt_s8"]
    say(f"[case] backward with landmarks vggt_s8 seed={seed} k={k} heads={heads}")
    inp, dO, g_idx, g_cnt, *_, grads, means, ol = _bwd_lm_setup(w, seed, k)
    dq, dk, dv, delta, dkbar, dvbar = (x.cpu().numpy() for x in grads)
    rdq, rdk, rdv, rD, rdkb, rdvb, mag = oracle.sparse_attend_bwd(
        inp.q, inp.k, inp.v, dO, ol, ol, 64, g_idx, g_cnt, 0.125, **means, heads=heads, means=True,
        magnitudes=True)
    hs = list(range(w.heads)) if heads is None else heads
    for n, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv), ("D", delta, rD),
                    ("dkbar", dkbar, rdkb), ("dvbar", dvbar, rdvb)):
        worst, fro = _grad_bound(g[hs], r[hs], mag[n][hs], n)
        say(f"  {n}: max err / bound {worst:.3f}, relative Frobenius error {fro:.2e}")
    qv = oracle.query_rows(ol)
    assert np.all(dq[:, ~qv] == 0) and np.all(dk[:, ~qv] == 0) and np.all(dv[:, ~qv] == 0)
    empty = means["kcount"] == 0
    assert np.all(dkbar[:, empty] == 0) and np.all(dvbar[:, empty] == 0)
    _sum_invariants(dO, ol, dk, dv)


def test_backward_landmarks_vggt_s32_one_head():
    # 32 views at about 90 % sparsity: 704 query tiles per head with ragged member ranges;
    # head 1 checked completely (every query tile contributes to its key and mean gradients)
    w = synth.WORKLOADS["vggt_s32"]
    say("[case] backward with landmarks vggt_s32 (k=45), head 1 complete")
    inp, dO, g_idx, g_cnt, *_, grads, means, ol = _bwd_lm_setup(w, seed=24, k=45)
    ref = oracle.sparse_attend_bwd(inp.q, inp.k, inp.v, dO, ol, ol, 64, g_idx, g_cnt, 0.125, **means,
                                   heads=[1], means=True, magnitudes=True)
    rdq, rdk, rdv, rD, rdkb, rdvb, mag = ref
    for n, g, r in zip(("dQ", "dK", "dV", "D", "dkbar", "dvbar"), grads, (rdq, rdk, rdv, rD, rdkb, rdvb)):
        worst, fro = _grad_bound(g[1].cpu().numpy(), r[1], mag[n][1], n)
        say(f"  {n}: max err / bound {worst:.3f}, relative Frobenius error {fro:.2e}")
    _sum_invariants(dO, ol, grads[1].cpu().numpy(), grads[2].cpu().numpy())


@pytest.mark.timeout(300)
def test_backward_landmarks_full_s256_sampled():
    # 256 views, about 96 % sparsity with landmarks (k = 180 of 5632 tiles): dQ and D on
    # sampled query tiles; on sampled key tiles the direct part of dK/dV (what the chain did
    # not add: the query tiles that selected a tile never see its mean); the means' gradients
    # through the whole-tensor sums.  The oracle's inputs at this size take most of the time.
    w = synth.WORKLOADS["vggt_s256_lm"]
    say("[case] backward with landmarks vggt_s256_lm (k=180), sampled tiles + sums")
    inp, dO, g_idx, g_cnt, t_end, t_list, grads, means, ol = _bwd_lm_setup(w, seed=0, k=180)
    dq, dk, dv, delta, dkbar, dvbar = grads
    H, Tq = g_idx.shape[0], g_idx.shape[1]
    pairs = sample_tiles(H, Tq, 6, seed=5)
    hs, ts = sorted({h for h, _ in pairs}), sorted({t for _, t in pairs})
    rdq, _, _, rD, mag = oracle.sparse_attend_bwd(inp.q, inp.k, inp.v, dO, ol, ol, 64, g_idx, g_cnt, 0.125,
                                                  **means, query_tiles=ts, heads=hs, magnitudes=True)
    for (h, t) in pairs:
        r = slice(t * 64, (t + 1) * 64)
        _grad_bound(dq[h, r].cpu().numpy(), rdq[h, r], mag["dQ"][h, r], ("dQ", h, t))
        _grad_bound(delta[h, r].cpu().numpy(), rD[h, r], mag["D"][h, r], ("D", h, t))
    say("  dQ, D: sampled query tiles ok")
    del rdq, rD, mag
    te, tl = t_end.cpu().numpy(), t_list.cpu().numpy()
    tpf = w.layout[2] // 64
    kc = means["kcount"]
    for (h, t) in [(2, 3 * tpf + 7), (H - 1, Tq - 2)]:            # not the anchor frame
        b = 0 if t == 0 else int(te[h, t - 1])
        qt = tl[h, b:int(te[h, t])].tolist()
        _, rdk, rdv, _, mag = oracle.sparse_attend_bwd(inp.q, inp.k, inp.v, dO, ol, ol, 64, g_idx, g_cnt, 0.125,
                                                       **means, query_tiles=qt, heads=[h], magnitudes=True)
        j = np.arange(t * 64, (t + 1) * 64)
        mem = j[oracle.member_rows(ol)[j]]
        gk = dk[h, mem].cpu().numpy().astype(np.float64) - dkbar[h, t].cpu().numpy().astype(np.float64) / kc[t]
        gv = dv[h, mem].cpu().numpy().astype(np.float64) - dvbar[h, t].cpu().numpy().astype(np.float64) / kc[t]
        _grad_bound(gk, rdk[h, mem], mag["dK"][h, mem], ("dK", h, t))
        _grad_bound(gv, rdv[h, mem], mag["dV"][h, mem], ("dV", h, t))
        del rdk, rdv, mag
    say("  dK, dV: direct part on sampled key tiles ok")
    _sum_invariants(dO, ol, dk.cpu().numpy(), dv.cpu().numpy())
    say("  sums of dK, dV ok")


# ----------------------------------------------------------------- output bounds (canaries)
_GUARD = 4096
_PAT = 0xA5


class _Guarded:
    """An output buffer of `nbytes` between two guard regions of a known byte pattern."""

    def __init__(self, nbytes):
        self.n = int(nbytes)
        self.buf = torch.full((self.n + 2 * _GUARD,), _PAT, dtype=torch.uint8, device=dev())

    @property
    def ptr(self):
        return self.buf.data_ptr() + _GUARD

    def check(self, name):
        b = self.buf.cpu().numpy()
        assert np.all(b[:_GUARD] == _PAT), f"{name}: bytes written before the buffer"
        assert np.all(b[_GUARD + self.n:] == _PAT), f"{name}: bytes written past the buffer"
        assert np.any(b[_GUARD:_GUARD + self.n] != _PAT), f"{name}: nothing written"


def test_outputs_stay_inside_their_buffers():
    # every entry point, called through the C ABI on one small ragged layer (4 views of 1374
    # tokens, 2 heads, landmarks on), writes only inside the output buffers it was given
    say("[case] canary guards around every output")
    import ctypes
    lib = S.library()
    H, d = 2, 64
    lay = (4, 1374, 1408, 5)
    L = lay[0] * lay[2]
    Tq = Tk = L // 64
    tpf = lay[2] // 64
    k, anchor = 12, 0
    kmax = S.kmax_for(Tk, k, tpf, anchor)
    rng = np.random.default_rng(31)
    q = to_dev(rng.standard_normal((H, L, d)).astype(np.float32), torch.bfloat16)
    v = to_dev(rng.standard_normal((H, L, d)).astype(np.float32), torch.bfloat16)
    dout = to_dev(rng.standard_normal((H, L, d)).astype(np.float32), torch.bfloat16)
    st = torch.cuda.current_stream().cuda_stream
    ql = S._Layout(*lay)
    rl = ctypes.byref(ql)
    g = {n: _Guarded(b) for n, b in dict(
        qbar=H * Tq * d * 4, kbar=H * Tk * d * 4, vbar=H * Tk * d * 4, scores=H * Tq * Tk * 4,
        idx=H * Tq * kmax * 4, cnt=H * Tq * 4, idx_h=H * Tq * kmax * 4, cnt_h=H * Tq * 4,
        kb16=H * Tk * d * 2, vb16=H * Tk * d * 2, out=H * L * d * 2, lse=H * L * 4,
        dense_out=H * L * d * 4, dense_lse=H * L * 4, frame_out=H * L * d * 2, frame_lse=H * L * 4,
        t_end=H * Tk * 4, t_list=H * Tq * kmax * 4, dq=H * L * d * 4, dk=H * L * d * 4, dv=H * L * d * 4,
        delta=H * L * 4, dkbar=H * Tk * d * 4, dvbar=H * Tk * d * 4, kmean=H * d * 4, vmean=H * d * 4,
        kop=H * Tk * d * 2, vop=H * Tk * d * 2).items()}
    P = {n: x.ptr for n, x in g.items()}
    ok = lambda status: S._check(status)
    ok(lib.sparse3d_tile_scores(q.data_ptr(), q.data_ptr(), v.data_ptr(), S.BF16, H, d, 64, rl, rl, 0.125,
                                P["qbar"], P["kbar"], P["vbar"], P["scores"], P["kop"], P["vop"], st))
    ok(lib.sparse3d_select_topk(P["scores"], H, Tq, Tk, k, tpf, anchor, P["idx"], P["cnt"], kmax, st))
    kh = (ctypes.c_int32 * H)(k, k - 5)
    ok(lib.sparse3d_select_topk_per_head(P["scores"], H, Tq, Tk, kh, tpf, anchor, P["idx_h"], P["cnt_h"], kmax, st))
    ok(lib.sparse3d_cast(P["kbar"], H * Tk * d, S.BF16, P["kb16"], st))
    ok(lib.sparse3d_cast(P["vbar"], H * Tk * d, S.BF16, P["vb16"], st))
    ok(lib.sparse3d_sparse_attn_fwd(q.data_ptr(), q.data_ptr(), v.data_ptr(), S.BF16, H, d, 64, rl, rl, P["idx"],
                                    P["cnt"], kmax, P["kb16"], P["vb16"], math.log(64.0), 0.125, None, P["out"],
                                    S.BF16, P["lse"], st))
    ok(lib.sparse3d_dense_attn_fwd(q.data_ptr(), q.data_ptr(), v.data_ptr(), S.BF16, H, d, rl, rl, 0.125, None,
                                   P["dense_out"], S.F32, P["dense_lse"], st))
    ok(lib.sparse3d_frame_attn_fwd(q.data_ptr(), q.data_ptr(), v.data_ptr(), S.BF16, H, d, rl, rl, 0.125,
                                   P["frame_out"], S.BF16, P["frame_lse"], st))
    ok(lib.sparse3d_selection_transpose(P["idx"], P["cnt"], H, Tq, Tk, kmax, P["t_end"], P["t_list"], st))
    ok(lib.sparse3d_sparse_attn_bwd(q.data_ptr(), q.data_ptr(), v.data_ptr(), P["out"], dout.data_ptr(), P["lse"],
                                    S.BF16, H, d, 64, rl, rl, P["idx"], P["cnt"], kmax, P["t_end"], P["t_list"],
                                    P["kb16"], P["vb16"], math.log(64.0), 0.125, P["dq"], P["dk"], P["dv"],
                                    P["delta"], P["dkbar"], P["dvbar"], st))
    ok(lib.sparse3d_discarded_mean(q.data_ptr(), v.data_ptr(), S.BF16, H, d, rl, 37, 37, 2, P["kmean"],
                                   P["vmean"], st))
    sl = S._Layout()
    ok(lib.sparse3d_subsample_layout(rl, 37, 37, 2, 64, ctypes.byref(sl)))
    rows_out = sl.frames * sl.stride
    ko, vo = _Guarded(H * rows_out * d * 2), _Guarded(H * rows_out * d * 2)
    ok(lib.sparse3d_grid_subsample_kv(q.data_ptr(), v.data_ptr(), S.BF16, H, d, rl, 37, 37, 2, ko.ptr, vo.ptr,
                                      ctypes.byref(sl), st))
    torch.cuda.synchronize()
    for n, x in g.items():
        x.check(n)
    ko.check("k_out")
    vo.check("v_out")
    # the pooling pass's operand-dtype means equal the cast of its fp32 means, bit for bit
    for a, b in (("kop", "kb16"), ("vop", "vb16")):
        assert torch.equal(g[a].buf[_GUARD:_GUARD + g[a].n], g[b].buf[_GUARD:_GUARD + g[b].n]), a


def test_rejected_calls_launch_nothing():
    # every wrapper checks shapes and dtypes of device tensors before it touches the device,
    # and a call the library refuses writes nothing (its output keeps a sentinel)
    say("[case] rejected calls on device tensors")
    import ctypes
    d = dev()
    lay = (2, 256, 256, 0)
    q = torch.randn((2, 512, 64), device=d).to(torch.bfloat16)
    sc = torch.zeros((2, 8, 8), device=d)
    idx = torch.zeros((2, 8, 8), dtype=torch.int32, device=d)
    cnt = torch.full((2, 8), 4, dtype=torch.int32, device=d)
    with pytest.raises(ValueError):
        S.sparse3d_tile_scores(q, q[:, :448].contiguous(), lay)               # k shorter than its layout
    with pytest.raises(TypeError):
        S.sparse3d_tile_scores(q, q.float(), lay)                            # k dtype differs from q
    with pytest.raises(TypeError):
        S.sparse3d_select_topk(sc.double(), 4, 4, 0)                         # scores must be fp32
    with pytest.raises(TypeError):
        S.sparse3d_sparse_attn_fwd(q, q, q, lay, lay, idx.long(), cnt)       # idx must be int32
    with pytest.raises(ValueError):
        S.sparse3d_sparse_attn_fwd(q, q, q, lay, lay, idx, cnt[:, :7].contiguous())
    with pytest.raises(ValueError):
        S.sparse3d_dense_attn_fwd(q, q, q[:, :500].contiguous(), lay)
    with pytest.raises(ValueError, match="kbar and vbar"):
        S.sparse3d_sparse_attn_fwd(q, q, q, lay, lay, idx, cnt, kbar=torch.zeros((2, 8, 64), device=d, dtype=q.dtype))
    lse = torch.zeros((2, 512), device=d)
    with pytest.raises(ValueError):
        S.sparse3d_sparse_attn_bwd(q, q, q, q, q, lse[:, :511].contiguous(), lay, lay, idx, cnt,
                                   torch.zeros((2, 8), dtype=torch.int32, device=d),
                                   torch.zeros((2, 64), dtype=torch.int32, device=d))
    torch.cuda.synchronize()
    # the C ABI with real device buffers: refused calls leave the output untouched
    lib = S.library()
    out = torch.full((2, 512, 64), 7.0, device=d)
    ql = S._Layout(*lay)
    rl = ctypes.byref(ql)
    st = torch.cuda.current_stream().cuda_stream
    bad = [
        dict(scale=0.0, out=out.data_ptr(), status=3),                # scale must be > 0
        dict(scale=0.125, out=q.data_ptr(), status=5),                # out aliases q
        dict(scale=float("nan"), out=out.data_ptr(), status=3),
    ]
    for b in bad:
        r = lib.sparse3d_sparse_attn_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), S.BF16, 2, 64, 64, rl, rl,
                                         idx.data_ptr(), cnt.data_ptr(), 8, None, None, math.log(64.0), b["scale"],
                                         None, b["out"], S.F32, None, st)
        assert r == b["status"], (b, r)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    # and a valid call afterwards still runs
    o = S.sparse3d_sparse_attn_fwd(q, q, q, lay, lay, idx, cnt)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
