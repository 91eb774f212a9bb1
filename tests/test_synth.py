"""The seeded generator: determinism, dtype rounding, shapes and planted structure."""
import numpy as np
import torch

from dynamic_block_sparse_tile_amd import synth


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1e-40, -3.0e38, 65504.0, 1.00390625, 1.01171875],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(synth.round_bf16(x).view(np.uint32), want.view(np.uint32))


def test_deterministic_and_shapes():
    w = synth.with_frames(synth.WORKLOADS["vggt_s32"], 3, heads=2)
    a = synth.make_inputs(w, seed=5)
    b = synth.make_inputs(w, seed=5)
    c = synth.make_inputs(w, seed=6)
    assert a.q.shape == (2, 3 * 1408, 64) and a.v.shape == a.q.shape
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    assert not np.array_equal(a.q, c.q)
    assert a.q is a.k                               # one draw serves Q and K
    # bf16-representable values; pad rows zero
    assert np.array_equal(synth.round_bf16(a.q), a.q)
    j = np.arange(a.q.shape[1]) % 1408
    assert np.all(a.q[:, j >= 1374] == 0) and np.all(a.v[:, j >= 1374] == 0)
    assert np.all(a.shifts[0] == 0) and np.all(np.abs(a.shifts) <= 4)


def test_nan_pad():
    w = synth.with_frames(synth.WORKLOADS["vggt_s8"], 2, heads=1)
    a = synth.make_inputs(w, seed=1, pad_value=np.nan)
    j = np.arange(a.q.shape[1]) % 1408
    assert np.all(np.isnan(a.q[:, j >= 1374])) and np.all(np.isfinite(a.q[:, j < 1374]))


def test_planted_correspondences():
    """Corresponding patches of two frames share a latent: their Q rows are close."""
    w = synth.with_frames(synth.WORKLOADS["vggt_s32"], 2, heads=1, noise=0.0)
    a = synth.make_inputs(w, seed=9)
    dy, dx = a.shifts[1]
    P, nsp = 1408, 5
    for (y, x) in [(0, 0), (10, 20), (36, 36)]:
        # frame 1 patch (y, x) uses latent ((y+dy)%37, (x+dx)%37) = frame 0 patch there
        r1 = P + nsp + y * 37 + x
        r0 = nsp + ((y + dy) % 37) * 37 + (x + dx) % 37
        assert np.array_equal(a.q[0, r1], a.q[0, r0])


def test_frame_unique_patches():
    w = synth.with_frames(synth.WORKLOADS["vggt_s128"], 3, heads=1, noise=0.0)
    a = synth.make_inputs(w, seed=2)
    P, nsp = 1408, 5
    f0 = a.q[0, nsp:1374]
    f1 = a.q[0, P + nsp:P + 1374]
    # every frame-0 row is matched by frame-1 rows except for the unique ones (both sides)
    s0 = {r.tobytes() for r in f0}
    matched = sum(r.tobytes() in s0 for r in f1)
    assert 1369 - 2 * 274 <= matched <= 1369 - 274


def test_workload_table():
    for name, w in synth.WORKLOADS.items():
        assert w.stride % w.tile == 0 and w.tokens <= w.stride and w.specials < w.tokens
        assert w.head_dim == 64 and w.tile == 64
    t = synth.WORKLOADS["tiny_s2"]
    assert (t.frames, t.tokens, t.heads, t.dtype, t.k) == (2, 256, 2, "f32", 4)
