"""Host-side bookkeeping of the layer (no GPU): pseudo-tiles, sparsity, k calibration, FLOPs."""
import numpy as np

from dynamic_block_sparse_tile_amd import layer as LY


def test_special_tiles_and_tpf():
    assert LY.special_tiles((128, 1374, 1408, 5)) == 10
    assert LY.special_tiles((256, 1374, 1408, 5)) == 20
    assert LY.special_tiles((8, 1374, 1408, 5)) == 1
    assert LY.special_tiles((2, 256, 256, 0)) == 0
    assert LY.tiles_per_frame((128, 1374, 1408, 5)) == 22


def test_measured_sparsity():
    # 10 pseudo-tiles + 159 selected of 2816 -> 94.0 %
    assert abs(LY.measured_sparsity(159 * 100, 100, 10, 2816) - (1 - 169 / 2816)) < 1e-12


def test_calibrate_k_monotone_search():
    rng = np.random.default_rng(0)
    for trial in range(50):
        tk = int(rng.integers(5, 400))
        rows = int(rng.integers(1, 50))
        ts = int(rng.integers(0, 4))
        # selection size per row: k plus a data-dependent overlap with 'anchor' tiles, capped
        extra = rng.integers(0, 6, size=rows)
        count = lambda k: int(np.minimum(k + np.where(k > 0, extra, extra), tk).sum())
        target = float(rng.uniform(0.0, 1.0))
        k = LY.calibrate_k(count, rows, ts, tk, target)
        sp = lambda kk: LY.measured_sparsity(count(kk), rows, ts, tk)
        best = min(range(tk + 1), key=lambda kk: (abs(sp(kk) - target), -sp(kk)))
        assert abs(sp(k) - target) <= abs(sp(best) - target) + 1e-12


def test_flops():
    assert LY.pair_flops() == 4 * 64 ** 3 == 1048576
    assert LY.selected_flops(total_cnt=5, rows=2, ts=1) == 7 * 1048576
    assert LY.selected_flops(total_cnt=0, rows=1, ts=0, landmarks=10) == 10 * 64 * 4 * 64


def test_valid_pair_flops_brute_force():
    # two frames of N=150 tokens (3 specials) padded to P=192: three 64-row tiles per frame
    S, N, P, nsp = 2, 150, 192, 3
    lay = (S, N, P, nsp)
    rng = np.random.default_rng(5)
    Tq = Tk = S * P // 64
    kmax = 4
    idx = np.full((2, Tq, kmax), -1, np.int32)
    cnt = np.zeros((2, Tq), np.int32)
    for h in range(2):
        for t in range(Tq):
            c = int(rng.integers(0, kmax + 1))
            idx[h, t, :c] = np.sort(rng.choice(Tk, c, replace=False))
            cnt[h, t] = c
    total = 0
    for h in range(2):
        for tq in range(Tq):
            for r in range(64):
                pos = (tq % 3) * 64 + r                      # in-frame position of the query row
                if pos >= N:
                    continue
                keys = S * nsp                                 # every frame's special tokens
                for t in idx[h, tq, :cnt[h, tq]]:
                    for kr in range(64):
                        kpos = (t % 3) * 64 + kr
                        keys += nsp <= kpos < N                # patch tokens of the tile only
                total += keys
    assert LY.valid_pair_flops(idx, cnt, lay, lay) == total * 4 * 64


def test_special_row_quotient_by_fp64_fma():
    # The bf16 attention kernel finds the frame of special token e (e // nsp) as
    # trunc(fma(e, fl(1/nsp), fl(1/nsp) / 2)) in fp64.  The fma is replayed exactly (the exact
    # rational e * inv + inv / 2, rounded once to the nearest double), on the e where a
    # truncation would first go wrong, just below and at every multiple of nsp, up to 2^31.
    from fractions import Fraction
    rng = np.random.default_rng(3)
    for nsp in [1, 2, 3, 5, 7, 64, 70, 127, 1000, 65535, 1 << 20, (1 << 30) + 7]:
        inv = 1.0 / nsp
        half = inv * 0.5
        qs = np.unique(np.concatenate([np.arange(1, 200), rng.integers(1, max(2, (1 << 31) // nsp), 300),
                                       [(1 << 31) // nsp - 1]]))
        for q in qs:
            for e in (int(q) * nsp - 1, int(q) * nsp):
                if not 0 <= e < (1 << 31):
                    continue
                f = float(Fraction(e) * Fraction(inv) + Fraction(half))
                assert int(f) == e // nsp, (nsp, e)
