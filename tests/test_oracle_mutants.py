"""Planted mistakes in copies of the oracle must each be caught by some pin.

The mistakes are the plausible ones: a dropped term, a wrong sign, index or
constant, a transposed operand.  Each mutant is a fresh module built from the
oracle's source with one textual change; the real oracle is never modified.
"""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "sparse3d_oracle.py")

MUTANTS = {
    "landmark_bias_ln63": ("LN64 = math.log(64.0)", "LN64 = math.log(63.0)"),
    "key_pool_keeps_specials": ("return (j >= lay.specials) & (j < lay.tokens)",
                                "return (j < lay.tokens)"),
    "query_pool_drops_specials": ("return _inframe(lay) < lay.tokens\n\n\ndef member_rows",
                                  "return (_inframe(lay) < lay.tokens) & (_inframe(lay) >= lay.specials)\n\n\ndef member_rows"),
    "ties_to_higher_index": ("np.lexsort((np.arange(Tk), -row))", "np.lexsort((-np.arange(Tk), -row))"),
    "smallest_scores": ("np.lexsort((np.arange(Tk), -row))", "np.lexsort((np.arange(Tk), row))"),
    "specials_dropped": ("keys = [spec] + ", "keys = [spec[:0]] + "),
    "scores_transposed": ("np.matmul(qbar, np.swapaxes(kbar, 1, 2))", "np.matmul(kbar, np.swapaxes(qbar, 1, 2))"),
    "landmark_unscaled": ("scale * (q @ kbar[h, lm].T) + landmark_bias", "(q @ kbar[h, lm].T) + landmark_bias"),
    "anchor_short": ("(anchor + 1) * tiles_per_frame)\n", "(anchor + 1) * tiles_per_frame - 1)\n"),
    "landmarks_include_selected": ("~chosen & (kcount > 0))[0]\n                logits", "(kcount > 0))[0]\n                logits"),
    "dense_reads_pad": ("return _inframe(lay) < lay.tokens\n\n\n# ---", "return _inframe(lay) <= lay.tokens\n\n\n# ---"),
    "lse_without_log": ("(m + np.log(den))[:, 0]", "(m + den)[:, 0]"),
    "subsample_odd_rows": ("for y in range(0, gh, window)", "for y in range(1, gh, window)"),
    "empty_tiles_not_masked": ("sig[:, :, kcount == 0] = -np.inf", "pass"),
    "mean_over_tile_size": ("mean[h, nz] = s[nz] / count[nz, None]", "mean[h, nz] = s[nz] / Xh.shape[1]"),
    "per_head_budget_ignored": ("select_tiles(scores[h, t], ks[h], tiles_per_frame, anchor)",
                                "select_tiles(scores[h, t], ks[0], tiles_per_frame, anchor)"),
    "frame_keys_from_next_frame": ("J = s * klay.stride + np.arange(klay.tokens)",
                                   "J = ((s + 1) % klay.frames) * klay.stride + np.arange(klay.tokens)"),
    "frame_keys_skip_specials": ("J = s * klay.stride + np.arange(klay.tokens)",
                                 "J = s * klay.stride + np.arange(klay.specials, klay.tokens)"),
    "sga_diag_on_kept_positions": ('drop[discarded_positions(qlay.specials, sga["grid"], sga["window"])] = True',
                                   "drop[qlay.specials:qlay.tokens] = True"),
    "sga_mean_without_bias": ('ml = scale * (q @ sga["kmean"][h]) + sga["mean_bias"]',
                              'ml = scale * (q @ sga["kmean"][h])'),
    "sga_mean_over_all_patches": ("if y % window or x % window]", "if True]"),
    "sga_bias_count_plus_one": ("return math.log(count)", "return math.log(count + 1)"),
    "mask_ties_to_higher_index": ("out[h] = above | (tie & (np.cumsum(tie, axis=1) <= room[:, None]))",
                                  "out[h] = above | (tie & (np.cumsum(tie[:, ::-1], axis=1)[:, ::-1] <= room[:, None]))"),
    "mask_takes_every_tie": ("out[h] = above | (tie & (np.cumsum(tie, axis=1) <= room[:, None]))",
                             "out[h] = above | tie"),
    "bwd_without_rowsum": ("ds = p * (dp - Di[:, None])", "ds = p * dp"),
    "bwd_dk_unscaled": ("gk, gv = scale * (ds.T @ q), p.T @ g", "gk, gv = ds.T @ q, p.T @ g"),
    "bwd_dv_from_ds": ("gk, gv = scale * (ds.T @ q), p.T @ g", "gk, gv = scale * (ds.T @ q), ds.T @ g"),
    "bwd_landmark_mean_not_divided": ("dK[h, rows_t[t]] += dkb[h, t] / kcount[t]",
                                      "dK[h, rows_t[t]] += dkb[h, t]"),
    "bwd_landmark_bias_dropped": ("s = scale * (q @ kk.T) + bias", "s = scale * (q @ kk.T)"),
    "bwd_landmark_value_grad_lost": ("dvb[h, lm] += gv[J.size:]", "pass"),
    "bwd_landmarks_include_selected": ("lm = np.nonzero(~chosen & (kcount > 0))[0]\n                kk = ",
                                       "lm = np.nonzero(kcount > 0)[0]\n                kk = "),
    "bwd_dq_transposed_keys": ("dQ[h, rows_q] = scale * (ds @ kk)", "dQ[h, rows_q] = scale * (ds @ vv)"),
    "transpose_drops_first": ("            for t in idx[h, tq, : cnt[h, tq]]:\n                out[h][int(t)].append(tq)",
                              "            for t in idx[h, tq, 1: cnt[h, tq]]:\n                out[h][int(t)].append(tq)"),
    "sga_diag_value_from_key": ('np.nan_to_num(sga["v_full"][h, rows_q].astype(np.float64))',
                                'np.nan_to_num(sga["k_full"][h, rows_q].astype(np.float64))'),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:
            return
    pytest.fail(f"planted mistake {name!r} passed every oracle pin")
