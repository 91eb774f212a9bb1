"""The counter reader of bench.py on small hand-made rocprofv3 outputs (no GPU): scaling of
the byte counters by the copy reference, GB/s, clock, matrix-core busy share, FLOP rate."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

ATTN = "void s3d::k_attn_bf16<false, false, false, false, 1>(s3d::AttnDev)"
POOLQ = "void s3d::k_tile_pool<true, false>(void const*, int, s3d::Lay, float*)"
POOLK = "void s3d::k_tile_pool<true, true>(void const*, int, s3d::Lay, float*)"
SEL = "void s3d::k_select_topk_wave<44, true>(float const*, int)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctor_add<float> >(int)"
BWD = "void s3d::k_attn_bwd_dq<false>(s3d::BwdDev)"


def _pmc(path, rows):
    os.makedirs(path)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for r in rows:
            w.writerow(r)


def test_counter_reader(tmp_path, monkeypatch):
    d = tmp_path / "prof"
    os.makedirs(d / "trace")
    with open(d / "trace" / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
        w.writerow([ATTN, 3, 30e6, 10e6, 9e6, 11e6])   # 10 ms
        w.writerow([POOLQ, 3, 3e5, 1e5, 1e5, 1e5])     # 0.1 ms
        w.writerow([POOLK, 3, 3e5, 1e5, 1e5, 1e5])
        w.writerow([SEL, 9, 1.8e6, 2e5, 2e5, 2e5])     # 0.2 ms (calibration launches too)
        w.writerow([COPY, 2, 1e6, 5e5, 5e5, 5e5])
        w.writerow([BWD, 1, 1e6, 1e6, 1e6, 1e6])       # not a layer kernel
    mib = bench.PROFILE_COPY_MB * 1024                  # KiB moved each way by the copy
    # FETCH_SIZE counts half the bytes (scale 2), WRITE_SIZE all (scale 1)
    _pmc(str(d / "fetch"), [[1, COPY, "FETCH_SIZE", mib / 2, 0, 1], [2, ATTN, "FETCH_SIZE", 5e6, 0, 1],
                            [3, ATTN, "FETCH_SIZE", 7e6, 0, 1], [4, SEL, "FETCH_SIZE", 2.5e5, 0, 1]])
    _pmc(str(d / "write"), [[1, COPY, "WRITE_SIZE", mib, 0, 1], [2, ATTN, "WRITE_SIZE", 1e5, 0, 1],
                            [3, ATTN, "WRITE_SIZE", 1e5, 0, 1], [4, SEL, "WRITE_SIZE", 1e3, 0, 1]])
    # the attention dispatch in the counter pass: 10 ms at 2.0 GHz on every XCD
    cyc = 2.0e9 * 10e-3
    _pmc(str(d / "sq"), [[7, ATTN, "GRBM_GUI_ACTIVE", cyc * bench.N_XCD, 0, 10_000_000],
                         [7, ATTN, "SQ_VALU_MFMA_BUSY_CYCLES", 0.4 * cyc * bench.N_SIMD, 0, 10_000_000],
                         [7, ATTN, "SQ_ACTIVE_INST_ANY", 100.0, 0, 10_000_000],
                         [7, ATTN, "SQ_ACTIVE_INST_VALU", 55.0, 0, 10_000_000],
                         [7, ATTN, "SQ_WAVE_CYCLES", 400.0, 0, 10_000_000]])
    # the wait pass: 30 % of wave cycles in s_waitcnt, 20 % waiting to issue, 40 % of the matrix
    # core's busy cycles with vector work alongside, a quarter of LDS cycles in bank conflicts
    _pmc(str(d / "wait"), [[7, ATTN, "SQ_WAVE_CYCLES", 1000.0, 0, 10_000_000],
                           [7, ATTN, "SQ_WAIT_ANY", 300.0, 0, 10_000_000],
                           [7, ATTN, "SQ_WAIT_INST_ANY", 200.0, 0, 10_000_000],
                           [7, ATTN, "SQ_ACTIVE_INST_ANY", 250.0, 0, 10_000_000],
                           [7, ATTN, "SQ_VALU_MFMA_BUSY_CYCLES", 500.0, 0, 10_000_000],
                           [7, ATTN, "SQ_VALU_MFMA_COEXEC_CYCLES", 200.0, 0, 10_000_000],
                           [7, ATTN, "SQ_LDS_IDX_ACTIVE", 80.0, 0, 10_000_000],
                           [7, ATTN, "SQ_LDS_BANK_CONFLICT", 20.0, 0, 10_000_000]])
    info = {"workload": "fake", "kernel_source_sha256": "abc", "dtype": "bf16", "heads": 2, "q_tiles": 4, "k_tiles": 4, "top_k": 1,
            "kmax": 2, "landmarks": False, "layers": 3, "attn_flops_per_launch": 8e12,
            "alg_per_dispatch": {"pool_query": 4e8, "pool_key": 4e8, "score": 1e9, "select": 1e9,
                                 "cast": 0, "attention": 8e12},
            "dispatches_per_layer": {"pool_query": 1, "pool_key": 1, "score": 1, "select": 1, "attention": 1}}
    json.dump(info, open(d / "run_info.json", "w"))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    bench.write_counters(str(d))
    c = json.load(open(tmp_path / "profiles" / "counters_fake.json"))
    assert c["counter_scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    k = {x["family"]: x for x in c["kernels"]}
    assert set(k) == {"attention", "pool_query", "pool_key", "select"}   # backward and copy left out
    a = k["attention"]
    assert a["fetch_bytes"] == round(6e6 * 1024 * 2) and a["write_bytes"] == round(1e5 * 1024)
    assert a["counted_gbs"] == pytest.approx((6e6 * 2 + 1e5) * 1024 / 10e-3 / 1e9, rel=1e-3)
    assert a["tflops"] == pytest.approx(800.0) and a["frac_peak"] == pytest.approx(0.32)
    assert a["clock_ghz"] == pytest.approx(2.0) and a["mfma_busy"] == pytest.approx(0.4)
    assert a["frac_peak_at_clock"] == pytest.approx(800.0 / (2500.0 * 2.0 / 2.4), rel=1e-3)
    assert a["valu_share_of_issue"] == pytest.approx(0.55)
    assert a["wait_counter_share"] == pytest.approx(0.3) and a["wait_issue_share"] == pytest.approx(0.2)
    assert a["issue_share"] == pytest.approx(0.25) and a["coexec_share_of_mfma_busy"] == pytest.approx(0.4)
    assert a["lds_conflict_share"] == pytest.approx(0.25)
    assert a["issue_share_of_wave_cycles"] == pytest.approx(0.25)
    s = k["select"]
    assert s["alg_gbs"] == pytest.approx(1e9 / 2e-4 / 1e9) and s["alg_frac_hbm"] == pytest.approx(0.625)
    assert s["counted_gbs"] == pytest.approx((2.5e5 * 2 + 1e3) * 1024 / 2e-4 / 1e9, rel=1e-3)
    assert "counted_gbs" not in k["pool_query"]                          # no counter rows for it
    assert c["layer_ms_by_family"] == {"pool_query": 0.1, "pool_key": 0.1, "select": 0.2, "attention": 10.0}
    md = open(tmp_path / "profiles" / "counters_fake.md").read()
    assert "rocprofv3 --pmc FETCH_SIZE" in md and "| attention |" in md
    assert "| 30.0% | 20.0% | 25.0% | 40.0% | 25.0% |" in md
    assert c["kernel_source_sha256"] == "abc"                  # the run's, not the current sources'
    tr = open(tmp_path / "profiles" / "trace_fake.md").read()
    assert "--kernel-trace --stats" in tr and "k_attn_bf16" in tr


def test_kernel_family():
    assert bench.kernel_family(POOLQ) == "pool_query"
    assert bench.kernel_family(POOLK) == "pool_key"
    assert bench.kernel_family("void s3d::k_tile_scores_mfma(float const*)") == "score"
    assert bench.kernel_family(SEL) == "select"
    assert bench.kernel_family("void s3d::k_select_topk(float const*)") == "select"
    assert bench.kernel_family(ATTN) == "attention"
    assert bench.kernel_family("void s3d::k_attn<true, true, false>(s3d::AttnDev)") == "attention"
    assert bench.kernel_family(BWD) is None
    assert bench.kernel_family("void s3d::k_attn_bwd_dkv<true>(s3d::BwdDev)") is None
    assert bench.kernel_family("void s3d::k_cast_bf16(float const*, long, __bf16*)") == "cast"
    assert bench.kernel_family(COPY) == "copy"
    assert bench.kernel_family("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, "
                               "std::array<char*, 1ul> >(int, at::native::FillFunctor<float>, std::array<char*, 1ul>)") is None
    assert bench.kernel_family("void other::kernel()") is None


def test_counter_reader_keeps_the_timed_layers(tmp_path, monkeypatch):
    # nine selections: six calibration launches at other budgets (0.5 ms, 4e5 KiB fetched)
    # before the three timed layers (0.1 ms, 1e5 KiB); only the last three may count
    d = tmp_path / "prof"
    os.makedirs(d / "trace")
    with open(d / "trace" / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
        w.writerow([SEL, 9, 3.3e6, 3.67e5, 1e5, 5e5])
        w.writerow([COPY, 1, 5e5, 5e5, 5e5, 5e5])
    with open(d / "trace" / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for i in range(9):
            dt = 500_000 if i < 6 else 100_000
            w.writerow([SEL, t, t + dt])
            t += 10 * dt
        w.writerow([COPY, t, t + 500_000])
    mib = bench.PROFILE_COPY_MB * 1024
    _pmc(str(d / "fetch"), [[0, COPY, "FETCH_SIZE", mib / 2, 0, 1]] +
         [[i + 1, SEL, "FETCH_SIZE", 4e5 if i < 6 else 1e5, 0, 1] for i in range(9)])
    _pmc(str(d / "write"), [[0, COPY, "WRITE_SIZE", mib, 0, 1]] +
         [[i + 1, SEL, "WRITE_SIZE", 0.0, 0, 1] for i in range(9)])
    _pmc(str(d / "sq"), [[0, COPY, "SQ_WAVES", 1.0, 0, 1]])
    info = {"workload": "fake2", "kernel_source_sha256": "abc", "dtype": "bf16", "heads": 1, "q_tiles": 4,
            "k_tiles": 4, "top_k": 1, "kmax": 2, "landmarks": False, "layers": 3, "attn_flops_per_launch": 1.0,
            "alg_per_dispatch": {"select": 1e8}, "dispatches_per_layer": {"select": 1}}
    json.dump(info, open(d / "run_info.json", "w"))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    bench.write_counters(str(d))
    c = json.load(open(tmp_path / "profiles" / "counters_fake2.json"))
    s = {x["family"]: x for x in c["kernels"]}["select"]
    assert s["dispatches"] == 3 and s["avg_ms"] == pytest.approx(0.1)
    assert s["fetch_bytes"] == round(1e5 * 1024 * 2)
    assert c["layer_ms_by_family"]["select"] == pytest.approx(0.1)
