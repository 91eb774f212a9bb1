"""Benchmark of one dynamic tile-sparse global-attention layer on one MI355X.

One step = the whole hot path on one batch of synthetic multi-view tokens:
pooled tile scores -> per-row top-k united with the anchor frame -> exact
attention over the selected tiles (plus landmarks when the workload has them).
Inputs are resident in HBM before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vggt_s128]

Prints one JSON line.  ``value`` is the effective TFLOP/s of the layer: the
algorithmic FLOPs of every attended (query tile, key tile) pair divided by the
wall time of the whole step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse global-attn effective TFLOP/s + ms/layer at S=128 frames, % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
ATTN_SRCS = [os.path.join(ROOT, "dynamic_block_sparse_tile_amd", "csrc", f)
             for f in ("attn_bf16.hip", "attn_common.h", "device.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="vggt_s128")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--dense-reps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-gate", action="store_true", help="skip the 90%% sparsity speedup point")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first run a plain elementwise copy of this many MiB (fp32) twice, as a "
                         "known-size reference for the HBM byte counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter files of a FETCH_SIZE run and a WRITE_SIZE "
                         "run (rocprofv3 --pmc, both with --copy-mb) into profiles/traffic.json")
    return ap.parse_args()


ATTN_KERNEL = "k_attn_bf16<false, false, false, false, 1>"     # the sparse bf16 attention kernel


def write_traffic(fetch_csv, write_csv, copy_mb, workload):
    """HBM bytes per attention launch from two counter runs.  Each counter is scaled by
    what it reads for the plain copy of known size in the same run (the largest elementwise
    launch: copy_mb MiB read and written)."""
    import csv
    from collections import defaultdict

    def per_dispatch(path, counter):
        vals, names = defaultdict(float), {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] == counter:
                vals[row["Dispatch_Id"]] += float(row["Counter_Value"])
                names[row["Dispatch_Id"]] = row["Kernel_Name"]
        attn = [v for d, v in vals.items() if ATTN_KERNEL in names[d]]
        copy = [v for d, v in vals.items() if "elementwise" in names[d]]
        if not attn or not copy:
            raise SystemExit(f"{path}: no {ATTN_KERNEL} or copy dispatch with {counter}")
        return sum(attn) / len(attn), max(copy), len(attn)

    copy_bytes = copy_mb * (1 << 20)
    out = {"workload": workload, "kernel": ATTN_KERNEL, "attn_source_sha256": attn_source_sha256(),
           "copy_reference_bytes": copy_bytes}
    total = 0.0
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        a, c, n = per_dispatch(path, counter)
        scale = copy_bytes / (c * 1024.0)
        out[key] = {"counter": counter, "attn_kib_per_launch": a, "launches": n, "copy_kib": c,
                    "scale": round(scale, 4), "bytes_per_launch": round(a * 1024.0 * scale)}
        total += a * 1024.0 * scale
    out["bytes_per_launch"] = round(total)
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


class Layer:
    """The three library calls of one layer on preallocated-by-torch outputs."""

    def __init__(self, S, LY, w, q, v, seed_k=None):
        self.S, self.LY, self.w = S, LY, w
        self.q, self.v = q, v
        self.lay = w.layout
        self.K, self.V, self.klay = q, v, w.layout
        if w.kv_window > 1:
            self.K, self.V, self.klay = S.sparse3d_grid_subsample_kv(q, v, self.lay, w.grid, w.kv_window)
        self.tpf = self.klay[2] // 64
        self.ts = LY.special_tiles(self.klay)
        self.Tq = w.rows // 64
        self.Tk = self.klay[0] * self.klay[2] // 64
        self.rows = w.heads * self.Tq
        _, _, _, scores = S.sparse3d_tile_scores(q, self.K, self.lay, self.klay)
        if seed_k is not None:
            self.k = seed_k
        elif w.k is not None:
            self.k = w.k
        else:
            self.k = LY.calibrate_k(LY.device_count_fn(scores, self.tpf, w.anchor), self.rows,
                                    self.ts, self.Tk, w.target_sparsity)
        del scores

    def subsample(self):
        if self.w.kv_window > 1:
            self.K, self.V, _ = self.S.sparse3d_grid_subsample_kv(self.q, self.v, self.lay,
                                                                  self.w.grid, self.w.kv_window)

    def scores(self):
        lm = self.w.landmarks
        return self.S.sparse3d_tile_scores(self.q, self.K, self.lay, self.klay, v=self.V if lm else None)

    def select(self, scores):
        return self.S.sparse3d_select_topk(scores, self.k, self.tpf, self.w.anchor)

    def attend(self, idx, cnt, kbar, vbar):
        lm = self.w.landmarks
        if lm and self.q.dtype != kbar.dtype:        # landmark means in the operand precision
            kbar, vbar = self.S.sparse3d_cast(kbar, self.q.dtype), self.S.sparse3d_cast(vbar, self.q.dtype)
        return self.S.sparse3d_sparse_attn_fwd(self.q, self.K, self.V, self.lay, self.klay, idx, cnt,
                                               kbar=kbar if lm else None, vbar=vbar if lm else None)


def run_layer(torch, L, steps, warmup):
    """Time `steps` whole layers; also time each kernel family with events on its stream."""
    st = torch.cuda.current_stream()
    for _ in range(warmup):
        L.subsample()
        qbar, kbar, vbar, sc = L.scores()
        idx, cnt = L.select(sc)
        L.attend(idx, cnt, kbar, vbar)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(st)
    for i in range(steps):
        e = ev[i]
        e[0].record(st)
        L.subsample()
        e[1].record(st)
        qbar, kbar, vbar, sc = L.scores()
        e[2].record(st)
        idx, cnt = L.select(sc)
        e[3].record(st)
        out = L.attend(idx, cnt, kbar, vbar)
        e[4].record(st)
    end.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in ev])
    total_cnt = int(cnt.sum().item())
    return dict(ms_per_step=ms, wall_ms=1e3 * wall / steps, sub_ms=float(per[:, 0].mean()),
                scores_ms=float(per[:, 1].mean()), select_ms=float(per[:, 2].mean()),
                attn_ms=float(per[:, 3].mean()), total_cnt=total_cnt, out=out, idx=idx, cnt=cnt,
                kmax=int(idx.shape[2]))


def time_dense(torch, S, q, v, lay, reps):
    st = torch.cuda.current_stream()
    S.sparse3d_dense_attn_fwd(q, q, v, lay)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(reps):
        S.sparse3d_dense_attn_fwd(q, q, v, lay)
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def attn_source_sha256() -> str:
    h = hashlib.sha256()
    for f in ATTN_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def time_frame(torch, S, q, v, lay, reps):
    """Mean time of the frame-attention call (every query over its own frame)."""
    S.sparse3d_frame_attn_fwd(q, q, v, lay)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(reps):
        S.sparse3d_frame_attn_fwd(q, q, v, lay)
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_sga(torch, S, LY, q, v, w, reps=3):
    """AVGGT subsampled global attention on the same inputs: 2x2 key/value subsample, the
    dropped patches' mean pair, then every query over all kept keys + its own key (where
    dropped) + the mean pair.  Times the mean and the attention call."""
    K2, V2, klay = S.sparse3d_grid_subsample_kv(q, v, w.layout, w.grid, 2)
    km, vm, n = S.sparse3d_discarded_mean(q, v, w.layout, w.grid, 2)
    sga = S.Sga(w.grid, 2, k_full=q, v_full=v, kmean=km, vmean=vm, mean_bias=math.log(n))
    S.sparse3d_dense_attn_fwd(q, K2, V2, w.layout, klay, sga=sga)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(st)
    for _ in range(reps):
        S.sparse3d_discarded_mean(q, v, w.layout, w.grid, 2)
    ev[1].record(st)
    for _ in range(reps):
        S.sparse3d_dense_attn_fwd(q, K2, V2, w.layout, klay, sga=sga)
    ev[2].record(st)
    torch.cuda.synchronize()
    mean_ms = ev[0].elapsed_time(ev[1]) / reps
    attn_ms = ev[1].elapsed_time(ev[2]) / reps
    flops = LY.pair_flops() * w.heads * (w.rows // 64) * (klay[0] * klay[2] // 64)
    return {"window": 2, "kept_keys_per_frame": klay[1], "dropped_rows": n,
            "discarded_mean_ms": round(mean_ms, 4), "attn_ms": round(attn_ms, 4),
            "attn_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 2)}


def time_backward(torch, S, LY, L, fwd_flops, reps=3):
    """Backward of the sparse attention on the bench selection: the selection transpose,
    then dQ, dK, dV (with landmarks also the means' gradients and their chain into the
    member rows).  Algorithmic work = 2.5x the forward's (five products per attended pair or
    landmark: the recomputed scores, dP, dV, dQ, dK, against the forward's two)."""
    qbar, kbar, vbar, sc = L.scores()
    idx, cnt = L.select(sc)
    del sc, qbar
    lm = {}
    if L.w.landmarks:
        lm = dict(kbar=S.sparse3d_cast(kbar, L.q.dtype), vbar=S.sparse3d_cast(vbar, L.q.dtype))
    del kbar, vbar
    out, lse = S.sparse3d_sparse_attn_fwd(L.q, L.K, L.V, L.lay, L.klay, idx, cnt, return_lse=True, **lm)
    g = torch.Generator(device=L.q.device).manual_seed(0)
    dout = torch.randn(L.q.shape, device=L.q.device, dtype=torch.float32, generator=g).to(L.q.dtype)
    t_end, t_list = S.sparse3d_selection_transpose(idx, cnt, L.Tk)
    S.sparse3d_sparse_attn_bwd(L.q, L.K, L.V, out, dout, lse, L.lay, L.klay, idx, cnt, t_end, t_list, **lm)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(st)
    for _ in range(reps):
        S.sparse3d_selection_transpose(idx, cnt, L.Tk)
    ev[1].record(st)
    for _ in range(reps):
        S.sparse3d_sparse_attn_bwd(L.q, L.K, L.V, out, dout, lse, L.lay, L.klay, idx, cnt, t_end, t_list, **lm)
    ev[2].record(st)
    torch.cuda.synchronize()
    tr_ms = ev[0].elapsed_time(ev[1]) / reps
    bw_ms = ev[1].elapsed_time(ev[2]) / reps
    return {"transpose_ms": round(tr_ms, 4), "ms": round(bw_ms, 4), "landmarks": bool(lm),
            "tflops": round(2.5 * fwd_flops / (bw_ms * 1e-3) / 1e12, 2)}


def traffic_entry():
    """Per-launch HBM bytes of the attention kernel from committed counter runs, or None
    when the kernel source changed after the counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    sha = attn_source_sha256()
    if t.get("attn_source_sha256") != sha:
        return None
    return t


def rocminfo_peak():
    """Matrix peak recomputed from the agent's compute-unit count and maximum clock as rocminfo
    reports them (4096 bf16 FLOP per clock per CU), or None where rocminfo is unavailable."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for block in txt.split("Agent ")[1:]:
        if "gfx950" not in block:
            continue
        cu = clk = None
        for line in block.splitlines():
            key, _, val = line.strip().partition(":")
            if key == "Compute Unit":
                cu = int(val.split()[0])
            elif key == "Max Clock Freq. (MHz)":
                clk = int(val.split()[0])
        if cu and clk:
            return {"cus": cu, "max_clock_mhz": clk, "peak_tflops": round(cu * clk * 1e6 * 4096 / 1e12, 1)}
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inp, k, budget_s, LY):
    """The fp64 oracle on a bounded sample of the same workload, scaled to TFLOP/s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:                                   # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))
    lay = oracle.Layout(*w.layout)
    H = w.heads
    heads = [0]                                        # pool/score/select/attend for one head
    t0 = time.perf_counter()
    qbar, qc = oracle.tile_pool(inp.q[:1], lay, 64, "query")
    kbar, kc = oracle.tile_pool(inp.k[:1], lay, 64, "key")
    sig = oracle.tile_scores(qbar, qc, kbar, kc, 0.125)
    t_ps = time.perf_counter() - t0
    Tq, Tk = sig.shape[1], sig.shape[2]
    tpf = w.stride // 64
    rng = np.random.default_rng(0)
    order = rng.permutation(Tq)
    done, t_att, cnt_sum = 0, 0.0, 0
    kmax = oracle.kmax_for(Tk, k, tpf, w.anchor)
    while done < Tq and (t_ps + t_att) < budget_s:
        chunk = order[done:done + 8]
        t1 = time.perf_counter()
        idx = np.full((1, Tq, kmax), -1, dtype=np.int32)
        cnt = np.zeros((1, Tq), dtype=np.int32)
        for t in chunk:
            sel = oracle.select_tiles(sig[0, t], k, tpf, w.anchor)
            cnt[0, t] = len(sel)
            idx[0, t, :len(sel)] = sel
        oracle.sparse_attend(inp.q, inp.k, inp.v, lay, lay, 64, idx, cnt, 0.125,
                             query_tiles=chunk, heads=heads)
        t_att += time.perf_counter() - t1
        cnt_sum += int(cnt.sum())
        done += len(chunk)
    # whole layer = H heads x (pool+score for a head + Tq tiles of select+attend)
    t_layer = H * (t_ps + t_att * Tq / done)
    ts = LY.special_tiles(w.layout)
    flops_sample = LY.selected_flops(cnt_sum, done, ts)
    flops_layer = flops_sample * (H * Tq / done)
    return dict(value=flops_layer / t_layer / 1e12, unit="TFLOP/s", cores=int(min(threads, cores)),
                kind="oracle", cpu_model=cpu_model(),
                sample=(f"head 0: full pool+score ({t_ps:.1f}s), select+attend on {done} of {Tq} "
                        f"query tiles ({t_att:.1f}s); layer time extrapolated x{H} heads, "
                        f"x{Tq / done:.1f} tiles = {t_layer:.0f}s"),
                layer_seconds=t_layer)


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(*args.traffic_from, args.copy_mb or 1024, args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the layer shards by "
                          "head across GPUs with no communication, so per-GPU throughput is the "
                          "one-GPU figure", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from dynamic_block_sparse_tile_amd import layer as LY
    from dynamic_block_sparse_tile_amd import sparse3d as S
    from dynamic_block_sparse_tile_amd import synth
    S.library()
    torch.cuda.init()
    dev = torch.device("cuda:0")
    if args.copy_mb > 0:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.rand(n, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            torch.add(src, 0.0, out=dst)          # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        log(f"copy reference: {args.copy_mb} MiB read + {args.copy_mb} MiB written per launch")
        del src, dst
    w = synth.WORKLOADS[args.workload]
    log(f"workload {w.name}: S={w.frames} N={w.tokens} H={w.heads}; generating inputs")
    inp = synth.make_inputs(w, seed=args.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = torch.from_numpy(inp.q).to(dev, dt)
    v = torch.from_numpy(inp.v).to(dev, dt)
    torch.cuda.synchronize()
    L = Layer(S, LY, w, q, v)
    log(f"k={L.k}; timing {args.steps} steps after {args.warmup} warmup")
    torch.cuda.synchronize()
    r = run_layer(torch, L, args.steps, args.warmup)
    rows = L.rows
    lm_count = 0
    flops = LY.selected_flops(r["total_cnt"], rows, L.ts)
    if w.landmarks:
        # landmarks per (head, query tile) = non-empty unselected tiles; every key tile of
        # these layouts has members, so it is Tk - cnt
        lm_count = rows * L.Tk - r["total_cnt"]
        flops += lm_count * 64 * 4 * 64
    sparsity = LY.measured_sparsity(r["total_cnt"], rows, L.ts, L.Tk)
    value = flops / (r["ms_per_step"] * 1e-3) / 1e12
    attn_tflops = flops / (r["attn_ms"] * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded multi-view latent-bank tokens)",
        "config": {"workload": w.name, "frames": w.frames, "tokens_per_frame": w.tokens,
                   "stride": w.stride, "specials": w.specials, "heads": w.heads,
                   "head_dim": w.head_dim, "tile": w.tile, "top_k": L.k,
                   "target_sparsity": w.target_sparsity, "measured_sparsity": round(sparsity, 5),
                   "landmarks": w.landmarks, "kv_window": w.kv_window, "anchor_frame": w.anchor,
                   "seed": args.seed},
        "pct_bf16_peak_layer": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {"grid_subsample": round(r["sub_ms"], 4), "tile_scores": round(r["scores_ms"], 4),
                       "select_topk": round(r["select_ms"], 4), "sparse_attn": round(r["attn_ms"], 4)},
        "selected_flops": flops,
        "valid_pair_flops": LY.valid_pair_flops(r["idx"].cpu().numpy(), r["cnt"].cpu().numpy(),
                                                w.layout, L.klay),
    }
    Lq = w.rows
    bytes_in = 2 * w.heads * Lq * 64 * (2 if w.dtype == "bf16" else 4)
    sc_bytes = 4 * w.heads * L.Tq * L.Tk
    res["kernels_gbs"] = {
        "tile_scores": round((bytes_in * (1.5 if w.landmarks else 1.0) + sc_bytes) / (r["scores_ms"] * 1e-3) / 1e9, 1),
        "select_topk": round((sc_bytes + 4 * rows * (r["kmax"] + 1)) / (r["select_ms"] * 1e-3) / 1e9, 1),
    }
    # roofline of the dominant kernel (sparse attention): algorithmic FLOPs per launch
    # over its mean launch time, measured with events on its stream during the timed steps
    tr = traffic_entry()
    res["roofline"] = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                       "traffic": (tr["bytes_per_launch"] if tr and tr.get("workload") == w.name else None)}
    dev_peak = rocminfo_peak()
    if dev_peak:
        dev_peak["attn_frac"] = round(attn_tflops / dev_peak["peak_tflops"], 4)
        res["peak_rocminfo"] = dev_peak
    if not args.no_dense:
        log("timing the dense kernel")
        dms = time_dense(torch, S, q, v, w.layout, args.dense_reps)
        dflops = LY.pair_flops() * w.heads * L.Tq * (w.rows // 64)
        res["dense"] = {"ms": round(dms, 3), "tflops": round(dflops / (dms * 1e-3) / 1e12, 2),
                        "speedup_layer_vs_dense": round(dms / r["ms_per_step"], 2)}
    if not args.no_dense:
        # frame attention (early layers, every query over its own frame) on the same inputs
        fms = time_frame(torch, S, q, v, w.layout, 5)
        fflops = LY.pair_flops() * w.heads * L.Tq * (w.stride // 64)
        res["frame_attention"] = {"ms": round(fms, 4), "tflops": round(fflops / (fms * 1e-3) / 1e12, 2)}
        if w.landmarks is False and w.kv_window == 1:
            res["subsampled_global_attention"] = time_sga(torch, S, LY, q, v, w)
        if w.kv_window == 1:
            res["backward"] = time_backward(torch, S, LY, L, flops)
    if not args.no_gate and not args.no_dense and w.name == "vggt_s128":
        w90 = synth.WORKLOADS["vggt_s128_90"]
        L90 = Layer(S, LY, w90, q, v)
        r90 = run_layer(torch, L90, max(5, args.steps // 2), 1)
        sp90 = LY.measured_sparsity(r90["total_cnt"], rows, L90.ts, L90.Tk)
        f90 = LY.selected_flops(r90["total_cnt"], rows, L90.ts)
        res["sparsity_90"] = {"top_k": L90.k, "measured_sparsity": round(sp90, 5),
                              "ms_per_layer": round(r90["ms_per_step"], 4),
                              "attn_ms": round(r90["attn_ms"], 4),
                              "tflops_layer": round(f90 / (r90["ms_per_step"] * 1e-3) / 1e12, 2),
                              "speedup_vs_dense": round(res["dense"]["ms"] / r90["ms_per_step"], 2)}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(w, inp, L.k, args.cpu_budget, LY)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
