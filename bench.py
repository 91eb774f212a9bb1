"""Benchmark of one dynamic tile-sparse global-attention layer on one MI355X.

One step = the whole hot path on one batch of synthetic multi-view tokens:
pooled tile scores -> per-row top-k united with the anchor frame -> exact
attention over the selected tiles (plus landmarks when the workload has them).
Inputs are resident in HBM before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vggt_s128]

Prints one JSON line (one per configuration with --all-configs).  ``value`` is
the effective TFLOP/s of the layer: the algorithmic FLOPs of every attended
(query tile, key tile) pair divided by the wall time of the whole step.  Before
the warmup steps the GPU runs 0.3 s of dense matrix work, so that host-only phases
(input generation, the CPU baseline) do not leave it at idle clocks.
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
PEAK_TFLOPS = {"bf16": 2500.0,   # MI355X dense matrix peaks (published): bf16
               "f32": 157.3}     # fp32 (the fp32 path runs on v_mfma_f32_32x32x2_f32)
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E (published)
N_XCD, N_SIMD = 8, 1024          # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "dynamic_block_sparse_tile_amd", "csrc")
# the configurations of the pages' workloads, smallest first; the default run is vggt_s128
CONFIGS = ["tiny_s2", "vggt_s8", "vggt_s32", "vggt_s128", "vggt_s128_90", "vggt_s256_lm",
           "vggt_s256_lm_sub2"]


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
    ap.add_argument("--all-configs", action="store_true",
                    help="one JSON line per configuration: " + ", ".join(CONFIGS))
    ap.add_argument("--top-k", type=int, default=None, help="fixed k instead of the calibrated one")
    ap.add_argument("--run-info", metavar="PATH",
                    help="write the layer's algorithmic work per kernel dispatch (for --counters-from)")
    ap.add_argument("--profile-commands", metavar="OUTDIR",
                    help="no GPU work: print the rocprofv3 passes that --counters-from reads")
    ap.add_argument("--counters-from", metavar="OUTDIR",
                    help="no GPU work: turn the rocprofv3 passes under OUTDIR into "
                         "profiles/counters_<workload>.json and .md")
    return ap.parse_args()


def kernel_source_sha256() -> str:
    """Hash of every kernel source: counters taken before a change to any of them are stale."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


# rocprofv3 passes over one short benchmark run (the layer kernels plus a plain copy of
# known size, the reference that scales the byte counters); pass name -> profiler options
COUNTER_PASSES = [
    ("trace", "--kernel-trace --stats"),
    ("fetch", "--pmc FETCH_SIZE"),
    ("write", "--pmc WRITE_SIZE"),
    ("sq", "--pmc SQ_WAVE_CYCLES SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES "
           "SQ_INSTS_VALU SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE"),
    # where the waves spend their cycles: waiting on counters (memory, LDS, barriers), waiting
    # for an instruction to issue, matrix/vector overlap, LDS bank conflicts
    ("wait", "--pmc SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
             "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT"),
]
PROFILE_COPY_MB = 1024


def profile_commands(workload: str, outdir: str) -> list:
    bench = (f"python3 {os.path.join(ROOT, 'bench.py')} --workload {workload} --steps 2 --warmup 1 "
             f"--no-cpu-baseline --no-dense --no-gate --copy-mb {PROFILE_COPY_MB}")
    cmds = []
    for name, opts in COUNTER_PASSES:
        d = os.path.join(outdir, name)
        info = f" --run-info {os.path.join(outdir, 'run_info.json')}" if name == "trace" else ""
        regex = "" if name == "trace" else " --kernel-include-regex 's3d::|elementwise'"
        cmds.append(f"timeout -s KILL 300 rocprofv3 {opts}{regex} --output-format csv -d {d} -o run -- "
                    f"{bench}{info}")
    return cmds


def kernel_family(name: str):
    """Which step of the layer a kernel name belongs to (None: not a layer kernel)."""
    if "elementwise" in name:
        # the copy reference is torch's add (src + 0 into dst); other elementwise kernels
        # (the fill of the stream references) are not layer kernels
        return "copy" if "_add" in name else None
    if "s3d::" not in name:
        return None
    if "k_tile_pool" in name:
        # template arguments <bf16, key_rows>
        return "pool_key" if name.split("<", 1)[1].split(">", 1)[0].replace(" ", "").endswith("true") else "pool_query"
    for key, fam in (("k_tile_scores", "score"), ("k_select_topk", "select"), ("k_cast_bf16", "cast"),
                     ("k_grid_subsample", "subsample"), ("k_attn_bwd", None), ("k_attn", "attention")):
        if key in name:
            return fam
    return None


def write_counters(outdir: str):
    """Per-kernel figures of one layer from the rocprofv3 passes under outdir: mean duration
    (kernel trace), HBM bytes per dispatch (FETCH_SIZE / WRITE_SIZE, each scaled by what the
    counter reads for the plain copy of known size), counted and algorithmic GB/s against
    the 8 TB/s peak, and for the attention kernel the shader clock, matrix-core busy share
    (SQ_VALU_MFMA_BUSY_CYCLES over SIMD cycles) and FLOP rate against the matrix peak."""
    import csv
    import glob
    from collections import defaultdict

    info = json.load(open(os.path.join(outdir, "run_info.json")))
    if "kernel_source_sha256" not in info:
        raise SystemExit(f"{outdir}/run_info.json records no kernel source hash")
    stats = glob.glob(os.path.join(outdir, "trace", "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"{outdir}/trace: no kernel_stats.csv")
    # The figures of one layer come from the layers the run timed (warm-up included): the
    # last dispatches_per_layer x layers dispatches of each kernel.  Dispatches before them
    # (the sparsity calibration's selections at other budgets) are left out.
    def keep(name):
        fam = kernel_family(name)
        n = info["dispatches_per_layer"].get(fam, 0) if fam else 0
        return n * info.get("layers", 0)

    dur = {}                                            # name -> (calls, mean ns)
    traces = glob.glob(os.path.join(outdir, "trace", "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        per_name = defaultdict(list)                    # name -> [(start, duration ns)]
        for row in csv.DictReader(open(traces[0])):
            t0, t1 = int(row["Start_Timestamp"]), int(row["End_Timestamp"])
            per_name[row["Kernel_Name"]].append((t0, t1 - t0))
        for name, ds in per_name.items():
            ds.sort()
            n = keep(name)
            if n:
                ds = ds[-n:]
            dur[name] = (len(ds), sum(d for _, d in ds) / len(ds))
    else:
        for row in csv.DictReader(open(stats[0])):
            dur[row["Name"]] = (int(row["Calls"]), float(row["AverageNs"]))

    def counters(pass_name):
        files = glob.glob(os.path.join(outdir, pass_name, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"{outdir}/{pass_name}: no counter_collection.csv")
        per = defaultdict(lambda: defaultdict(float))   # (name, counter) -> dispatch -> value
        span = {}
        for row in csv.DictReader(open(files[0])):
            per[(row["Kernel_Name"], row["Counter_Name"])][row["Dispatch_Id"]] += float(row["Counter_Value"])
            span[row["Dispatch_Id"]] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
        return per, span

    fetch, _ = counters("fetch")
    write, _ = counters("write")
    sq, span = counters("sq")
    # the wait pass is optional (profiles taken before it existed have four passes)
    wait = counters("wait")[0] if glob.glob(os.path.join(outdir, "wait", "**", "*counter_collection.csv"),
                                          recursive=True) else {}

    def mean_of(per, name, counter):
        v = per.get((name, counter))
        if not v:
            return None
        vals = [v[d] for d in sorted(v, key=int)]
        n = keep(name)
        if n:
            vals = vals[-n:]
        return sum(vals) / len(vals)

    copy_bytes = PROFILE_COPY_MB * (1 << 20)
    scale = {}
    for cname, per in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        copies = [max(v.values()) for (n, c), v in per.items() if c == cname and kernel_family(n) == "copy"]
        if not copies:
            raise SystemExit(f"no copy reference dispatch with {cname}")
        scale[cname] = copy_bytes / (max(copies) * 1024.0)   # known bytes per counted KiB

    alg = info["alg_per_dispatch"]
    kernels = []
    for name, (calls, ns) in sorted(dur.items(), key=lambda x: -x[1][0] * x[1][1]):
        fam = kernel_family(name)
        if fam in (None, "copy"):
            continue
        sec = ns * 1e-9
        fb = mean_of(fetch, name, "FETCH_SIZE")
        wb = mean_of(write, name, "WRITE_SIZE")
        k = {"name": name, "family": fam, "dispatches": calls, "avg_ms": round(sec * 1e3, 4),
             "per_layer": info["dispatches_per_layer"].get(fam, 0)}
        if fb is not None and wb is not None:
            byt = fb * 1024.0 * scale["FETCH_SIZE"] + wb * 1024.0 * scale["WRITE_SIZE"]
            k.update(fetch_bytes=round(fb * 1024.0 * scale["FETCH_SIZE"]),
                     write_bytes=round(wb * 1024.0 * scale["WRITE_SIZE"]),
                     counted_gbs=round(byt / sec / 1e9, 1), counted_frac_hbm=round(byt / sec / 1e9 / PEAK_HBM_GBS, 4))
        if fam != "attention" and fam in alg:
            k.update(alg_bytes=alg[fam], alg_gbs=round(alg[fam] / sec / 1e9, 1),
                     alg_frac_hbm=round(alg[fam] / sec / 1e9 / PEAK_HBM_GBS, 4))
        grbm = sq.get((name, "GRBM_GUI_ACTIVE"))
        # the clock (and the busy share that uses it) only for dispatches of at least 0.1 ms:
        # on shorter ones the active-cycle count and the dispatch timestamps do not line up
        if grbm and sec >= 1e-4:
            # cycles per XCD over the dispatch's own span in that pass
            ids = sorted(grbm, key=int)
            if keep(name):
                ids = ids[-keep(name):]
            clocks = [grbm[d] / N_XCD / span[d] for d in ids if span.get(d, 0) > 0]
            cyc = sum(grbm[d] for d in ids) / len(ids) / N_XCD
            k["clock_ghz"] = round(sum(clocks) / len(clocks) / 1e9, 3) if clocks else None
            busy = mean_of(sq, name, "SQ_VALU_MFMA_BUSY_CYCLES")
            anyi = mean_of(sq, name, "SQ_ACTIVE_INST_ANY")
            valu = mean_of(sq, name, "SQ_ACTIVE_INST_VALU")
            wavec = mean_of(sq, name, "SQ_WAVE_CYCLES")
            if busy is not None:
                k["mfma_busy"] = round(busy / (cyc * N_SIMD), 4)
            if anyi and valu is not None:
                k["valu_share_of_issue"] = round(valu / anyi, 4)
            if anyi and wavec:
                k["issue_share_of_wave_cycles"] = round(anyi / wavec, 4)
        if wait and sec >= 1e-4:
            w = {c: mean_of(wait, name, c) for c in ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                                                      "SQ_ACTIVE_INST_ANY", "SQ_VALU_MFMA_BUSY_CYCLES",
                                                      "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_IDX_ACTIVE",
                                                      "SQ_LDS_BANK_CONFLICT")}
            if w["SQ_WAVE_CYCLES"]:
                for key, c in (("wait_counter_share", "SQ_WAIT_ANY"), ("wait_issue_share", "SQ_WAIT_INST_ANY"),
                               ("issue_share", "SQ_ACTIVE_INST_ANY")):
                    if w[c] is not None:
                        k[key] = round(w[c] / w["SQ_WAVE_CYCLES"], 4)
            if w["SQ_VALU_MFMA_BUSY_CYCLES"] and w["SQ_VALU_MFMA_COEXEC_CYCLES"] is not None:
                k["coexec_share_of_mfma_busy"] = round(w["SQ_VALU_MFMA_COEXEC_CYCLES"] / w["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
            if w["SQ_LDS_IDX_ACTIVE"] and w["SQ_LDS_BANK_CONFLICT"] is not None:
                k["lds_conflict_share"] = round(w["SQ_LDS_BANK_CONFLICT"] / w["SQ_LDS_IDX_ACTIVE"], 4)
        if fam == "attention":
            flops = info["attn_flops_per_launch"]
            peak = PEAK_TFLOPS[info["dtype"]]
            k.update(flops=flops, tflops=round(flops / sec / 1e12, 2), frac_peak=round(flops / sec / 1e12 / peak, 4))
            if k.get("clock_ghz"):
                # the same peak at the clock the kernel actually ran (peak is quoted at 2.4 GHz)
                k["frac_peak_at_clock"] = round(k["tflops"] / (peak * k["clock_ghz"] / 2.4), 4)
        kernels.append(k)
    fam_ms = defaultdict(float)
    for fam, n in info["dispatches_per_layer"].items():
        ks = [k for k in kernels if k["family"] == fam]
        if ks:                                          # instances of one family: mean over dispatches
            tot = sum(k["avg_ms"] * k["dispatches"] for k in ks) / sum(k["dispatches"] for k in ks)
            fam_ms[fam] = round(n * tot, 4)
    # the hash of the kernel sources the counters were measured with (recorded by the run)
    out = {"workload": info["workload"], "kernel_source_sha256": info["kernel_source_sha256"],
           "run": info, "copy_reference_bytes": copy_bytes,
           "counter_scale": {c: round(v, 4) for c, v in scale.items()},
           "commands": [c.replace(ROOT, "$R") for c in profile_commands(info["workload"], outdir)],
           "kernels": kernels,
           "layer_ms_by_family": dict(fam_ms)}
    os.makedirs(PROFILES, exist_ok=True)
    base = os.path.join(PROFILES, f"counters_{info['workload']}")
    with open(base + ".json", "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    with open(base + ".md", "w") as f:
        f.write(counters_markdown(out))
    trace = os.path.join(PROFILES, f"trace_{info['workload']}.md")
    with open(trace, "w") as f:
        f.write(trace_markdown(info["workload"], stats[0], profile_commands(info["workload"], outdir)[0]))
    print(json.dumps({"written": [base + ".json", base + ".md", trace]}))


def trace_markdown(workload: str, stats_csv: str, command: str) -> str:
    """The kernel-trace summary (rocprofv3 --kernel-trace --stats) of the profiled bench run."""
    import csv
    rows = [r for r in csv.DictReader(open(stats_csv))]
    L = [f"# Kernel trace: {workload} (generated by `bench.py --counters-from` from the trace pass)", "",
         "Command (`$R` = repository root, run from /tmp with TMPDIR=/tmp):", "", "```",
         command.replace(ROOT, "$R"), "```", "",
         "| kernel | calls | mean ms | min ms | max ms | total ms |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        L.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                 f"{float(r['MinNs']) / 1e6:.4f} | {float(r['MaxNs']) / 1e6:.4f} | "
                 f"{float(r['TotalDurationNs']) / 1e6:.3f} |")
    L.append("")
    return "\n".join(L)


def counters_markdown(c) -> str:
    """The generated summary of counters_<workload>.json."""
    run = c["run"]
    L = [f"# Kernel counters: one layer of {c['workload']} (generated by `bench.py --counters-from`)", "",
         f"{run['heads']} heads, {run['q_tiles']} query tiles x {run['k_tiles']} key tiles per head, "
         f"k = {run['top_k']}, landmarks {run['landmarks']}, dtype {run['dtype']}.  Durations from the kernel "
         f"trace; bytes from FETCH_SIZE and WRITE_SIZE per dispatch, scaled by what each counter reads for "
         f"a plain copy of {c['copy_reference_bytes'] >> 20} MiB read + written "
         f"(FETCH_SIZE x{c['counter_scale']['FETCH_SIZE']}, WRITE_SIZE x{c['counter_scale']['WRITE_SIZE']}); "
         f"peaks: HBM {PEAK_HBM_GBS / 1000:g} TB/s, matrix {PEAK_TFLOPS[run['dtype']]:g} TFLOP/s "
         f"({run['dtype']}, quoted at 2.4 GHz).", "",
         f"Each kernel's figures are means over the dispatches of the {run.get('layers', '?')} layers the run "
         f"timed (warm-up included), one layer's worth per layer; the sparsity calibration's selections "
         f"before them are left out.  The shader clock and the matrix-core busy share are given for "
         f"dispatches of at least 0.1 ms.",
         "", "Commands (`$R` = repository root, run from /tmp with TMPDIR=/tmp):", "", "```"]
    for cmd in c["commands"]:
        L.append(cmd)
    L.append(f"python3 $R/bench.py --counters-from {c['commands'][0].split(' -d ')[1].split('/trace')[0]}")
    L += ["```", "", "| kernel | step | dispatches | ms | counted GB/s | of 8 TB/s | algorithmic GB/s | of 8 TB/s | clock GHz | MFMA busy | VALU share of issue |",
          "|---|---|---|---|---|---|---|---|---|---|---|"]

    def f(x, fmt="{:.4g}"):
        return "—" if x is None else fmt.format(x)
    for k in c["kernels"]:
        L.append(f"| `{k['name'][:70]}` | {k['family']} | {k['dispatches']} | {k['avg_ms']:.4f} | "
                 f"{f(k.get('counted_gbs'), '{:.0f}')} | {f(k.get('counted_frac_hbm'), '{:.1%}')} | "
                 f"{f(k.get('alg_gbs'), '{:.0f}')} | {f(k.get('alg_frac_hbm'), '{:.1%}')} | "
                 f"{f(k.get('clock_ghz'), '{:.2f}')} | {f(k.get('mfma_busy'), '{:.1%}')} | "
                 f"{f(k.get('valu_share_of_issue'), '{:.1%}')} |")
    if any("wait_counter_share" in k for k in c["kernels"]):
        L += ["", "Where the waves of each kernel (dispatches of at least 0.1 ms) spend their cycles, from the "
              "wait pass: shares of SQ_WAVE_CYCLES spent in s_waitcnt or a barrier (SQ_WAIT_ANY), waiting for "
              "an instruction to issue (SQ_WAIT_INST_ANY) and issuing (SQ_ACTIVE_INST_ANY); the share of "
              "matrix-core busy cycles with vector work issued alongside (SQ_VALU_MFMA_COEXEC_CYCLES over "
              "SQ_VALU_MFMA_BUSY_CYCLES); LDS bank-conflict cycles over LDS-active cycles.", "",
              "| kernel | step | waiting on counters | waiting to issue | issuing | vector under matrix | LDS conflicts |",
              "|---|---|---|---|---|---|---|"]
        for k in c["kernels"]:
            if "wait_counter_share" in k:
                L.append(f"| `{k['name'][:70]}` | {k['family']} | {f(k.get('wait_counter_share'), '{:.1%}')} | "
                         f"{f(k.get('wait_issue_share'), '{:.1%}')} | {f(k.get('issue_share'), '{:.1%}')} | "
                         f"{f(k.get('coexec_share_of_mfma_busy'), '{:.1%}')} | {f(k.get('lds_conflict_share'), '{:.1%}')} |")
    for k in c["kernels"]:
        if k["family"] == "attention":
            L += ["", f"Attention `{k['name'][:70]}`: {k['flops']:.4g} FLOP per launch in {k['avg_ms']:.3f} ms = "
                  f"{k['tflops']:.1f} TFLOP/s, {k['frac_peak']:.1%} of the published peak"
                  + (f", {k['frac_peak_at_clock']:.1%} of the peak at the {k['clock_ghz']:.2f} GHz it ran"
                     if k.get("frac_peak_at_clock") else "")
                  + (f"; HBM traffic {(k['fetch_bytes'] + k['write_bytes']) / 1e9:.2f} GB per launch."
                     if "fetch_bytes" in k else ".")]
            ev = c["run"].get("events_ms", {}).get("attention")
            if ev:
                L += ["", f"The traced run's own bench line (events on the kernel's stream over its timed "
                          f"steps) measured the attention launch at {ev:.3f} ms, against the trace's "
                          f"{k['avg_ms']:.3f} ms mean."]
    L += ["", "Per layer (dispatches per layer x mean duration): " +
          ", ".join(f"{fam} {ms:.4f} ms" for fam, ms in c["layer_ms_by_family"].items()), ""]
    return "\n".join(L)


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
        """(qbar, kbar, vbar, scores): with landmarks, kbar/vbar are the means in the operand
        dtype that the pooling pass writes alongside the fp32 ones."""
        lm = self.w.landmarks
        r = self.S.sparse3d_tile_scores(self.q, self.K, self.lay, self.klay, v=self.V if lm else None,
                                        operand_means=lm)
        return (r[0], r[4], r[5], r[3]) if lm else r

    def select(self, scores):
        return self.S.sparse3d_select_topk(scores, self.k, self.tpf, self.w.anchor)

    def attend(self, idx, cnt, kbar, vbar):
        lm = self.w.landmarks
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
    enq = time.perf_counter() - t0                  # host time to enqueue the K steps
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in ev])
    total_cnt = int(cnt.sum().item())
    return dict(ms_per_step=ms, wall_ms=1e3 * wall / steps, enqueue_ms=1e3 * enq / steps,
                sub_ms=float(per[:, 0].mean()),
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
    lm = dict(kbar=kbar, vbar=vbar) if L.w.landmarks else {}     # operand-dtype means
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


def counters_entry(workload: str):
    """The committed counter summary of this workload, or None when any kernel source changed
    after the counters were taken."""
    try:
        c = json.load(open(os.path.join(PROFILES, f"counters_{workload}.json")))
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return c


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
    """The fp64 oracle on a bounded sample of the same workload (subsampled keys and the
    landmark term where the workload has them), scaled to TFLOP/s."""
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
    Q, K, V, klay = inp.q[:1], inp.k[:1], inp.v[:1], lay
    if w.kv_window > 1:
        K, V, klay = oracle.subsample_keys(K, V, lay, w.grid, w.kv_window, 64)
    qbar, qc = oracle.tile_pool(Q, lay, 64, "query")
    kbar, kc = oracle.tile_pool(K, klay, 64, "key")
    lm = {}
    if w.landmarks:
        vbar, _ = oracle.tile_pool(V, klay, 64, "key")
        lm = dict(kbar=kbar, vbar=vbar, kcount=kc)
    sig = oracle.tile_scores(qbar, qc, kbar, kc, 0.125)
    t_ps = time.perf_counter() - t0
    Tq, Tk = sig.shape[1], sig.shape[2]
    tpf = klay.stride // 64
    nonempty = kc > 0
    rng = np.random.default_rng(0)
    order = rng.permutation(Tq)
    done, t_att, cnt_sum, lm_sum = 0, 0.0, 0, 0
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
            if w.landmarks:
                lm_sum += int(nonempty.sum() - nonempty[sel].sum())
        oracle.sparse_attend(Q, K, V, lay, klay, 64, idx, cnt, 0.125, query_tiles=chunk, heads=heads, **lm)
        t_att += time.perf_counter() - t1
        cnt_sum += int(cnt.sum())
        done += len(chunk)
    # whole layer = H heads x (pool+score for a head + Tq tiles of select+attend)
    t_layer = H * (t_ps + t_att * Tq / done)
    ts = LY.special_tiles(tuple(klay))
    # landmarks: 4 * 64 FLOP per (query row, landmark), 64 rows per query tile
    flops_sample = LY.selected_flops(cnt_sum, done, ts) + lm_sum * 64 * 4 * 64
    flops_layer = flops_sample * (H * Tq / done)
    return dict(value=flops_layer / t_layer / 1e12, unit="TFLOP/s", cores=int(min(threads, cores)),
                kind="oracle", cpu_model=cpu_model(),
                sample=(f"head 0: full pool+score ({t_ps:.1f}s), select+attend"
                        f"{' with landmarks' if w.landmarks else ''} on {done} of {Tq} query tiles "
                        f"({t_att:.1f}s); layer time extrapolated x{H} heads, x{Tq / done:.1f} tiles = "
                        f"{t_layer:.0f}s"),
                layer_seconds=t_layer)


def alg_per_dispatch(w, L, kmax: int, attn_flops: int) -> dict:
    """Algorithmic bytes each kernel dispatch of the layer must move (FLOPs for attention):
    operands read once, outputs written once."""
    eb = 2 if w.dtype == "bf16" else 4
    H, d = w.heads, w.head_dim
    rows_q, rows_k = w.rows, L.klay[0] * L.klay[2]
    out = {"pool_query": H * rows_q * d * eb + H * L.Tq * d * 4,
           # with landmarks the key/value pools also write the means in the operand dtype
           "pool_key": H * rows_k * d * eb + H * L.Tk * d * 4 + (H * L.Tk * d * eb if w.landmarks else 0),
           "score": H * L.Tq * L.Tk * 4 + H * (L.Tq + L.Tk) * d * 4,
           "select": H * L.Tq * L.Tk * 4 + H * L.Tq * (kmax + 1) * 4,
           "cast": H * L.Tk * d * (4 + eb),
           "attention": attn_flops}
    if w.kv_window > 1:
        kept = L.klay[0] * L.klay[1]                   # valid rows after the subsample
        out["subsample"] = 2 * H * kept * d * eb + 2 * H * rows_k * d * eb
    return out


def stream_refs(torch, dev, nbytes: int, reps: int = 10) -> dict:
    """What a library store kernel reaches on a buffer the size of the score matrix: torch's
    fill (stores only, in address order, the score kernel's kind of traffic), mean GB/s over
    `reps` launches timed with events on the current stream.  The score kernel is quoted
    against this rate as well as against the published 8 TB/s."""
    buf = torch.empty(nbytes // 4, device=dev, dtype=torch.float32)
    out = {"bytes": int(buf.numel() * 4)}
    for _ in range(2):
        buf.fill_(1.0)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        buf.fill_(1.0)
    b.record()
    torch.cuda.synchronize()
    out["fill_gbs"] = round(out["bytes"] / (a.elapsed_time(b) / reps * 1e-3) / 1e9, 1)
    del buf
    return out


def spin_up(torch, dev, seconds: float = 0.3):
    """Bring the GPU out of its idle clocks before the warmup steps: a few hundred
    milliseconds of dense matrix work (seconds of host-only work, such as input generation
    or the CPU baseline, leave it idle; a small layer's warmup steps alone do not ramp it
    up, and the timed steps then ran several times slower)."""
    a = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            b = a @ a
        torch.cuda.synchronize()
    del a, b


def bench_workload(args, w, torch, S, LY, synth, dev, single: bool) -> dict:
    log(f"workload {w.name}: S={w.frames} N={w.tokens} H={w.heads}; generating inputs")
    inp = synth.make_inputs(w, seed=args.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = torch.from_numpy(inp.q).to(dev, dt)
    v = torch.from_numpy(inp.v).to(dev, dt)
    torch.cuda.synchronize()
    L = Layer(S, LY, w, q, v, seed_k=args.top_k)
    log(f"k={L.k}; timing {args.steps} steps after {args.warmup} warmup")
    spin_up(torch, dev)
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
    peak = PEAK_TFLOPS[w.dtype]
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
        f"pct_{w.dtype}_peak_layer": round(100 * value / peak, 2),
        "kernels_ms": {"grid_subsample": round(r["sub_ms"], 4), "tile_scores": round(r["scores_ms"], 4),
                       "select_topk": round(r["select_ms"], 4), "sparse_attn": round(r["attn_ms"], 4)},
        # host time to enqueue one step: close to ms_per_step means the step was launch-bound
        "enqueue_ms_per_step": round(r["enqueue_ms"], 4),
        "selected_flops": flops,
        "valid_pair_flops": LY.valid_pair_flops(r["idx"].cpu().numpy(), r["cnt"].cpu().numpy(),
                                                w.layout, L.klay),
    }
    alg = alg_per_dispatch(w, L, r["kmax"], flops)
    # pool + score are one library call (timed together); select is one call
    ps_bytes = alg["pool_query"] + alg["pool_key"] * (2 if w.landmarks else 1) + alg["score"]
    res["kernels_gbs"] = {
        "tile_scores": round(ps_bytes / (r["scores_ms"] * 1e-3) / 1e9, 1),
        "select_topk": round(alg["select"] / (r["select_ms"] * 1e-3) / 1e9, 1)}
    res["kernels_frac_hbm"] = {n: round(g / PEAK_HBM_GBS, 4) for n, g in res["kernels_gbs"].items()}
    res["stream_refs"] = stream_refs(torch, dev, w.heads * L.Tq * L.Tk * 4)
    if args.run_info:
        per_layer = {"pool_query": 1, "pool_key": 2 if w.landmarks else 1, "score": 1, "select": 1,
                     "attention": 1}
        if w.kv_window > 1:
            per_layer["subsample"] = 1
        with open(args.run_info, "w") as f:
            json.dump({"workload": w.name, "kernel_source_sha256": kernel_source_sha256(),
                       "dtype": w.dtype, "heads": w.heads, "q_tiles": L.Tq,
                       "k_tiles": L.Tk, "top_k": L.k, "kmax": r["kmax"], "landmarks": w.landmarks,
                       "layers": args.steps + args.warmup, "attn_flops_per_launch": flops,
                       "alg_per_dispatch": alg, "dispatches_per_layer": per_layer,
                       # the same run's own timing: events on the stream over the timed steps
                       "events_ms": {"attention": round(r["attn_ms"], 4),
                                     "score_call": round(r["scores_ms"], 4),
                                     "select": round(r["select_ms"], 4)}}, f, indent=1)
    # roofline of the dominant kernel (sparse attention): algorithmic FLOPs per launch
    # over its mean launch time, measured with events on its stream during the timed steps
    c = counters_entry(w.name)
    attn_c = next((k for k in c["kernels"] if k["family"] == "attention"), None) if c else None
    res["roofline"] = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                       "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                       "traffic": (attn_c["fetch_bytes"] + attn_c["write_bytes"]
                                   if attn_c and "fetch_bytes" in attn_c else None)}
    if c:
        # per-kernel split from the committed counters of this workload (same kernel sources)
        res["counters"] = {k["family"]: {kk: k.get(kk) for kk in ("avg_ms", "counted_gbs", "counted_frac_hbm",
                                                                     "alg_gbs", "alg_frac_hbm", "mfma_busy",
                                                                     "clock_ghz") if k.get(kk) is not None}
                           for k in c["kernels"] if k["family"] in ("pool_query", "pool_key", "score",
                                                                   "select", "attention")}
    dev_peak = rocminfo_peak() if w.dtype == "bf16" else None
    if dev_peak:
        dev_peak["attn_frac"] = round(attn_tflops / dev_peak["peak_tflops"], 4)
        res["peak_rocminfo"] = dev_peak
    if not args.no_dense:
        log("timing the dense kernel")
        dms = time_dense(torch, S, q, v, w.layout, args.dense_reps)
        dflops = LY.pair_flops() * w.heads * L.Tq * (w.rows // 64)
        res["dense"] = {"ms": round(dms, 3), "tflops": round(dflops / (dms * 1e-3) / 1e12, 2),
                        "speedup_layer_vs_dense": round(dms / r["ms_per_step"], 2)}
        # frame attention (early layers, every query over its own frame) on the same inputs
        fms = time_frame(torch, S, q, v, w.layout, 5)
        fflops = LY.pair_flops() * w.heads * L.Tq * (w.stride // 64)
        res["frame_attention"] = {"ms": round(fms, 4), "tflops": round(fflops / (fms * 1e-3) / 1e12, 2)}
        if w.landmarks is False and w.kv_window == 1:
            res["subsampled_global_attention"] = time_sga(torch, S, LY, q, v, w)
        if w.kv_window == 1 and w.dtype == "bf16":
            log("timing the backward")
            res["backward"] = time_backward(torch, S, LY, L, flops)
    if single and not args.no_gate and not args.no_dense and w.name == "vggt_s128":
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
    del r, L, q, v, inp
    return res


def main():
    args = parse()
    if args.profile_commands:
        print("\n".join(profile_commands(args.workload, args.profile_commands)))
        return
    if args.counters_from:
        write_counters(args.counters_from)
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
    if not args.all_configs:
        res = bench_workload(args, synth.WORKLOADS[args.workload], torch, S, LY, synth, dev, single=True)
        print(json.dumps(res), flush=True)
        return
    # every configuration's GPU timing first, then the CPU baselines: the oracle's BLAS threads
    # keep the host busy for a while after each call, which slowed the launches of the next
    # configuration (a 1.1 ms layer measured 4.6 ms that way)
    results = []
    cpu = args.no_cpu_baseline
    args.no_cpu_baseline = True
    for name in CONFIGS:
        results.append(bench_workload(args, synth.WORKLOADS[name], torch, S, LY, synth, dev, single=False))
        torch.cuda.empty_cache()
    for name, res in zip(CONFIGS, results):
        if not cpu:
            w = synth.WORKLOADS[name]
            log(f"timing the CPU oracle on a bounded sample of {name}")
            res["cpu_baseline"] = cpu_baseline(w, synth.make_inputs(w, seed=args.seed), res["config"]["top_k"],
                                               args.cpu_budget, LY)
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
