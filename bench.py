#!/usr/bin/env python3
"""Benchmark of the hybrid attention hot path on one MI355X.

A step is one forward + backward pass of the layer (GLA branch + anchor
window, every row of the hot path except decode) over one batch of the
training workload B=4, H=32, L=8192, d=128, W=128, M=4, chunk 64, bf16
activations with fp32 gates; inputs are seeded synthetic tensors already in
HBM.  The constant-memory decode step is measured in the same run on its own
workload (B=64 sequences after a 4096-token prefill) and reported under
"decode"; the 65 536-token prefill, one shot and as continued segments, under
"prefill"; the training step with one gate per head and token under
"scalar_gate"; the gate projection g = log sigmoid(x W^T)/tau that feeds
the layer, per key dimension and scalar, under "gate_proj"; the stage-1
attention-approximation step (layer forward, teacher attention + MSE, layer
backward) under "stage1"; the layer with a Hedgehog feature map on its GLA
branch under "features".  Prints one JSON line.

Per-kernel times come from HIP events recorded on the stream the kernels
run on; the backward records them between its kernels through the
library's stage-event hook.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-attn fwd+bwd tokens/s (8B-shaped layer) + % MFMA/HBM roofline"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6        # MI355X dense bf16 matrix peak, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")


def flops_per_head_token(L, d, C, W, M):
    """Fixed-work FLOP convention: intra-chunk blocks counted full C x C,
    window keys counted exactly (sum_t min(t+1, W) / L on average)."""
    wk = sum(min(t + 1, W) for t in range(min(L, W))) + max(0, L - W) * W
    wavg = wk / L
    fwd = 4 * C * d + 4 * d * d + 2 * (wavg + M) * d + 2 * wavg * d
    bwd = 10 * C * d + 10 * d * d + 6 * (wavg + M) * d + 4 * wavg * d
    return fwd, bwd


# compulsory HBM bytes per head-token (bf16 q,k,v,o,dO,dq,dk,dv; fp32 g, dg)
FWD_BYTES = 3 * 2 * 128 + 4 * 128 + 2 * 128          # 1536
BWD_BYTES = 4 * 2 * 128 + 4 * 128 + 3 * 2 * 128 + 4 * 128   # 2816


class Hip:
    """Minimal HIP event API through ctypes (events on torch's stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        P = ctypes.c_void_p
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(P)]
        self.lib.hipEventRecord.argtypes = [P, P]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ev, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current sources of that kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get(kernel)
    if not ent or ent.get("source_sha") != source_sha(ent.get("sources", [])):
        return None
    return ent.get("bytes_per_launch")


def load_counters(kernel):
    """Matrix-core and LDS counter figures of one kernel from the committed rocprofv3 summary, if
    they were taken on the current sources of that kernel; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get(kernel)
    if not ent or ent.get("source_sha") != source_sha(ent.get("sources", [])):
        return None
    return {k: ent[k] for k in ("mfma_busy_frac", "lds_bank_conflict_cycles_per_lds_inst") if k in ent}


# ------------------------------------------------------------ rocprofv3 summaries
# The kernels of the training step and of one decode step, as the counter runs name them:
# (name in the summaries, kernel template, grid in threads, source file)
PROFILED = [
    ("sweep_kernel_fwd", "sweep_kernel<bf16_t, 128, false, false, false, false>", 131072, "lz_sweep.hip"),
    ("out_kernel", "out_kernel<bf16_t, 128, false, false, false>", 4194304, "lz_fwd.hip"),
    ("sweep_kernel_bwd", "sweep_kernel<bf16_t, 128, true, false, false, false>", 131072, "lz_sweep.hip"),
    ("chunk_kernel", "chunk_kernel<bf16_t, 128, false, false>", 8388608, "lz_bwd.hip"),
    ("decode_kernel", "decode_kernel<bf16_t, 128, false>", 1048576, "lz_decode.hip"),
    ("decode_pos_kernel", "decode_pos_kernel", 256, "lz_decode.hip"),
]
XCDS, CUS, SIMDS_PER_CU = 8, 256, 4
PROFILE_ARGS = ("--steps 5 --warmup 2 --no-cpu-baseline --no-prefill --no-scalar-gate --no-gate-proj --no-stage1 "
                "--no-features --no-fwd-8b --no-recompute --no-strong-gates --decode-steps 16 --copy-calibration")


def _kernel_key(name):
    import re
    n = name.replace("void ", "").replace("(anonymous namespace)::", "").replace("lz::", "")
    return re.sub(r"\(.*$", "", n).strip()


def _rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_profiles(prof_dir, out_dir):
    """Turn four rocprofv3 runs of `bench.py PROFILE_ARGS` under prof_dir (kt: --kernel-trace
    --stats; fetch: --pmc FETCH_SIZE; write: --pmc WRITE_SIZE; mfma: --pmc of the matrix-core,
    LDS and busy counters) into profiles/traffic.json, profiles/counters.json and a text table."""
    import collections
    csrc = "gated_linear_attention_chunkwise_amd/csrc/"

    def per_kernel(sub, fname, counter=None):
        d = collections.defaultdict(list)
        for r in _rows(os.path.join(prof_dir, sub, fname)):
            key = (_kernel_key(r["Kernel_Name"]), int(r.get("Grid_Size") or r.get("Grid_Size_X")))
            if counter is None:
                d[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            elif r["Counter_Name"] == counter:
                d[key].append(float(r["Counter_Value"]))
        return d

    dur = per_kernel("kt", "run_kernel_trace.csv")
    fetch = per_kernel("fetch", "run_counter_collection.csv", "FETCH_SIZE")
    write = per_kernel("write", "run_counter_collection.csv", "WRITE_SIZE")
    pmc = {c: per_kernel("mfma", "run_counter_collection.csv", c)
           for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE", "SQ_INSTS_LDS",
                     "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES")}
    mean = lambda v: sum(v) / len(v)
    # calibration: the largest plain device copy in the runs (1 GiB read, 1 GiB written)
    copy = max((k for k in fetch if k[0].startswith("__amd_rocclr_copyBuffer")), key=lambda k: k[1])
    ff = (1 << 30) / (mean(fetch[copy]) * 1024)
    wf = (1 << 30) / (mean(write[copy]) * 1024)
    traffic = {"_calibration": {"copy_bytes": 1 << 30, "fetch_kib": mean(fetch[copy]), "write_kib": mean(write[copy]),
                                "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
                                "kernel": "__amd_rocclr_copyBuffer (torch copy_ of a 1 GiB bf16 tensor)"}}
    counters = {"_normalisation": (
        "mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 256 * 4): the matrix-core busy "
        "cycles summed over all SIMDs (16 per v_mfma_f32_16x16x32_bf16, = 16 * SQ_INSTS_MFMA) over the SIMD-cycles "
        "of the launch (GRBM_GUI_ACTIVE sums the busy cycles of the 8 XCDs; 256 CUs of 4 SIMDs)")}
    lines = []
    for name, tmpl, grid, src in PROFILED:
        key = (tmpl, grid)
        srcs = [csrc + "lz_common.hpp", csrc + "lz_kernels.hpp", csrc + src]
        sha = source_sha(srcs)
        launch = f"{tmpl}, {grid} threads"
        row = {"kernel": name, "launches": len(dur.get(key, []))}
        if key in dur:
            row["us_mean"] = mean(dur[key]) / 1e3
        if key in fetch and key in write:
            rb, wb = mean(fetch[key]) * 1024 * ff, mean(write[key]) * 1024 * wf
            traffic[name] = {"bytes_per_launch": round(rb + wb), "read_bytes": round(rb), "write_bytes": round(wb),
                             "launch": launch, "sources": srcs, "source_sha": sha}
            row.update(read_gb=rb / 1e9, write_gb=wb / 1e9)
        if all(key in pmc[c] for c in pmc):
            gui = mean(pmc["GRBM_GUI_ACTIVE"][key])
            busy = mean(pmc["SQ_VALU_MFMA_BUSY_CYCLES"][key])
            lds = mean(pmc["SQ_INSTS_LDS"][key])
            ent = {"mfma_busy_frac": round(busy / (gui / XCDS * CUS * SIMDS_PER_CU), 4),
                   "mfma_busy_cycles": busy, "mfma_insts": mean(pmc["SQ_INSTS_MFMA"][key]),
                   "gui_active_cycles_per_xcd": gui / XCDS,
                   "lds_insts": lds, "lds_bank_conflict_cycles": mean(pmc["SQ_LDS_BANK_CONFLICT"][key]),
                   "lds_bank_conflict_cycles_per_lds_inst": (round(mean(pmc["SQ_LDS_BANK_CONFLICT"][key]) / lds, 3)
                                                             if lds else None),
                   "launch": launch, "sources": srcs, "source_sha": sha}
            counters[name] = ent
            row.update(mfma_busy=ent["mfma_busy_frac"], conflicts_per_lds=ent["lds_bank_conflict_cycles_per_lds_inst"],
                       clock_ghz=(gui / XCDS) / (row["us_mean"] * 1e3) if "us_mean" in row else None)
        lines.append(row)
    if "decode_kernel" in traffic and "decode_pos_kernel" in traffic:
        a, b = traffic["decode_kernel"], traffic["decode_pos_kernel"]
        traffic["decode"] = {"bytes_per_launch": a["bytes_per_launch"] + b["bytes_per_launch"],
                             "read_bytes": a["read_bytes"] + b["read_bytes"],
                             "write_bytes": a["write_bytes"] + b["write_bytes"],
                             "launch": a["launch"] + " + " + b["launch"] + " (one decode step)",
                             "sources": a["sources"], "source_sha": a["source_sha"]}
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    with open(os.path.join(out_dir, "counters.json"), "w") as f:
        json.dump(counters, f, indent=1)
    cmd = f"python -u bench.py {PROFILE_ARGS}"
    txt = ["# train_8k forward+backward (B=4 H=32 L=8192 d=128 W=128 M=4, bf16) and decode_b64 (B=64 H=32 d=128):",
           "# kernel times, HBM bytes and matrix-core / LDS counters per launch",
           "#",
           "# made by (TMPDIR=/tmp, from the repository root), one run each:",
           f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/kt -o run -- {cmd}",
           f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o run -- {cmd}",
           f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o run -- {cmd}",
           "#   rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
           f"SQ_BUSY_CYCLES --output-format csv -d <dir>/mfma -o run -- {cmd}",
           "#   python bench.py --summarize-profiles <dir> --profiles-out profiles",
           "#",
           f"# HBM bytes: FETCH_SIZE x 1024 x {ff:.4f} (read), WRITE_SIZE x 1024 x {wf:.4f} (written); the factors make",
           "# the counters of a plain 1 GiB device copy in the same runs read 1 GiB each way.",
           "# " + counters["_normalisation"],
           "# clock = GRBM_GUI_ACTIVE / 8 over the trace's mean duration (a check of the normalisation).",
           "",
           f"{'kernel':24s}{'launches':>9s}{'us mean':>10s}{'read GB':>9s}{'write GB':>9s}{'GB/s':>8s}"
           f"{'MFMA busy':>11s}{'LDS confl/inst':>16s}{'clock GHz':>10s}"]
    for r in lines:
        gbs = ((r.get("read_gb", 0) + r.get("write_gb", 0)) / (r["us_mean"] * 1e-6)) if "us_mean" in r and "read_gb" in r else None
        f = lambda v, fmt: (fmt % v) if v is not None else "-"
        txt.append(f"{r['kernel']:24s}{r['launches']:>9d}{f(r.get('us_mean'), '%.1f'):>10s}{f(r.get('read_gb'), '%.3f'):>9s}"
                   f"{f(r.get('write_gb'), '%.3f'):>9s}{f(gbs, '%.0f'):>8s}{f(r.get('mfma_busy'), '%.4f'):>11s}"
                   f"{f(r.get('conflicts_per_lds'), '%.2f'):>16s}{f(r.get('clock_ghz'), '%.2f'):>10s}")
    with open(os.path.join(out_dir, "train_8k_and_decode_counters.txt"), "w") as f:
        f.write("\n".join(txt) + "\n")
    print("\n".join(txt))
    kt = ["# Kernel trace: train_8k forward+backward (B=4 H=32 L=8192 d=128 W=128 M=4, bf16) and decode_b64",
          "# (B=64 H=32 d=128, 16 steps after a 4096-token prefill)",
          "#",
          "# command (TMPDIR=/tmp, from the repository root):",
          f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/kt -o run -- {cmd}",
          "#   python bench.py --summarize-profiles <dir> --profiles-out profiles",
          "# durations in microseconds per launch (kernel trace start/end); grid in workgroups; the step's kernels",
          "# are the state sweeps (grid 256), out_kernel and chunk_kernel (grid 16384), the dmeta reduction and the",
          "# empty sub-block launches; grid 4096 / 131072 sweeps and outputs are the decode workload's prefill;",
          "# torch's own kernels (input generation) are left out.",
          ""]
    with open(os.path.join(out_dir, "train_8k_and_decode_kernel_trace.txt"), "w") as f:
        f.write("\n".join(kt + trace_table(os.path.join(prof_dir, "kt", "run_kernel_trace.csv"))) + "\n")


def trace_table(path):
    """Every kernel of a rocprofv3 kernel trace (csv), grouped by template and grid, as text rows."""
    import collections
    groups = collections.defaultdict(list)
    for r in _rows(path):
        if "at::" in r["Kernel_Name"]:
            continue   # torch's own kernels (input generation, copies)
        wg = int(r["Workgroup_Size_X"])
        key = (_kernel_key(r["Kernel_Name"])[:64], int(r["Grid_Size_X"]) // wg, wg, int(r["VGPR_Count"]),
               int(r["Accum_VGPR_Count"]), int(r["LDS_Block_Size"]))
        groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"{'kernel':66s}{'wgs':>8s}{'thr':>5s}{'vgpr':>6s}{'agpr':>6s}{'lds':>7s}{'calls':>7s}{'avg_us':>10s}"
           f"{'median_us':>11s}{'min_us':>10s}{'max_us':>10s}"]
    for key, v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        name, wgs, wg, vg, ag, lds = key
        out.append(f"{name:66s}{wgs:>8d}{wg:>5d}{vg:>6d}{ag:>6d}{lds:>7d}{len(v):>7d}{sum(v) / len(v):>10.1f}"
                   f"{median(v):>11.1f}{min(v):>10.1f}{max(v):>10.1f}")
    return out


ALL_SECTIONS_ARGS = "--steps 3 --warmup 1 --no-cpu-baseline --decode-steps 16"


def summarize_trace(prof_dir, out_dir, bench_log=None):
    """profiles/bench_all_sections_kernel_trace.txt from one rocprofv3 --kernel-trace run of
    `bench.py ALL_SECTIONS_ARGS` under prof_dir; bench_log (the run's stdout) adds its JSON line's
    per-section times."""
    cmd = f"python -u bench.py {ALL_SECTIONS_ARGS}"
    txt = ["# Kernel trace of every bench.py section: train_8k forward+backward (B=4 H=32 L=8192 d=128 W=128 M=4,",
           "# bf16), the backward that recomputes the forward's states, the step with log-sigmoid gates (sub-block",
           "# path), the scalar-gate step, the stage-1 step (layer + teacher_mse_kernel), the Hedgehog feature-map",
           "# step, fwd_4k (B=1 H=32 L=4096), decode_b64 (16 steps after a B=64 L=4096 prefill), prefill_64k one",
           "# shot and in 8 continued segments, and the gate projection (x [4,8192,4096], per key dimension",
           "# Ng=4096 and scalar Ng=32).",
           "#",
           "# command (TMPDIR=/tmp, from the repository root):",
           f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/kt -o run -- {cmd} > <dir>/bench.log",
           "#   python bench.py --summarize-trace <dir> --profiles-out profiles",
           "# durations in microseconds per launch (kernel trace start/end); grid in workgroups; the template",
           "# arguments are those of the kernels' declarations; one name with several grids covers several",
           "# sections; torch's own kernels (input generation) are left out.  vgpr is the trace's VGPR_Count,",
           "# which on gfx950 is half the compiler's per-lane count rounded up to its granule of 8 (230 -> 116).",
           ""]
    txt += trace_table(os.path.join(prof_dir, "kt", "run_kernel_trace.csv"))
    if bench_log and os.path.exists(bench_log):
        lines = [l for l in open(bench_log) if l.startswith("{")]
        if lines:
            rec = json.loads(lines[-1])
            txt += ["", "# times from the bench.py line of the same run (under the tracer, so a little slower):",
                    f"#   train step {rec['ms_per_step']} ms, {rec['value']} tokens/s; kernels_ms {rec.get('kernels_ms')}"]
            for sec, v in rec.items():
                if not isinstance(v, dict) or sec in ("config", "roofline", "kernels_ms", "step_roofline", "device",
                                                      "kernel_counters"):
                    continue
                nums = {k: x for k, x in v.items() if isinstance(x, (int, float)) and
                        (k.endswith("_ms") or k in ("ms_per_step", "us_per_step", "ms_saved", "ms_recomputed"))}
                for sub, x in v.items():
                    if isinstance(x, dict) and sub not in ("roofline",):
                        nums.update({f"{sub}.{k}": y for k, y in x.items() if isinstance(y, (int, float)) and
                                     (k.endswith("_ms") or k in ("ms", "us_per_step", "us_per_step_median"))})
                if nums:
                    txt.append(f"#   {sec}: " + ", ".join(f"{k} {y}" for k, y in nums.items()))
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "bench_all_sections_kernel_trace.txt"), "w") as f:
        f.write("\n".join(txt) + "\n")
    print("\n".join(txt[:40]))


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def _oracle_shard(args):
    """One (batch, head) shard of the oracle's forward + backward (process-pool worker)."""
    q, k, v, g, dO, mk, window, scale, dtype = args
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import lizard_oracle as orc
    dt = np.float64 if dtype == "fp64" else np.float32
    with threadpool_limits(1):
        t0 = time.perf_counter()
        orc.hybrid_forward(q, k, v, g, mk, None, window=window, scale=scale, dtype=dt)
        orc.hybrid_backward(q, k, v, g, mk, None, dO, window=window, scale=scale, dtype=dt)
        return time.perf_counter() - t0


def cpu_baseline(x, w, heads):
    """Time the oracle as it stands on a bounded sample of the step's work: all batches of `heads`
    heads at full length, forward + backward, on this host's cores.  Three ways: fp64 (the
    parity reference) and fp32 in one process with BLAS threads = cores, and fp32 as a process
    pool over (batch, head) shards with one worker per core (capped by the shards)."""
    import multiprocessing as mp
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import lizard_oracle as orc
    cores = len(os.sched_getaffinity(0))
    hs = {n: x[n][:, :heads].float().cpu().numpy() for n in ("q", "k", "v", "g", "dO")}
    mk = x["meta_k"][:heads].float().cpu().numpy()
    tokens = w.B * w.L * heads / w.H          # a token is one position through all H heads
    modes = {}
    for dtype, dt in (("fp64", np.float64), ("fp32", np.float32)):
        with threadpool_limits(cores):
            t0 = time.perf_counter()
            orc.hybrid_forward(hs["q"], hs["k"], hs["v"], hs["g"], mk, None, window=w.W, scale=w.scale, dtype=dt)
            orc.hybrid_backward(hs["q"], hs["k"], hs["v"], hs["g"], mk, None, hs["dO"], window=w.W,
                                scale=w.scale, dtype=dt)
            sec = time.perf_counter() - t0
        modes[f"{dtype}_one_process"] = {"tokens_per_s": round(tokens / sec, 1), "seconds": round(sec, 2),
                                         "cores": cores, "blas_threads": cores}
    shards = [(np.ascontiguousarray(hs["q"][b:b + 1, h:h + 1]), np.ascontiguousarray(hs["k"][b:b + 1, h:h + 1]),
               np.ascontiguousarray(hs["v"][b:b + 1, h:h + 1]), np.ascontiguousarray(hs["g"][b:b + 1, h:h + 1]),
               np.ascontiguousarray(hs["dO"][b:b + 1, h:h + 1]), mk[h:h + 1], w.W, w.scale, "fp32")
              for b in range(w.B) for h in range(heads)]
    workers = max(1, min(cores, len(shards)))
    ctx = mp.get_context("spawn")            # fresh interpreters: nothing of this process's GPU state
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_shard, shards[:workers])   # start-up and imports outside the timed region
        t0 = time.perf_counter()
        pool.map(_oracle_shard, shards)
        sec = time.perf_counter() - t0
    modes["fp32_process_pool"] = {"tokens_per_s": round(tokens / sec, 1), "seconds": round(sec, 2),
                                  "cores": workers, "workers": workers}
    best = max(modes, key=lambda m: modes[m]["tokens_per_s"])
    return {"value": modes[best]["tokens_per_s"], "unit": "tokens/s", "cores": modes[best]["cores"],
            "kind": "oracle", "mode": best, "modes": modes, "host_cores": cores,
            "sample": f"numpy oracle, forward+backward of {w.B * heads} of {w.B * w.H} (batch, head) pairs at "
                      f"full L={w.L} ({heads}/{w.H} of the step's work), tokens scaled by {heads}/{w.H}; "
                      f"value = the fastest of the three modes"}


def bench_train(args, hip, torch, lib):
    from gated_linear_attention_chunkwise_amd.inputs import WORKLOADS, make_inputs_device
    w = WORKLOADS["train_8k"]
    x = make_inputs_device(w, "cuda", with_grad=True)
    stream = torch.cuda.current_stream().cuda_stream

    def step(ev=None):
        if ev:
            hip.record(ev[0], stream)
        f = lib.lizard_attn_fwd(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, window=w.W,
                                scale=w.scale, want_lse=True, want_o_swa=True,
                                want_chunk_states=True)
        b = lib.lizard_attn_bwd(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, x["dO"], f["lse"],
                                f["o_swa"], f["chunk_states"], window=w.W, scale=w.scale,
                                stage_events=None if ev is None else [e.value for e in ev[1:]])
        return f, b

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[hip.event() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # forward = state sweep + output kernel(s); then the backward's three stages.  Every figure is
    # the median over the timed steps of HIP-event intervals on the kernels' stream.
    names = ["forward", "sweep_kernel_bwd", "chunk_kernel", "dmeta_kernels"]
    per = {n: [] for n in names}
    for ev in evs:
        for i, n in enumerate(names):
            per[n].append(hip.ms(ev[i], ev[i + 1]))
    avg = {n: median(v) for n, v in per.items()}
    ms_step = median([hip.ms(ev[0], ev[4]) for ev in evs])

    ht = w.B * w.H * w.L
    f_fwd, f_bwd = flops_per_head_token(w.L, w.D, w.chunk, w.W, w.M)
    flops_step = (f_fwd + f_bwd) * ht
    bytes_step = (FWD_BYTES + BWD_BYTES) * ht
    # dominant kernel (the backward chunk kernel, more than half of the step),
    # priced at the backward's compulsory bytes
    dom = "chunk_kernel"
    dom_bytes = BWD_BYTES * ht
    achieved = dom_bytes / (avg[dom] * 1e-3) / 1e9
    traffic = load_traffic(dom)
    counters = {k: load_counters(k) for k in ("sweep_kernel_fwd", "out_kernel", "sweep_kernel_bwd", "chunk_kernel")}
    return w, {
        "ms_per_step": ms_step,
        "ms_per_step_wall_mean": wall * 1e3 / args.steps,
        "value": w.B * w.L / (ms_step * 1e-3),
        "kernels_ms": {n: round(v, 4) for n, v in avg.items()},
        "dominant": dom,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": dom, "algorithmic_bytes_per_launch": dom_bytes,
                     "mfma_busy_frac": (counters[dom] or {}).get("mfma_busy_frac")},
        "counters": counters,
        "step_roofline": {
            "flop": flops_step, "bytes": bytes_step,
            "mfma_frac": round(flops_step / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
            "hbm_frac": round(bytes_step / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
            "ideal_ms": round(max(flops_step / (PEAK_BF16_TFLOPS * 1e12), bytes_step / (PEAK_HBM_GBS * 1e9)) * 1e3, 4),
            # fraction of the attainable roofline: max(FLOP/peak, bytes/bandwidth) / measured time
            "attainable_frac": round(max(flops_step / (PEAK_BF16_TFLOPS * 1e12),
                                         bytes_step / (PEAK_HBM_GBS * 1e9)) / (ms_step * 1e-3), 4),
        },
    }, x


def bench_fwd_8b(args, hip, torch, lib):
    """The 8B-shaped forward, B=1 H=32 L=4096 d=128 (fwd_4k).  Its working set (201 MB) fits the
    256 MB last-level cache, so besides back-to-back forwards each is also timed alone after a
    read of 1 GiB elsewhere (cold cache); both are medians of HIP-event intervals."""
    from gated_linear_attention_chunkwise_amd.inputs import WORKLOADS, make_inputs_device
    w = WORKLOADS["fwd_4k"]
    x = make_inputs_device(w, "cuda")
    stream = torch.cuda.current_stream().cuda_stream
    o = torch.empty_like(x["q"])
    s = lib.make_shape(w.B, w.H, w.L, w.D, w.W, w.M, w.scale, 1.0, torch.bfloat16)
    nws = lib.workspace_bytes(s, lib.OP_FWD)
    ws = torch.empty(nws, device="cuda", dtype=torch.uint8)
    raw = lib.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    args_c = (ctypes.byref(s), P(x["q"]), P(x["k"]), P(x["v"]), P(x["g"]), P(x["meta_k"]), None, P(o), None,
              None, None, None, P(ws), nws, ctypes.c_void_p(stream))

    def fwd():   # the C entry point itself: outputs and workspace allocated once, outside the loop
        rc = raw.lizard_attn_fwd(*args_c)
        if rc != 0:
            raise RuntimeError(f"lizard_attn_fwd returned {rc}")

    for _ in range(5):
        fwd()
    n = max(5, args.steps)
    evs = [(hip.event(), hip.event()) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in evs:
        hip.record(a, stream)
        fwd()
        hip.record(b, stream)
    torch.cuda.synchronize()
    warm = median([hip.ms(a, b) for a, b in evs])
    flush = torch.ones(1 << 28, device="cuda", dtype=torch.float32)
    cold = []
    for _ in range(n):
        float(flush.max())
        a, b = hip.event(), hip.event()
        hip.record(a, stream)
        fwd()
        hip.record(b, stream)
        torch.cuda.synchronize()
        cold.append(hip.ms(a, b))
    del flush
    cold = median(cold)
    ht = w.B * w.H * w.L
    f_fwd, _ = flops_per_head_token(w.L, w.D, w.chunk, w.W, w.M)
    flop, byt = f_fwd * ht, FWD_BYTES * ht

    def fr(ms):
        return {"ms": round(ms, 4), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
                "mfma_frac": round(flop / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
                "hbm_frac": round(byt / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
                "attainable_frac": round(max(flop / (PEAK_BF16_TFLOPS * 1e12), byt / (PEAK_HBM_GBS * 1e9))
                                         / (ms * 1e-3), 4)}
    return {"workload": f"fwd_4k: B={w.B} H={w.H} L={w.L} d={w.D} W={w.W} M={w.M} chunk={w.chunk}, forward, "
                        "bf16 activations, fp32 gates",
            "flop": flop, "bytes": byt, "warm": fr(warm), "cold_cache": fr(cold),
            "method": "medians of HIP-event intervals: back-to-back forwards (warm), and single forwards "
                      "after a read of 1 GiB elsewhere (cold)"}


def bench_bwd_recompute(args, hip, torch, lib, x, w):
    """The training step's backward without the forward's saved tensors (lse, o_swa, chunk
    states recomputed inside the backward) against the backward from them."""
    stream = torch.cuda.current_stream().cuda_stream
    f = lib.lizard_attn_fwd(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, window=w.W, scale=w.scale,
                            want_lse=True, want_o_swa=True, want_chunk_states=True)
    saved = {"lse": f["lse"], "o_swa": f["o_swa"], "chunk_states": f["chunk_states"]}
    res = {}
    for name, kw in (("saved", saved), ("recomputed", {})):
        def bwd():
            lib.lizard_attn_bwd(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, x["dO"], window=w.W,
                                scale=w.scale, **kw)
        for _ in range(2):
            bwd()
        n = max(3, min(args.steps, 10))
        evs = [(hip.event(), hip.event()) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in evs:
            hip.record(a, stream)
            bwd()
            hip.record(b, stream)
        torch.cuda.synchronize()
        res[name] = median([hip.ms(a, b) for a, b in evs])
    kept = sum(t.numel() * t.element_size() for t in saved.values())
    return {"workload": "train_8k backward", "ms_saved": round(res["saved"], 4),
            "ms_recomputed": round(res["recomputed"], 4),
            "saved_tensor_bytes": kept,
            "note": "recomputing lse, o_swa and the chunk states costs the difference in time and saves "
                    "saved_tensor_bytes of memory kept between the passes per layer"}


def bench_strong_gates(args, hip, torch, lib, x, w):
    """The training step with the pages' own gate at temperature 1, g = log sigmoid(z) with
    pre-activations z ~ N(-1, 1): chunk sums near -86, so almost every chunk takes the 16-token
    sub-block path."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    z = torch.randn(x["g"].shape, generator=gen, device="cuda", dtype=torch.float32) - 1.0
    g = torch.nn.functional.logsigmoid(z)
    del z
    strong = float((g.reshape(w.B, w.H, w.L // 64, 64, w.D).sum(3).amin(-1) < -64).float().mean())
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        f = lib.lizard_attn_fwd(x["q"], x["k"], x["v"], g, x["meta_k"], None, window=w.W, scale=w.scale,
                                want_lse=True, want_o_swa=True, want_chunk_states=True)
        lib.lizard_attn_bwd(x["q"], x["k"], x["v"], g, x["meta_k"], None, x["dO"], f["lse"], f["o_swa"],
                            f["chunk_states"], window=w.W, scale=w.scale)
    for _ in range(2):
        step()
    n = max(3, min(args.steps, 10))
    evs = [(hip.event(), hip.event()) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in evs:
        hip.record(a, stream)
        step()
        hip.record(b, stream)
    torch.cuda.synchronize()
    ms = median([hip.ms(a, b) for a, b in evs])
    return {"workload": f"train_8k with g = log sigmoid(z), z ~ N(-1, 1) (tau = 1): B={w.B} H={w.H} L={w.L} "
                        f"d={w.D}, forward+backward",
            "strong_chunk_fraction": round(strong, 4), "ms_per_step": round(ms, 4),
            "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1)}


# compulsory bytes per head-token with one gate per head and token (4 B of gate, 4 B of dg)
FWD_BYTES_SCALAR = 3 * 2 * 128 + 4 + 2 * 128                  # 1028
BWD_BYTES_SCALAR = 4 * 2 * 128 + 4 + 3 * 2 * 128 + 4           # 1800


def bench_scalar_gate(args, hip, torch, lib, x, w):
    """The same training step with one log-gate per head and token (g, dg [B,H,L])."""
    g = x["g"][..., 0].contiguous()
    stream = torch.cuda.current_stream().cuda_stream

    def step(ev=None):
        f = lib.lizard_attn_fwd(x["q"], x["k"], x["v"], g, x["meta_k"], None, window=w.W, scale=w.scale,
                                want_lse=True, want_o_swa=True, want_chunk_states=True)
        lib.lizard_attn_bwd(x["q"], x["k"], x["v"], g, x["meta_k"], None, x["dO"], f["lse"], f["o_swa"],
                            f["chunk_states"], window=w.W, scale=w.scale,
                            stage_events=None if ev is None else [e.value for e in ev])

    for _ in range(3):
        step()
    steps = max(1, min(args.steps, 10))
    evs = [[hip.event() for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for k in range(steps):
        step(evs[k])
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.ms(e0, e1) / steps
    chunk_ms = sum(hip.ms(ev[1], ev[2]) for ev in evs) / steps
    ht = w.B * w.H * w.L
    step_bytes = (FWD_BYTES_SCALAR + BWD_BYTES_SCALAR) * ht
    ck = BWD_BYTES_SCALAR * ht / (chunk_ms * 1e-3) / 1e9
    return {"workload": f"train_8k with one log-gate per head and token: B={w.B} H={w.H} L={w.L} d={w.D} "
                        f"W={w.W} M={w.M}, forward+backward",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
            "chunk_kernel_ms": round(chunk_ms, 4),
            "step_hbm_frac": round(step_bytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
            "roofline": {"bound": "hbm", "achieved": round(ck, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(ck / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "chunk_kernel",
                         "algorithmic_bytes_per_launch": BWD_BYTES_SCALAR * ht}}


def bench_decode(args, hip, torch, lib):
    from gated_linear_attention_chunkwise_amd.inputs import WORKLOADS, make_inputs_device
    w = WORKLOADS["decode_b64"]
    x = make_inputs_device(w, "cuda")
    P, L = w.prefill, w.L
    pre = {n: x[n][:, :, :P].contiguous() for n in ("q", "k", "v", "g")}
    f = lib.lizard_attn_fwd(pre["q"], pre["k"], pre["v"], pre["g"], x["meta_k"], None, window=w.W,
                            scale=w.scale, want_state=True)
    state = f["state"]
    ring_k = torch.zeros(w.B, w.H, w.W, w.D, device="cuda", dtype=torch.bfloat16)
    ring_v = torch.zeros_like(ring_k)
    ts = torch.arange(P - w.W, P, device="cuda")
    ring_k[:, :, ts % w.W] = pre["k"][:, :, ts]
    ring_v[:, :, ts % w.W] = pre["v"][:, :, ts]
    pos = torch.full((w.B,), P, device="cuda", dtype=torch.int32)
    steps = L - P if args.decode_steps is None else min(args.decode_steps, L - P)
    tok = {n: x[n][:, :, P:P + steps].permute(2, 0, 1, 3).contiguous() for n in ("q", "k", "v", "g")}
    mk = x["meta_k"]
    out = torch.empty(steps, w.B, w.H, w.D, device="cuda", dtype=torch.bfloat16)
    ws = lib.decode_workspace(w.B, w.H, w.D, "cuda")
    del x, pre, f
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for t in range(steps):
        lib.lizard_attn_decode_step(tok["q"][t], tok["k"][t], tok["v"][t], tok["g"][t], mk,
                                    None, state, ring_k, ring_v, pos, window=w.W, scale=w.scale, out=out[t],
                                    workspace=ws)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    us = hip.ms(e0, e1) * 1e3 / steps
    # cold cache: the state and ring (268 MB) nearly fit the 256 MB last-level cache, so back-to-back
    # steps may read part of them from it.  Each of these steps runs on its own after a
    # synchronisation; "isolated" follows nothing else, "cold" follows a read of 1 GiB elsewhere
    # (clean lines: nothing left to write back), so their difference is the cache's share.
    flush = torch.ones(1 << 28, device="cuda", dtype=torch.float32)
    cold, iso = [], []
    ncold = min(16, steps)

    def one_step(t):
        ea, eb = hip.event(), hip.event()
        hip.record(ea, stream)
        lib.lizard_attn_decode_step(tok["q"][t], tok["k"][t], tok["v"][t], tok["g"][t], mk,
                                    None, state, ring_k, ring_v, pos, window=w.W, scale=w.scale, out=out[t],
                                    workspace=ws)
        hip.record(eb, stream)
        torch.cuda.synchronize()
        return hip.ms(ea, eb) * 1e3

    for t in range(ncold):
        torch.cuda.synchronize()
        iso.append(one_step(t))
        float(flush.max())
        cold.append(one_step(t))
    del flush
    us_cold = sorted(cold)[len(cold) // 2]
    us_iso = sorted(iso)[len(iso) // 2]
    # the step sequence captured once in a HIP graph (kernel nodes only) and replayed: no host
    # launch work between steps
    ng = min(64, steps)
    gstream = torch.cuda.Stream()
    gstream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        with torch.cuda.graph(graph, stream=gstream):
            for t in range(ng):
                lib.lizard_attn_decode_step(tok["q"][t], tok["k"][t], tok["v"][t], tok["g"][t], mk, None, state,
                                            ring_k, ring_v, pos, window=w.W, scale=w.scale, out=out[t], workspace=ws)
    torch.cuda.current_stream().wait_stream(gstream)
    graph.replay()
    torch.cuda.synchronize()
    reps = 5
    ga, gb = hip.event(), hip.event()
    hip.record(ga, stream)
    for _ in range(reps):
        graph.replay()
    hip.record(gb, stream)
    torch.cuda.synchronize()
    us_graph = hip.ms(ga, gb) * 1e3 / (reps * ng)
    del graph
    d = w.D
    bytes_step = (2 * w.B * w.H * d * d * 4 + 2 * w.B * w.H * w.W * d * 2
                  + 4 * w.B * w.H * d * 2 + w.B * w.H * d * 4 + 2 * w.B * w.H * d * 2)
    gbs = bytes_step / (us * 1e-6) / 1e9
    return {"workload": f"decode_b64: B={w.B} H={w.H} d={d} fp32 state, W={w.W} bf16 ring, M={w.M}; "
                        f"{steps} steps after a {P}-token prefill",
            "tokens_per_s": round(w.B / (us * 1e-6), 1), "us_per_step": round(us, 2),
            "graph": {"us_per_step": round(us_graph, 2), "steps_per_graph": ng,
                      "hbm_frac": round(bytes_step / (us_graph * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
            "cold_cache": {"us_per_step_median": round(us_cold, 2), "isolated_us_per_step_median": round(us_iso, 2),
                           "steps": ncold,
                           "hbm_frac": round(bytes_step / (us_cold * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                           "method": "single steps after a synchronisation, with (cold) and without (isolated) "
                                     "a read of 1 GiB elsewhere first"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": load_traffic("decode"),
                         "kernel": "decode_kernel + decode_pos_kernel",
                         "algorithmic_bytes_per_step": bytes_step}}


def bench_prefill(args, hip, torch, lib):
    """Forward of the 65 536-token prefill, one shot and as continued 8192-token segments
    (chunked prefill carrying state, key/value ring and position between calls)."""
    from gated_linear_attention_chunkwise_amd.inputs import WORKLOADS, make_inputs_device
    w = WORKLOADS["prefill_64k"]
    x = make_inputs_device(w, "cuda")
    S = 8192
    segs = [{n: x[n][:, :, a:a + S].contiguous() for n in ("q", "k", "v", "g")} for a in range(0, w.L, S)]
    mk = x["meta_k"]
    state = torch.zeros(w.B, w.H, w.D, w.D, device="cuda", dtype=torch.float32)
    ring_k = torch.zeros(w.B, w.H, w.W, w.D, device="cuda", dtype=torch.bfloat16)
    ring_v = torch.zeros_like(ring_k)
    pos = torch.zeros(w.B, device="cuda", dtype=torch.int32)
    ws = lib.continue_workspace(w.B, w.H, S, w.D, torch.bfloat16, "cuda")
    outs = [torch.empty_like(sg["q"]) for sg in segs]
    stream = torch.cuda.current_stream().cuda_stream

    def one_shot():
        lib.lizard_attn_fwd(x["q"], x["k"], x["v"], x["g"], mk, None, window=w.W, scale=w.scale)

    def chunked():
        state.zero_()
        pos.zero_()
        for sg, o in zip(segs, outs):
            lib.lizard_attn_fwd_continue(sg["q"], sg["k"], sg["v"], sg["g"], mk, None, state, ring_k, ring_v,
                                         pos, window=w.W, scale=w.scale, out=o, workspace=ws)

    res = {}
    reps = 5
    for name, fn in (("one_shot", one_shot), ("chunked", chunked)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for _ in range(reps):
            fn()
        hip.record(e1, stream)
        torch.cuda.synchronize()
        res[name] = hip.ms(e0, e1) / reps
    tokens = w.B * w.L
    alg = FWD_BYTES * w.B * w.H * w.L
    gbs = alg / (res["chunked"] * 1e-3) / 1e9
    return {"workload": f"prefill_64k: B={w.B} H={w.H} L={w.L} d={w.D} W={w.W} M={w.M}, gate input N(2,1); "
                        f"chunked = {w.L // S} continued segments of {S} tokens",
            "one_shot": {"ms": round(res["one_shot"], 4), "tokens_per_s": round(tokens / res["one_shot"] * 1e3, 1)},
            "chunked": {"ms": round(res["chunked"], 4), "tokens_per_s": round(tokens / res["chunked"] * 1e3, 1)},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                         "kernel": "chunked prefill (sweep + out kernel + ring update per segment)",
                         "algorithmic_bytes": alg}}


def bench_gate_proj(args, hip, torch, lib):
    """The gate projection g = log sigmoid(x W^T)/16 at the train shape (d_model = 4096 for H = 32
    heads of d = 128), forward + backward, per key dimension (Ng = 4096) and scalar (Ng = 32)."""
    from gated_linear_attention_chunkwise_amd.inputs import make_gate_device
    B, L, Dm, H, dk, tau = 4, 8192, 4096, 32, 128, 16.0
    T = B * L
    stream = torch.cuda.current_stream().cuda_stream
    out = {"workload": f"gate projection at train_8k: x [{B},{L},{Dm}] bf16, W [Ng,{Dm}] bf16, tau {tau:g}; "
                       "forward + backward (dz pass, dx = dz W, dW = dz^T x)"}
    for scalar in (False, True):
        ng = H if scalar else H * dk
        gshape = (B, H, L) if scalar else (B, H, L, dk)
        t = make_gate_device(B, L, Dm, ng, gshape, seed=77, device="cuda", dtype=torch.bfloat16)
        ws = lib.gate_proj_workspace((B, L, Dm), H, dk, torch.bfloat16, "cuda", scalar=scalar)
        g = lib.lizard_gate_proj_fwd(t["x"], t["w"], heads=H, d_k=dk, tau=tau, scalar=scalar)

        def fwd():
            return lib.lizard_gate_proj_fwd(t["x"], t["w"], heads=H, d_k=dk, tau=tau, scalar=scalar)

        def bwd():
            return lib.lizard_gate_proj_bwd(t["x"], t["w"], g, t["dg"], heads=H, d_k=dk, tau=tau,
                                            scalar=scalar, workspace=ws)
        for _ in range(2):
            fwd()
            bwd()
        torch.cuda.synchronize()
        n = max(2, min(args.steps, 10))
        e = [hip.event() for _ in range(3)]
        hip.record(e[0], stream)
        for _ in range(n):
            fwd()
        hip.record(e[1], stream)
        for _ in range(n):
            bwd()
        hip.record(e[2], stream)
        torch.cuda.synchronize()
        tf, tb = hip.ms(e[0], e[1]) / n, hip.ms(e[1], e[2]) / n
        flop_f = 2.0 * T * Dm * ng
        # compulsory bytes: forward x, W in, g out; backward x, W, g, dg in, dx, dW out
        bytes_f = T * Dm * 2 + ng * Dm * 2 + T * ng * 4
        bytes_b = T * Dm * 2 + ng * Dm * 2 + 2 * T * ng * 4 + T * Dm * 2 + ng * Dm * 4
        rec = {"Ng": ng, "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4),
               "tokens_per_s": round(T / ((tf + tb) * 1e-3), 1)}
        if scalar:
            gbs = (bytes_f + bytes_b) / ((tf + tb) * 1e-3) / 1e9
            rec["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                               "kernel": "gate projection forward + backward (skinny products, bound by x and dx)",
                               "algorithmic_bytes": bytes_f + bytes_b}
        else:
            tfs = 3 * flop_f / ((tf + tb) * 1e-3) / 1e12
            rec["roofline"] = {"bound": "mfma", "achieved": round(tfs, 1), "peak": PEAK_BF16_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(tfs / PEAK_BF16_TFLOPS, 4), "traffic": None,
                               "kernel": "gate projection forward + backward (three bf16 products of 2*T*d_model*Ng)",
                               "algorithmic_flop": 3 * flop_f}
        out["scalar" if scalar else "per_dim"] = rec
        del t, ws, g
        torch.cuda.empty_cache()
    return out


def bench_stage1(args, hip, torch, lib, x, w):
    """The stage-1 attention-approximation step at the train shape: the layer forward, the teacher's
    causal softmax attention with the MSE fused in (lizard_distill_mse), the layer backward from dO."""
    stream = torch.cuda.current_stream().cuda_stream
    ws = torch.empty(w.B * w.H * ((w.L + 127) // 128) * 4, device="cuda", dtype=torch.uint8)

    def step(ev=None):
        f = lib.lizard_attn_fwd(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, window=w.W, scale=w.scale,
                                want_lse=True, want_o_swa=True, want_chunk_states=True)
        if ev:
            hip.record(ev[0], stream)
        ls = lib.lizard_distill_mse(x["q"], x["k"], x["v"], f["o"], scale=w.scale, workspace=ws)
        if ev:
            hip.record(ev[1], stream)
        lib.lizard_attn_bwd(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, ls["dO"], f["lse"], f["o_swa"],
                            f["chunk_states"], window=w.W, scale=w.scale)

    for _ in range(2):
        step()
    steps = max(2, min(args.steps, 10))
    evs = [[hip.event() for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for k in range(steps):
        step(evs[k])
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.ms(e0, e1) / steps
    t_mse = sum(hip.ms(ev[0], ev[1]) for ev in evs) / steps
    flop = 4.0 * w.B * w.H * w.D * w.L * (w.L + 1) / 2     # teacher Q K^T and P V over the causal triangle
    tf = flop / (t_mse * 1e-3) / 1e12
    return {"workload": f"stage-1 step at train_8k: B={w.B} H={w.H} L={w.L} d={w.D} W={w.W} M={w.M}; teacher = "
                        "causal softmax attention of the same q, k, v",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
            "teacher_mse_ms": round(t_mse, 4),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                         "kernel": "teacher_mse_kernel (causal attention + MSE epilogue)", "algorithmic_flop": flop}}


def bench_features(args, hip, torch, lib, x, w):
    """The layer with a Hedgehog feature map on the GLA branch at the train shape: the map for q and
    k (log features), the log-feature layer forward + backward, the map's backward for q and k."""
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    Wq = (torch.randn(w.H, w.D, w.D // 2, generator=gen, device="cuda") * 8.0 / math.sqrt(w.D)).to(x["q"].dtype)
    Wk = (torch.randn(w.H, w.D, w.D // 2, generator=gen, device="cuda") * 8.0 / math.sqrt(w.D)).to(x["q"].dtype)
    ws = torch.empty(lib.workspace_bytes(lib.make_shape(w.B, w.H, w.L, w.D, 1, 0, 1.0, 1.0, x["q"].dtype),
                                         lib.OP_FEATURE_BWD), device="cuda", dtype=torch.uint8)

    def step(ev=None):
        if ev:
            hip.record(ev[0], stream)
        lq = lib.lizard_hedgehog_fwd(x["q"], Wq)
        lk = lib.lizard_hedgehog_fwd(x["k"], Wk)
        if ev:
            hip.record(ev[1], stream)
        f = lib.lizard_attn_fwd_feat(x["q"], x["k"], x["v"], lq, lk, x["g"], x["meta_k"], None, window=w.W,
                                     scale=w.scale, want_lse=True, want_o_swa=True, want_chunk_states=True)
        b = lib.lizard_attn_bwd_feat(x["q"], x["k"], x["v"], lq, lk, x["g"], x["meta_k"], None, x["dO"], f["lse"],
                                     f["o_swa"], f["chunk_states"], window=w.W, scale=w.scale)
        if ev:
            hip.record(ev[2], stream)
        lib.lizard_hedgehog_bwd(x["q"], Wq, b["dlq"], workspace=ws)
        lib.lizard_hedgehog_bwd(x["k"], Wk, b["dlk"], workspace=ws)
        if ev:
            hip.record(ev[3], stream)

    for _ in range(2):
        step()
    steps = max(2, min(args.steps, 10))
    evs = [[hip.event() for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    t = [sum(hip.ms(ev[i], ev[i + 1]) for ev in evs) / steps for i in range(3)]
    ms = sum(t)
    ht = w.B * w.H * w.L
    # feature map: x bf16 in, fp32 log features out (forward); x, fp32 dl in, dx out (backward); q and k each
    fbytes = 2 * ht * (2 * w.D + 4 * w.D)
    bbytes = 2 * ht * (2 * w.D + 4 * w.D + 2 * w.D)
    gbs = (fbytes + bbytes) / ((t[0] + t[2]) * 1e-3) / 1e9
    return {"workload": f"train_8k with a Hedgehog map on the GLA branch (log features, W_q, W_k [{w.H},{w.D},"
                        f"{w.D // 2}]); map forward for q, k + layer forward/backward + map backward for q, k",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
            "feature_map_fwd_ms": round(t[0], 4), "layer_fwd_bwd_ms": round(t[1], 4),
            "feature_map_bwd_ms": round(t[2], 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                         "kernel": "hedgehog_fwd_kernel + hedgehog_bwd_kernel (q and k)",
                         "algorithmic_bytes": fbytes + bbytes}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-scalar-gate", action="store_true")
    ap.add_argument("--no-gate-proj", action="store_true")
    ap.add_argument("--no-stage1", action="store_true")
    ap.add_argument("--no-features", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fwd-8b", action="store_true")
    ap.add_argument("--no-recompute", action="store_true")
    ap.add_argument("--no-strong-gates", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=2, help="heads in the oracle timing sample")
    ap.add_argument("--decode-steps", type=int, default=None, help="decode steps (default: the workload's)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference kernel for HBM byte counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="summarise rocprofv3 runs under DIR (kt, fetch, write, mfma) instead of measuring")
    ap.add_argument("--summarize-trace", metavar="DIR", default=None,
                    help="summarise one rocprofv3 --kernel-trace run of every section under DIR/kt instead of measuring")
    ap.add_argument("--profiles-out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.profiles_out, os.path.join(args.summarize_trace, "bench.log"))
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.profiles_out)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards over batch and heads with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_linear_attention_chunkwise_amd as lib
    lib.load()
    hip = Hip()
    w, tr, x = bench_train(args, hip, torch, lib)
    rec = {
        "metric": METRIC, "value": round(tr["value"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(tr["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"train_8k: B={w.B} H={w.H} L={w.L} d={w.D} W={w.W} M={w.M} chunk={w.chunk}, "
                               "forward+backward, bf16 activations, fp32 gates",
                   "global_batch": w.B, "seq_len": w.L, "parallelism": "none (1 GPU)"},
        "roofline": tr["roofline"],
        "kernels_ms": tr["kernels_ms"],
        "step_roofline": tr["step_roofline"],
        "kernel_counters": tr["counters"],
    }
    props = torch.cuda.get_device_properties(0)
    rec["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                     "compute_units": props.multi_processor_count, "l2_bytes": getattr(props, "L2_cache_size", None),
                     "hbm_bytes": props.total_memory,
                     "peaks_used": {"hbm_GBs": PEAK_HBM_GBS, "bf16_dense_TFLOPs": PEAK_BF16_TFLOPS,
                                    "basis": "256 CUs x 2.4 GHz x 4096 bf16 FLOP/clk/CU; the engine clock seen by "
                                             "the counters is in profiles/train_8k_and_decode_counters.txt"}}
    if args.copy_calibration:
        src = torch.empty(1 << 29, device="cuda", dtype=torch.bfloat16).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, w, args.cpu_heads)
    if not args.no_scalar_gate:
        rec["scalar_gate"] = bench_scalar_gate(args, hip, torch, lib, x, w)
    if not args.no_recompute:
        rec["bwd_recompute"] = bench_bwd_recompute(args, hip, torch, lib, x, w)
        torch.cuda.empty_cache()
    if not args.no_strong_gates:
        rec["strong_gates"] = bench_strong_gates(args, hip, torch, lib, x, w)
        torch.cuda.empty_cache()
    if not args.no_stage1:
        rec["stage1"] = bench_stage1(args, hip, torch, lib, x, w)
    if not args.no_features:
        rec["features"] = bench_features(args, hip, torch, lib, x, w)
    del x
    torch.cuda.empty_cache()
    if not args.no_fwd_8b:
        rec["fwd_8b"] = bench_fwd_8b(args, hip, torch, lib)
        torch.cuda.empty_cache()
    if not args.no_decode:
        rec["decode"] = bench_decode(args, hip, torch, lib)
        torch.cuda.empty_cache()
    if not args.no_prefill:
        rec["prefill"] = bench_prefill(args, hip, torch, lib)
        torch.cuda.empty_cache()
    if not args.no_gate_proj:
        rec["gate_proj"] = bench_gate_proj(args, hip, torch, lib)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
