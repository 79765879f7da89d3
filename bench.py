"""KDA prefill + verify benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--iters N]

One step is one pass of the whole hot path over one batch of synthetic input:
  * varlen chunked prefill of 4 sequences x 8192 tokens, H = 16, d = 128 (zero
    start state, fp32 final states): one kda_chunk_prefill call (the intra-chunk
    kernel, then the state-scan kernel);
  * fused verify of 64 rows x 8 draft tokens, H = 16, states gathered from a
    256-slot fp32 pool, per-step fp32 states written (kda_recurrent_verify).
Inputs are resident in HBM before timing starts.  Each call is bracketed by HIP
events on the stream it is launched on (torch's current stream, which the
binding hands to libkda); per-layer figures are medians.  Prints ONE JSON line
on stdout; progress goes to stderr.

`value` is prefill tokens/s at 4x8192 (the headline shape), and `roofline` is
that call's: its algorithmic bytes (1282 B per token-head plus the final states)
over the call's median time.  `configs` repeats the measurement per workload --
8 x 2048 with start states, 4 x 8192, 1 x 16384 with a gathered start state and
the verify -- as medians of at least 50 calls, warm and cold (1 GiB overwritten,
or read, before each call), with each prefill's two kernels also timed alone.
The oracle (fp64 CPU token loop) is timed on a bounded sample of the 4 x 8192
workload as `cpu_baseline`.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import re
import resource
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_attention_rule_amd import (causal_conv1d_prefill,  # noqa: E402
                                       causal_conv1d_update, chunk_prefill, commit_accepted,
                                       gated_rmsnorm, prefill_workspace_bytes,
                                       recurrent_verify, recurrent_verify_gated)
from linear_attention_rule_amd import workloads as W  # noqa: E402

METRIC = "KDA prefill µs/layer & tokens/s (8192x4, H=16, d=128); verify µs/layer"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16/fp16 MFMA
D = 128
# Algorithmic bytes per token-head: q, k, v, g (bf16, 4 x 256 B) + beta logit (2 B) + out (256 B).
BYTES_PER_TOKEN_HEAD = 4 * 2 * D + 2 + 2 * D
STATE_BYTES = 4 * D * D
# Algorithmic prefill MFMA flops per token-head at chunk 64 (triangular products at half).
FLOPS_PER_TOKEN_HEAD = 5 * 64 * D + 6 * D * D


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(data):
    return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in data.items()}


def cpu_baseline(case, tokens_per_seq):
    """Time the fp64 oracle on all sequences x all heads of `case`, first `tokens_per_seq` tokens."""
    from oracle import kda_oracle as O
    data = W.make_prefill(case)
    cu = data["cu_seqlens"].numpy().astype(np.int64)
    tokens_per_seq = min(tokens_per_seq, int(np.min(np.diff(cu))))
    rows = np.concatenate([np.arange(cu[n], cu[n] + tokens_per_seq) for n in range(len(cu) - 1)])
    f = W.to_f64
    sub_cu = np.arange(0, len(rows) + 1, tokens_per_seq)
    args = (f(data["q"])[rows], f(data["k"])[rows], f(data["v"])[rows], f(data["g"])[rows],
            f(data["beta_logits"])[rows], f(data["A_log"]), f(data["dt_bias"]), data["lower_bound"],
            sub_cu)
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    O.chunk_prefill(*args, scale=data["scale"])
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    tokens = len(rows)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": tokens / wall, "unit": "tokens/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle", "wall_s": round(wall, 2), "cpu_model": model,
            "sample": f"{case.name}: all {len(cu) - 1} sequences x {case.heads} heads, first "
                      f"{tokens_per_seq} tokens of each ({tokens} tokens, {wall:.1f} s wall, "
                      f"fp64 numpy token loop, {os.cpu_count()} host CPUs visible)"}


KERNEL_SOURCES = {
    "kda_prefill_intra": ("linear_attention_rule_amd/csrc/kda_prefill_intra.hip",
                          "linear_attention_rule_amd/csrc/kda_prefill_common.h"),
    "kda_prefill_scan": ("linear_attention_rule_amd/csrc/kda_prefill_scan.hip",
                         "linear_attention_rule_amd/csrc/kda_prefill_common.h"),
    "kda_verify": ("linear_attention_rule_amd/csrc/kda_verify.hip",),
    "kda_commit": ("linear_attention_rule_amd/csrc/kda_commit.hip",),
    "kda_seg_combine": ("linear_attention_rule_amd/csrc/kda_prefill_scan.hip",),
    "kda_gated_rmsnorm": ("linear_attention_rule_amd/csrc/kda_norm.hip",),
    "kda_conv_prefill": ("linear_attention_rule_amd/csrc/kda_conv.hip",),
    "kda_conv_state": ("linear_attention_rule_amd/csrc/kda_conv.hip",),
    "kda_conv_update": ("linear_attention_rule_amd/csrc/kda_conv.hip",),
}
# rocprofv3 kernel names -> the names used in this benchmark.
KERNEL_PATTERNS = {
    "kda_prefill_intra": "prefill_intra_kernel",
    "kda_prefill_scan": "prefill_scan_kernel",
    "kda_verify": "::verify_",   # the step and the block form
    "kda_commit": "commit_kernel",
    "kda_seg_combine": "seg_combine_kernel",
    "kda_gated_rmsnorm": "gated_rmsnorm_kernel",
    "kda_conv_prefill": "conv_prefill_kernel",
    "kda_conv_state": "conv_state_kernel",
    "kda_conv_update": "conv_update_kernel",
}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CALIB_BYTES = 1 << 30


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in (*KERNEL_SOURCES[kernel], "linear_attention_rule_amd/csrc/kda_internal.h",
                "linear_attention_rule_amd/build.py"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """Calibrated HBM bytes per launch from the committed counter runs, if still current.
    `kernel` is a summary label: a kernel name, or "name [template args, grid N]" when the
    run launched it in several forms."""
    try:
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f).get(f"{kernel}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(kernel.split(" [")[0]):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


MAIN_WORKLOAD = f"prefill {W.LONG.name} + verify {W.VERIFY.name}"
EXTRAS_WORKLOAD = (f"commit after {W.VERIFY.name} + conv {W.CONV_PREFILL.name} / "
                   f"{W.CONV_UPDATE.name} + gated norm {W.NORM.name} + mixed step {W.MIXED.name}")


FULL_WORKLOAD = (f"every configuration: prefill {W.VARLEN.name}, {W.LONG.name}, {W.SINGLE_LONG.name}; "
                 f"verify {W.VERIFY.name}, {W.VERIFY_B1.name}; next rows")


N_XCD = 8           # MI355X: XCDs (GRBM_GUI_ACTIVE is read once per XCD)
N_SIMD = 256 * 4    # compute units x SIMDs


def targs(kernel_name):
    """Template arguments of a (demangled) kernel name, e.g. '<4, 4, 1, 1>' (or ''), after
    the verify kernel's form ('step' or 'block')."""
    m = re.search(r"(\w+)_kernel(<[^()]*>)?\(", kernel_name)
    if not m:
        return ""
    form = m.group(1).split("_")[-1] + " " if m.group(1).startswith("verify_") else ""
    return (form + (m.group(2) or "")).strip()


def summarize(prof_dirs, workload, out_md, mode_flag):
    """Write a text summary of rocprofv3 CSV output (kernel trace, FETCH_SIZE and WRITE_SIZE
    passes) for the KDA kernels, and record calibrated traffic in profiles/traffic.json."""
    import csv
    import glob
    import re
    stats = {}
    counters = {}
    calib = {}
    for d in prof_dirs:
        has_counters = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        for f in ([] if has_counters else
                  glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
            for r in csv.DictReader(open(f)):
                for k, pat in KERNEL_PATTERNS.items():
                    if pat in r["Kernel_Name"]:
                        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
                        stats.setdefault((k, targs(r["Kernel_Name"]), int(r["Grid_Size_X"])),
                                         []).append(dur)
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                name, cname, val = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
                if re.search(r"elementwise_kernel.*Mul", name):
                    # the calibration copies (x * 1.0 over CALIB_BYTES) are the only such kernels
                    calib.setdefault(cname, []).append(val)
                for k, pat in KERNEL_PATTERNS.items():
                    if pat in name:
                        counters.setdefault((k, targs(name), int(r["Grid_Size"])),
                                            {}).setdefault(cname, []).append(val)
    factors = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        big = [v for v in calib.get(cname, []) if v * 1024 > 0.5 * CALIB_BYTES]
        factors[cname] = (CALIB_BYTES / 1024) / (sum(big) / len(big)) if big else None
    full = workload == FULL_WORKLOAD
    lines = [f"# rocprofv3 summary: {workload}", "",
             "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_trace -o trace "
             f"-- python3 $R/bench.py --no-cpu-baseline {mode_flag}".rstrip()]
    if full:
        lines += ["    python3 $R/bench.py --summarize OUT/prof_trace --summary-out <this file>", ""]
    else:
        lines += [
             "    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d OUT/prof_fetch "
             f"-o fetch -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline {mode_flag} "
             "--calib-copy",
             "    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d OUT/prof_write "
             f"-o write -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline {mode_flag} "
             "--calib-copy",
             "    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_BF16 "
             "SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --kernel-trace "
             "--output-format csv -d OUT/prof_mfma -o mfma -- python3 $R/bench.py --steps 3 "
             f"--warmup 1 --no-cpu-baseline {mode_flag}   (main mode only)",
             "    rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE --kernel-trace "
             "--output-format csv -d OUT/prof_lds -o lds -- python3 $R/bench.py --steps 3 "
             f"--warmup 1 --no-cpu-baseline {mode_flag}   (main mode only)",
             "    python3 $R/bench.py --summarize OUT/prof_trace OUT/prof_fetch OUT/prof_write "
             f"[OUT/prof_mfma OUT/prof_lds] {mode_flag} --summary-out <this file>", ""]
    lines += [
             "Kernel durations (kernel-trace run only):", "",
             "| kernel | dispatches | avg us | min us | max us |", "|---|---|---|---|---|"]
    def label(key, keys):
        # A kernel launched in one form keeps its plain name; else its template arguments
        # and grid size tell apart the launches it made.
        k, ta, grid = key
        if sum(1 for kk, _, _ in keys if kk == k) == 1:
            return k
        return f"{k} [{ta + ', ' if ta else ''}grid {grid}]"

    for key, v in sorted(stats.items()):
        lines.append(f"| {label(key, stats)} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | "
                     f"{max(v):.2f} |")
    if not full:
        lines += ["", "Counter calibration (--calib-copy: an elementwise kernel reading and writing "
                  "1 GiB): bytes = counter KiB x 1024 x factor, with "
                  + ", ".join(f"{c} factor {f:.4f}" if f else f"{c}: not measured"
                              for c, f in factors.items()), ""]
    try:
        with open(TRAFFIC_JSON) as f:
            store = json.load(f)
    except (OSError, ValueError):
        store = {}
    # Entries of workloads this script no longer measures are dropped, and so are this
    # workload's old entries when new counters replace them.
    have_counters = any("FETCH_SIZE" in cs and "WRITE_SIZE" in cs for cs in counters.values())
    store = {k: v for k, v in store.items()
             if k.rpartition("@")[2] in (MAIN_WORKLOAD, EXTRAS_WORKLOAD)
             and not (have_counters and k.rpartition("@")[2] == workload)}
    if not full:
        lines += ["| kernel | FETCH_SIZE KiB/dispatch (raw) | WRITE_SIZE KiB/dispatch (raw) | "
                  "calibrated HBM MB/dispatch |", "|---|---|---|---|"]
    for key, cs in sorted(counters.items()):
        k = label(key, counters)
        fr = cs.get("FETCH_SIZE")
        wr = cs.get("WRITE_SIZE")
        if not fr or not wr:
            continue
        f_kib, w_kib = sum(fr) / len(fr), sum(wr) / len(wr)
        ff, fw = factors["FETCH_SIZE"] or 1.0, factors["WRITE_SIZE"] or 1.0
        fb, wb = f_kib * 1024 * ff, w_kib * 1024 * fw
        lines.append(f"| {k} | {f_kib:.1f} | {w_kib:.1f} | {(fb + wb) / 1e6:.1f} |")
        if factors["FETCH_SIZE"] and factors["WRITE_SIZE"]:
            store[f"{k}@{workload}"] = {"fetch_bytes": fb, "write_bytes": wb,
                                       "source_hash": source_hash(key[0]),
                                       "calibration": factors}
    # MFMA and LDS counters (extra --pmc passes, when given): executed MFMA operations
    # (the MOPS counters count operations / 512 per data type), MFMA busy share of
    # all SIMD cycles (GRBM_GUI_ACTIVE: the GPU's busy clock, summed here over the
    # XCDs), LDS bank-conflict cycles against LDS-busy cycles.
    mf_rows = []
    for key, cs in sorted(counters.items()):
        mops = [cs.get(c) for c in ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                    "SQ_INSTS_VALU_MFMA_MOPS_F32")]
        if all(m is None for m in mops) and "SQ_LDS_BANK_CONFLICT" not in cs:
            continue
        avg = lambda c: (sum(cs[c]) / len(cs[c])) if cs.get(c) else None
        row = [label(key, counters)]
        if any(m is not None for m in mops):
            f16, b16, f32 = (avg(c) or 0.0 for c in ("SQ_INSTS_VALU_MFMA_MOPS_F16",
                                                      "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                                      "SQ_INSTS_VALU_MFMA_MOPS_F32"))
            row.append(f"{(f16 + b16 + f32) * 512 / 1e9:.2f} (f16 {f16 * 512 / 1e9:.2f}, "
                       f"bf16 {b16 * 512 / 1e9:.2f}, f32 {f32 * 512 / 1e9:.2f})")
            busy, act = avg("SQ_VALU_MFMA_BUSY_CYCLES"), avg("GRBM_GUI_ACTIVE")
            row.append(f"{100 * busy / (act / N_XCD * N_SIMD):.1f}" if busy and act else "-")
        else:
            row += ["-", "-"]
        conf, lact = avg("SQ_LDS_BANK_CONFLICT"), avg("SQ_LDS_IDX_ACTIVE")
        row.append(f"{100 * conf / lact:.1f}" if conf is not None and lact else "-")
        mf_rows.append("| " + " | ".join(row) + " |")
    if mf_rows:
        lines += ["", "MFMA and LDS counters (each from its own --pmc pass; MFMA operations "
                  "= MOPS counters x 512):", "",
                  "| kernel | MFMA operations per dispatch (1e9) | MFMA busy % of SIMD cycles "
                  "| LDS bank-conflict % of LDS-active cycles |", "|---|---|---|---|"] + mf_rows
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(store, f, indent=1, sort_keys=True)
    print("\n".join(lines))


def roofline(bytes_, flops, seconds, bound="hbm"):
    if bound == "hbm":
        ach = bytes_ / seconds / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    ach = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_BF16_PEAK_TFS, 4), "traffic": None}


def measured_ceilings():
    """Ceilings measured on this GPU in the same run, beside the published peaks: a
    write-only fill and an elementwise copy through the shader (1 GiB each way), and a
    dense bf16 GEMM from the vendor library (8192 x 8192 x 8192, contiguous operands)."""
    def timed(fn, iters):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / iters

    a = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    t_fill = timed(lambda: b.fill_(2.0), 20)
    t_copy = timed(lambda: torch.mul(a, 1.0, out=b), 20)
    del a, b
    m = 8192
    x = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    z = torch.empty(m, m, dtype=torch.bfloat16, device="cuda")
    t_gemm = timed(lambda: torch.matmul(x, y, out=z), 10)
    del x, y, z
    torch.cuda.empty_cache()
    return {"write_only_GBs": round(CALIB_BYTES / t_fill / 1e9, 1),
            "copy_GBs": round(2 * CALIB_BYTES / t_copy / 1e9, 1),
            "gemm_bf16_TFs": round(2 * m ** 3 / t_gemm / 1e12, 1),
            "how": "fill_ of 1 GiB; x*1.0 over 1 GiB (read + write); torch.matmul bf16 8192^3"}


def calibration_copies():
    """An elementwise kernel that reads 1 GiB and writes 1 GiB (a copy through the shader,
    unlike copy_, which may use the DMA engine and escape the counters)."""
    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def time_calls(fn, iters, warmup=3):
    """Mean seconds per call of fn, by HIP events on torch's current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / iters


def verify_latency_b1(iters):
    """The verify latency case (one row of 8 draft tokens at 16 heads): microseconds per
    call with plain launches, and per call replayed from a HIP graph of 20 calls (launch
    overhead excluded). Each of three replays is checked against a plain call first."""
    case = W.VERIFY_B1
    vd = to_dev(W.make_verify(case))
    B, Tv, H = case.batch, case.steps, case.heads
    out = torch.empty((B * Tv, H, D), dtype=torch.bfloat16, device="cuda")
    inter = torch.empty((B, Tv, H, D, D), dtype=torch.float32, device="cuda")

    def call():
        recurrent_verify(vd["q"], vd["k"], vd["v"], vd["g"], vd["beta_logits"], vd["A_log"],
                         vd["dt_bias"], vd["lower_bound"], vd["state_pool"], vd["state_idx"], Tv,
                         intermediate=inter, out=out, scale=vd["scale"])

    res = {"workload": case.name, "how": "mean over back-to-back calls (plain launches, and "
           "replays of a graph of 20 calls)",
           "us_plain_launch": round(time_calls(call, 10 * iters) * 1e6, 2)}
    call()
    torch.cuda.synchronize()
    ref = (out.clone(), inter.clone())
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(20):
                call()
        same = True
        for _ in range(3):
            out.zero_()
            inter.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            same = same and torch.equal(out, ref[0]) and torch.equal(inter, ref[1])
        res["us_graph_replay"] = round(time_calls(graph.replay, iters) / 20 * 1e6, 2) if same else None
        res["graph_replays_match_plain_call"] = bool(same)
    except RuntimeError as e:
        res["us_graph_replay"] = None
        res["graph_error"] = str(e)[:200]
    return res


def bench_next_rows(iters):
    """The rows after the hot path (medians of `iters` calls): the rollback commit at the
    verify size, the short conv (prefill and update), the gated output norm, and one mixed
    speculative step (prefill segment and spec rows scattered into one layer output)."""
    vcase = W.VERIFY
    B, Tv, H = vcase.batch, vcase.steps, vcase.heads
    rng = np.random.default_rng(4000)
    inter = torch.full((B, Tv, H, D, D), 0.5, dtype=torch.float32, device="cuda")
    pool = torch.zeros((vcase.pool_slots, H, D, D), dtype=torch.float32, device="cuda")
    idx = torch.from_numpy(rng.permutation(vcase.pool_slots)[:B].astype(np.int32)).cuda()
    nacc = torch.from_numpy(rng.integers(1, Tv + 1, size=B).astype(np.int32)).cuda()
    t_commit = median_call_us(lambda: commit_accepted(inter, idx, nacc, pool), iters) * 1e-6
    commit_bytes = B * H * 2 * STATE_BYTES + 2 * B * 4
    del inter, pool

    # Verify with the output-gate norm fused into its store, against verify then the
    # standalone norm over its output, at the verify size and at batch 1.
    gated = {}
    for vc in (W.VERIFY, W.VERIFY_B1):
        vd = to_dev(W.make_verify(vc))
        Bv, Tg, Hv = vc.batch, vc.steps, vc.heads
        nd = W.make_norm(W.NormCase("verify_gate", Bv * Tg, Hv, seed=4400))
        gate, wgt = nd["gate"].cuda(), nd["weight"].cuda()
        o_ = torch.empty((Bv * Tg, Hv, D), dtype=torch.bfloat16, device="cuda")
        y_ = torch.empty_like(o_)
        it_ = torch.empty((Bv, Tg, Hv, D, D), dtype=torch.float32, device="cuda")
        r_ = torch.empty((Bv * Tg, Hv), dtype=torch.float32, device="cuda")
        args_ = (vd["q"], vd["k"], vd["v"], vd["g"], vd["beta_logits"], vd["A_log"],
                 vd["dt_bias"], vd["lower_bound"], vd["state_pool"], vd["state_idx"], Tg)

        def fused():
            recurrent_verify_gated(*args_, gate, wgt, nd["eps"], intermediate=it_, out=y_,
                                   rstd=r_, scale=vd["scale"])

        def separate():
            recurrent_verify(*args_, intermediate=it_, out=o_, scale=vd["scale"])
            gated_rmsnorm(o_, gate, wgt, nd["eps"], out=y_, rstd=r_)

        gated[vc.name] = {"fused_us": round(median_call_us(fused, iters), 2),
                          "verify_then_norm_us": round(median_call_us(separate, iters), 2)}
        del vd, o_, y_, it_, r_
    torch.cuda.empty_cache()

    m = W.make_mixed(W.MIXED)
    pre, spec = to_dev(m["prefill"]), to_dev(m["spec"])
    Tp, Hm = pre["q"].shape[0], pre["q"].shape[1]
    Np = pre["cu_seqlens"].numel() - 1
    Bs, Ts = W.MIXED.spec.batch, W.MIXED.spec.steps
    core = torch.empty((m["out_rows"], Hm, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(prefill_workspace_bytes(Np, Tp, Hm), dtype=torch.uint8, device="cuda")
    fin = torch.empty((Np, Hm, D, D), dtype=torch.float32, device="cuda")
    sinter = torch.empty((Bs, Ts, Hm, D, D), dtype=torch.float32, device="cuda")
    ns_idx, sp_idx = m["non_spec_idx"].cuda(), m["spec_idx"].cuda()

    def mixed():
        chunk_prefill(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta_logits"], pre["A_log"],
                      pre["dt_bias"], pre["lower_bound"], pre["cu_seqlens"], out=core,
                      final_state=fin, workspace=ws, scale=pre["scale"], out_token_index=ns_idx)
        recurrent_verify(spec["q"], spec["k"], spec["v"], spec["g"], spec["beta_logits"],
                         spec["A_log"], spec["dt_bias"], spec["lower_bound"], spec["state_pool"],
                         spec["state_idx"], Ts, intermediate=sinter, out=core, scale=spec["scale"],
                         out_token_index=sp_idx)

    t_mixed = median_call_us(mixed, iters) * 1e-6
    del core, ws, fin, sinter

    tokens = Tp + Bs * Ts
    mixed_bytes = (tokens * Hm * BYTES_PER_TOKEN_HEAD + Np * Hm * STATE_BYTES
                   + Bs * Hm * STATE_BYTES * (1 + Ts))
    nd = W.make_norm(W.NORM)
    nx, ng, nw = nd["x"].cuda(), nd["gate"].cuda(), nd["weight"].cuda()
    ny = torch.empty_like(nx)
    nr = torch.empty(nx.shape[:2], dtype=torch.float32, device="cuda")
    t_norm = median_call_us(lambda: gated_rmsnorm(nx, ng, nw, nd["eps"], out=ny, rstd=nr), iters) * 1e-6
    norm_rows = nx.shape[0] * nx.shape[1]
    norm_bytes = norm_rows * (3 * 2 * D + 4)
    rl_norm = roofline(norm_bytes, 0, t_norm)
    rl_norm["traffic"] = stored_traffic(f"kda_gated_rmsnorm [grid {norm_rows // 32 * 256}]",
                                        EXTRAS_WORKLOAD)
    del nx, ng, ny, nr

    # Short conv on the packed q|k|v columns: prefill at 4 x 8192, update at 64 x 8.
    cp = W.make_conv(W.CONV_PREFILL)
    cx, cw, cb = cp["x"].cuda(), cp["weight"].cuda(), cp["bias"].cuda()
    cst, cidx, ccu = cp["state"].cuda(), cp["state_idx"].cuda(), cp["cu_seqlens"].cuda()
    cy = torch.empty_like(cx)
    t_convp = median_call_us(lambda: causal_conv1d_prefill(cx, cw, cb, ccu, conv_state=cst,
                                                           state_idx=cidx, out=cy), iters) * 1e-6
    Tc, Cc = cx.shape
    Wc = W.CONV_PREFILL.width
    Nc = ccu.numel() - 1
    convp_bytes = 2 * Tc * Cc * 2 + 2 * Nc * (Wc - 1) * Cc * 2 + Cc * (Wc + 1) * 2
    del cx, cy, cst
    cu_ = W.make_conv(W.CONV_UPDATE)
    ux, uw, ub = cu_["x"].cuda(), cu_["weight"].cuda(), cu_["bias"].cuda()
    upool, uidx = cu_["state"].cuda(), cu_["state_idx"].cuda()
    Bu, Tu = W.CONV_UPDATE.batch, W.CONV_UPDATE.steps
    uy = torch.empty_like(ux)
    uint = torch.empty((Bu, Tu, Wc - 1, Cc), dtype=torch.bfloat16, device="cuda")
    t_convu = median_call_us(lambda: causal_conv1d_update(ux, uw, ub, upool, uidx, Tu,
                                                          intermediate=uint, out=uy), iters) * 1e-6
    convu_bytes = (2 * Bu * Tu * Cc * 2 + Bu * (Wc - 1) * Cc * 2 + Bu * Tu * (Wc - 1) * Cc * 2
                   + Cc * (Wc + 1) * 2)
    del ux, uy, upool, uint
    rl_convp = roofline(convp_bytes, 0, t_convp)
    rl_convp["traffic"] = stored_traffic("kda_conv_prefill", EXTRAS_WORKLOAD)
    rl_convu = roofline(convu_bytes, 0, t_convu)

    rl_commit = roofline(commit_bytes, 0, t_commit)
    rl_commit["traffic"] = stored_traffic("kda_commit", EXTRAS_WORKLOAD)
    return {
        "commit": {"workload": f"commit after {vcase.name}", "us": round(t_commit * 1e6, 2),
                   "roofline": rl_commit, "algorithmic_bytes": commit_bytes},
        "conv_prefill": {"workload": W.CONV_PREFILL.name, "us": round(t_convp * 1e6, 2),
                         "roofline": rl_convp, "algorithmic_bytes": convp_bytes},
        "conv_update": {"workload": W.CONV_UPDATE.name, "us": round(t_convu * 1e6, 2),
                        "roofline": rl_convu, "algorithmic_bytes": convu_bytes},
        "gated_rmsnorm": {"workload": W.NORM.name, "us": round(t_norm * 1e6, 2),
                          "roofline": rl_norm, "algorithmic_bytes": norm_bytes},
        "verify_gated_norm": gated,
        "mixed_step": {"workload": W.MIXED.name, "us": round(t_mixed * 1e6, 2),
                       "tokens_per_s": round(tokens / t_mixed, 1),
                       "roofline": roofline(mixed_bytes, 0, t_mixed),
                       "algorithmic_bytes": mixed_bytes},
    }


def median_call_us(fn, iters, warmup=3):
    """Median microseconds over `iters` calls of fn, each bracketed by its own pair of HIP
    events on torch's current stream (the stream libkda launches on)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3


def cold_call_us(fn, iters, flush, how):
    """Median microseconds of fn with the caches emptied first: `how` = "write" overwrites
    the 1 GiB buffer `flush` (the protocol's cold run: evicts L2 and the 256 MB memory-side
    cache, leaving them full of dirty lines), "read" reads it (evicts without dirty lines);
    the flush completes before the timed call starts."""
    ts = []
    for _ in range(iters):
        if how == "write":
            flush.fill_(1.0)
        else:
            flush.sum()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts)) * 1e3


def prefill_alg(case, T, H, N, init_rows_read):
    """Algorithmic bytes and MFMA flops of one prefill call: 1282 B and 139,264 flop per
    token-head, plus each start state read and each final state written (64 KiB)."""
    bytes_ = T * H * BYTES_PER_TOKEN_HEAD + (init_rows_read + N) * H * STATE_BYTES
    return bytes_, T * H * FLOPS_PER_TOKEN_HEAD


def config_line(name, us, tokens, bytes_, flops, cold=None, extra=None):
    t = us * 1e-6
    hbm = roofline(bytes_, 0, t)
    line = {"workload": name, "us_per_layer": round(us, 2), "tokens_per_s": round(tokens / t, 1),
            "algorithmic_bytes": bytes_, "hbm": hbm}
    if flops:
        line["mfma"] = roofline(0, flops, t, bound="mfma")
        line["roofline_frac"] = round(max(bytes_ / (HBM_PEAK_GBS * 1e9),
                                          flops / (MFMA_BF16_PEAK_TFS * 1e12)) / t, 4)
    else:
        line["roofline_frac"] = hbm["frac"]
    if cold:
        line["cold_us"] = {k: round(v, 2) for k, v in cold.items()}
        line["cold_hbm_frac"] = {k: round(bytes_ / (v * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                 for k, v in cold.items()}
    if extra:
        line.update(extra)
    return line


class PrefillRun:
    """Device inputs and caller buffers of one prefill workload (out preallocated)."""

    def __init__(self, case):
        self.case = case
        self.d = to_dev(W.make_prefill(case))
        d = self.d
        self.T, self.H = d["q"].shape[0], d["q"].shape[1]
        self.N = d["cu_seqlens"].numel() - 1
        self.ws = torch.empty(prefill_workspace_bytes(self.N, self.T, self.H), dtype=torch.uint8,
                              device="cuda")
        self.out = torch.empty((self.T, self.H, D), dtype=torch.bfloat16, device="cuda")
        self.fin = torch.empty((self.N, self.H, D, D), dtype=torch.float32, device="cuda")
        self.init_rows_read = 0 if d["initial_state"] is None else self.N

    def __call__(self, phase="both"):
        d = self.d
        chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"], d["dt_bias"],
                      d["lower_bound"], d["cu_seqlens"], initial_state=d["initial_state"],
                      initial_state_idx=d["initial_state_idx"], out=self.out,
                      final_state=self.fin, workspace=self.ws, scale=d["scale"], phase=phase)

    def alg(self):
        return prefill_alg(self.case, self.T, self.H, self.N, self.init_rows_read)

    def free(self):
        del self.d, self.ws, self.out, self.fin
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--iters", type=int, default=50,
                    help="calls per median in the per-configuration protocol (at least 50)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens per sequence in the oracle's timed sample (8192: the whole "
                         "4 x 8192 workload, about 10 s of one host core)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run 1 GiB device copies (counter calibration under rocprofv3)")
    ap.add_argument("--summarize", nargs="+", metavar="PROF_DIR",
                    help="summarize rocprofv3 CSV output into --summary-out and exit")
    ap.add_argument("--summary-out", default=None)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-configuration protocol and the next rows (the timed "
                         "steps and the per-kernel split only: for profiling)")
    ap.add_argument("--extras-only", action="store_true",
                    help="measure only the next rows (one JSON line)")
    args = ap.parse_args()
    if args.summarize:
        # --extras-only: the next rows; --no-extras: the timed steps and the kernel split;
        # neither: the full default run (every configuration, kernel trace only).
        if args.extras_only:
            wl, flag = EXTRAS_WORKLOAD, "--extras-only"
        elif args.no_extras:
            wl, flag = MAIN_WORKLOAD, "--no-extras"
        else:
            wl, flag = FULL_WORKLOAD, ""
        summarize(args.summarize, wl, args.summary_out or os.path.join(ROOT, "profiles", "summary.md"),
                  flag)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the library runs the "
              "path on one GPU (heads, sequences and verify rows shard without communication)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    iters = max(50, args.iters)

    if args.calib_copy:
        calibration_copies()
    if args.extras_only:
        print(json.dumps({"next_rows": bench_next_rows(iters)}), flush=True)
        return

    vcase = W.VERIFY
    log(f"generating {W.LONG.name} and {vcase.name}")
    long = PrefillRun(W.LONG)
    vd = to_dev(W.make_verify(vcase))
    T, H, N = long.T, long.H, long.N
    B, Tv = vcase.batch, vcase.steps
    vout = torch.empty((B * Tv, H, D), dtype=torch.bfloat16, device="cuda")
    inter = torch.empty((B, Tv, H, D, D), dtype=torch.float32, device="cuda")

    def verify():
        recurrent_verify(vd["q"], vd["k"], vd["v"], vd["g"], vd["beta_logits"], vd["A_log"],
                         vd["dt_bias"], vd["lower_bound"], vd["state_pool"], vd["state_idx"], Tv,
                         intermediate=inter, out=vout, scale=vd["scale"])

    # One step = one pass of the hot path: the whole prefill call (kda_chunk_prefill, both
    # kernels) at 4 x 8192, then the verify call at 64 x 8; each call between its own events.
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        long()
        if ev is not None:
            ev[1].record()
        verify()
        if ev is not None:
            ev[2].record()

    # The two kernels of the prefill call, each timed as its own call (same arguments).
    # Measured before the timed steps: the GPU leaves its idle clocks during the first
    # few milliseconds of sustained work (a step sequence started from idle runs its first
    # dozen steps 5-10% slower), so the timed steps follow this work rather than the
    # host-side input generation; the first of these calls get as many untimed ones first.
    us_intra = median_call_us(lambda: long("intra"), iters, warmup=iters)
    us_scan = median_call_us(lambda: long("scan"), iters)
    log(f"split: intra {us_intra:.1f} us  scan {us_scan:.1f} us")

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    s_prefill = float(np.median([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    s_ver = float(np.median([e[1].elapsed_time(e[2]) for e in evs])) * 1e-3
    log(f"timed steps: prefill call {s_prefill * 1e6:.1f} us  verify {s_ver * 1e6:.1f} us "
        f"(medians of {args.steps})")


    p_bytes, p_flops = long.alg()
    token_heads = T * H
    intra_bytes = token_heads * (3 * 2 * D + 2)                      # q, k, g, beta logit
    scan_bytes = token_heads * (2 * D + 2 * D) + N * H * STATE_BYTES  # v, out, final states
    verify_bytes = (B * Tv * H * BYTES_PER_TOKEN_HEAD + B * H * STATE_BYTES
                    + B * Tv * H * STATE_BYTES)
    workload = MAIN_WORKLOAD
    by_kernel = {
        "kda_prefill_intra": roofline(intra_bytes, 0, us_intra * 1e-6),
        "kda_prefill_scan": roofline(scan_bytes, 0, us_scan * 1e-6),
        "kda_verify": roofline(verify_bytes, 0, s_ver),
    }
    for k, rl_k in by_kernel.items():
        rl_k["traffic"] = stored_traffic(k, workload)
    # The headline roofline is the prefill call's: its algorithmic bytes over the call's
    # time (both kernels), with the calibrated traffic of both kernels per call.
    rl = roofline(p_bytes, 0, s_prefill)
    ti, ts_ = stored_traffic("kda_prefill_intra", workload), stored_traffic("kda_prefill_scan", workload)
    rl["traffic"] = (ti + ts_) if ti is not None and ts_ is not None else None
    rl["kernel"] = "kda_chunk_prefill (kda_prefill_intra + kda_prefill_scan)"

    configs = None
    cold_verify = None
    ceil = None
    lat_b1 = None
    if not args.no_extras:
        flush = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        log("protocol: medians of %d calls, warm and cold" % iters)
        cold = lambda fn: {"write_flush": cold_call_us(fn, 10, flush, "write"),
                           "read_flush": cold_call_us(fn, 10, flush, "read")}
        configs = {}
        us2 = median_call_us(long, iters)
        configs["long_4x8192"] = config_line(W.LONG.name, us2, T, p_bytes, p_flops, cold(long),
                                             {"intra_us": round(us_intra, 2),
                                              "scan_us": round(us_scan, 2)})
        us4 = median_call_us(verify, iters)
        cold_verify = cold(verify)
        configs["verify_64x8"] = config_line(vcase.name, us4, B * Tv, verify_bytes, 0, cold_verify)
        long.free()
        del vd, vout, inter
        torch.cuda.empty_cache()
        for key, case in (("varlen_8x2048", W.VARLEN), ("single_16384", W.SINGLE_LONG)):
            log(f"protocol: {case.name}")
            run = PrefillRun(case)
            us = median_call_us(run, iters)
            ui = median_call_us(lambda: run("intra"), iters)
            uscan = median_call_us(lambda: run("scan"), iters)
            b_, f_ = run.alg()
            configs[key] = config_line(case.name, us, run.T, b_, f_, cold(run),
                                       {"intra_us": round(ui, 2), "scan_us": round(uscan, 2)})
            run.free()
        del flush
        torch.cuda.empty_cache()
        log("verify latency case (B = 1)")
        lat_b1 = verify_latency_b1(iters)
        log("measured ceilings (fill, copy, GEMM)")
        ceil = measured_ceilings()

    cpu = None
    if not args.no_cpu_baseline:
        log(f"oracle baseline on {args.cpu_tokens} tokens/sequence")
        cpu = cpu_baseline(W.LONG, args.cpu_tokens)

    extras = None if args.no_extras else bench_next_rows(iters)
    if extras:
        log(f"commit {extras['commit']['us']} us  mixed step {extras['mixed_step']['us']} us")

    value = T / s_prefill
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "prefill": {"seqs": N, "seq_len": T // N, "heads": H, "head_dim": D, "chunk": 64,
                        "initial_state": "zero"},
            "verify": {"batch": B, "draft_steps": Tv, "heads": H, "pool_slots": vcase.pool_slots},
            "parallelism": "single GPU",
            "compute": "bf16 in/out; fp16 and bf16 MFMA operands with fp32 accumulation; fp32 state",
        },
        "prefill_us_per_layer": round(s_prefill * 1e6, 2),
        "prefill_tokens_per_s": round(value, 1),
        "verify_us_per_layer": round(s_ver * 1e6, 2),
        "verify_tokens_per_s": round(B * Tv / s_ver, 1),
        "timing": f"medians of per-call HIP events over the {args.steps} timed steps; "
                  f"kernel split and configurations: medians of {iters} calls",
        "kernel_us": {"kda_prefill_intra": round(us_intra, 2),
                      "kda_prefill_scan": round(us_scan, 2),
                      "kda_verify": round(s_ver * 1e6, 2)},
        "roofline": rl,
        "roofline_by_kernel": by_kernel,
        "roofline_prefill_call": {
            "hbm": roofline(p_bytes, 0, s_prefill),
            "mfma": roofline(0, p_flops, s_prefill, bound="mfma"),
            "roofline_frac": round(max(p_bytes / (HBM_PEAK_GBS * 1e9),
                                       p_flops / (MFMA_BF16_PEAK_TFS * 1e12)) / s_prefill, 4),
        },
        "configs": configs,
        "verify_latency_b1": lat_b1,
        "measured_ceilings": ceil,
        "cpu_baseline": cpu,
        "next_rows": extras,
        "context": {"flashkda_gb300_us_per_layer": {"2048x8": 49, "8192x4": 146, "16384x1": 787},
                    "note": "the pages' numbers, other hardware; not targets"},
    }
    if ceil:
        res["fraction_of_measured"] = {
            "verify_vs_write_only": round(by_kernel["kda_verify"]["achieved"] / ceil["write_only_GBs"], 4),
            "prefill_hbm_vs_copy": round(rl["achieved"] / ceil["copy_GBs"], 4),
            "prefill_mfma_vs_gemm": round(res["roofline_prefill_call"]["mfma"]["achieved"]
                                          / ceil["gemm_bf16_TFs"], 4),
        }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
