"""KDA prefill + verify benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over one batch of synthetic input:
  * varlen chunked prefill of 4 sequences x 8192 tokens, H = 16, d = 128
    (zero start state, fp32 final states): the intra-chunk kernel then the
    state-scan kernel (kda_chunk_prefill_intra + kda_chunk_prefill_scan, which
    together are exactly kda_chunk_prefill);
  * fused verify of 64 rows x 8 draft tokens, H = 16, states gathered from a
    256-slot fp32 pool, per-step fp32 states written (kda_recurrent_verify).
Inputs are resident in HBM before timing starts.  Each kernel is bracketed by
HIP events on the stream it is launched on (torch's current stream, which the
binding hands to libkda).  Prints ONE JSON line on stdout; progress goes to stderr.

`value` is prefill tokens/s at 4x8192 (the headline shape); prefill and verify
microseconds per layer are reported beside it.  The oracle (fp64 CPU token
loop) is timed on a bounded sample of the same prefill workload as
`cpu_baseline`.
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
                                       recurrent_verify)
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
    "kda_verify": "verify_kernel",
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
    """Calibrated HBM bytes per launch from the committed counter runs, if still current."""
    try:
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f).get(f"{kernel}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


MAIN_WORKLOAD = f"prefill {W.LONG.name} + verify {W.VERIFY.name}"
EXTRAS_WORKLOAD = (f"commit after {W.VERIFY.name} + conv {W.CONV_PREFILL.name} / "
                   f"{W.CONV_UPDATE.name} + gated norm {W.NORM.name} + segmented prefill "
                   f"{W.SINGLE_LONG.name} + mixed step {W.MIXED.name}")


N_XCD = 8           # MI355X: XCDs (GRBM_GUI_ACTIVE is read once per XCD)
N_SIMD = 256 * 4    # compute units x SIMDs


def targs(kernel_name):
    """Template arguments of a (demangled) kernel name, e.g. '<4, 4, 1, 1>' (or '')."""
    m = re.search(r"_kernel(<[^()]*>)\(", kernel_name)
    return m.group(1) if m else ""


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
    lines = [f"# rocprofv3 summary: {workload}", "",
             "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_trace -o trace "
             f"-- python3 $R/bench.py --no-cpu-baseline {mode_flag}",
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
             f"[OUT/prof_mfma OUT/prof_lds] {mode_flag} --summary-out <this file>", "",
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
    lines += ["", "Counter calibration (--calib-copy: an elementwise kernel reading and writing "
              "1 GiB): bytes = counter KiB x 1024 x factor, with "
              + ", ".join(f"{c} factor {f:.4f}" if f else f"{c}: not measured"
                          for c, f in factors.items()), ""]
    try:
        with open(TRAFFIC_JSON) as f:
            store = json.load(f)
    except (OSError, ValueError):
        store = {}
    # Entries of workloads this script no longer measures are dropped.
    store = {k: v for k, v in store.items()
             if k.rpartition("@")[2] in (MAIN_WORKLOAD, EXTRAS_WORKLOAD)}
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

    res = {"workload": case.name, "us_plain_launch": round(time_calls(call, 10 * iters) * 1e6, 2)}
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
    """The rows after the hot path: the rollback commit at the verify size, and one mixed
    speculative step (prefill segment and spec rows scattered into one layer output)."""
    vcase = W.VERIFY
    B, Tv, H = vcase.batch, vcase.steps, vcase.heads
    rng = np.random.default_rng(4000)
    inter = torch.full((B, Tv, H, D, D), 0.5, dtype=torch.float32, device="cuda")
    pool = torch.zeros((vcase.pool_slots, H, D, D), dtype=torch.float32, device="cuda")
    idx = torch.from_numpy(rng.permutation(vcase.pool_slots)[:B].astype(np.int32)).cuda()
    nacc = torch.from_numpy(rng.integers(1, Tv + 1, size=B).astype(np.int32)).cuda()
    t_commit = time_calls(lambda: commit_accepted(inter, idx, nacc, pool), iters)
    commit_bytes = B * H * 2 * STATE_BYTES + 2 * B * 4
    del inter, pool

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

    t_mixed = time_calls(mixed, iters)
    del core, ws, fin, sinter

    # One long sequence with a gathered start state: few (sequence, head) pairs, so the
    # scan runs segment-parallel (state maps per segment, combine, then the segments).
    sc = W.SINGLE_LONG
    sd = to_dev(W.make_prefill(sc))
    Ts1, Hs1 = sd["q"].shape[0], sd["q"].shape[1]
    s_ws = torch.empty(prefill_workspace_bytes(1, Ts1, Hs1), dtype=torch.uint8, device="cuda")
    s_out = torch.empty((Ts1, Hs1, D), dtype=torch.bfloat16, device="cuda")
    s_fin = torch.empty((1, Hs1, D, D), dtype=torch.float32, device="cuda")

    def single(phase):
        chunk_prefill(sd["q"], sd["k"], sd["v"], sd["g"], sd["beta_logits"], sd["A_log"],
                      sd["dt_bias"], sd["lower_bound"], sd["cu_seqlens"],
                      initial_state=sd["initial_state"], initial_state_idx=sd["initial_state_idx"],
                      out=s_out, final_state=s_fin, workspace=s_ws, scale=sd["scale"], phase=phase)

    t_s_intra = time_calls(lambda: single("intra"), iters)
    t_s_scan = time_calls(lambda: single("scan"), iters)
    s_bytes = Ts1 * Hs1 * BYTES_PER_TOKEN_HEAD + 2 * Hs1 * STATE_BYTES
    t_single = t_s_intra + t_s_scan
    tokens = Tp + Bs * Ts
    mixed_bytes = (tokens * Hm * BYTES_PER_TOKEN_HEAD + Np * Hm * STATE_BYTES
                   + Bs * Hm * STATE_BYTES * (1 + Ts))
    nd = W.make_norm(W.NORM)
    nx, ng, nw = nd["x"].cuda(), nd["gate"].cuda(), nd["weight"].cuda()
    ny = torch.empty_like(nx)
    nr = torch.empty(nx.shape[:2], dtype=torch.float32, device="cuda")
    t_norm = time_calls(lambda: gated_rmsnorm(nx, ng, nw, nd["eps"], out=ny, rstd=nr), iters)
    norm_rows = nx.shape[0] * nx.shape[1]
    norm_bytes = norm_rows * (3 * 2 * D + 4)
    rl_norm = roofline(norm_bytes, 0, t_norm)
    rl_norm["traffic"] = stored_traffic("kda_gated_rmsnorm", EXTRAS_WORKLOAD)
    del nx, ng, ny, nr

    # Short conv on the packed q|k|v columns: prefill at 4 x 8192, update at 64 x 8.
    cp = W.make_conv(W.CONV_PREFILL)
    cx, cw, cb = cp["x"].cuda(), cp["weight"].cuda(), cp["bias"].cuda()
    cst, cidx, ccu = cp["state"].cuda(), cp["state_idx"].cuda(), cp["cu_seqlens"].cuda()
    cy = torch.empty_like(cx)
    t_convp = time_calls(lambda: causal_conv1d_prefill(cx, cw, cb, ccu, conv_state=cst,
                                                       state_idx=cidx, out=cy), iters)
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
    t_convu = time_calls(lambda: causal_conv1d_update(ux, uw, ub, upool, uidx, Tu,
                                                      intermediate=uint, out=uy), iters)
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
        "segmented_prefill": {"workload": sc.name, "us": round(t_single * 1e6, 2),
                              "intra_us": round(t_s_intra * 1e6, 2),
                              "scan_us": round(t_s_scan * 1e6, 2),
                              "tokens_per_s": round(Ts1 / t_single, 1),
                              "roofline": roofline(s_bytes, 0, t_single),
                              "algorithmic_bytes": s_bytes},
        "mixed_step": {"workload": W.MIXED.name, "us": round(t_mixed * 1e6, 2),
                       "tokens_per_s": round(tokens / t_mixed, 1),
                       "roofline": roofline(mixed_bytes, 0, t_mixed),
                       "algorithmic_bytes": mixed_bytes},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
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
                    help="skip the commit and mixed-step measurements")
    ap.add_argument("--extras-only", action="store_true",
                    help="measure only the commit and the mixed step (one JSON line)")
    args = ap.parse_args()
    if args.summarize:
        extras = args.extras_only
        summarize(args.summarize, EXTRAS_WORKLOAD if extras else MAIN_WORKLOAD,
                  args.summary_out or os.path.join(ROOT, "profiles", "summary.md"),
                  "--extras-only" if extras else "--no-extras")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the library runs the "
              "path on one GPU (heads, sequences and verify rows shard without communication)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.calib_copy:
        calibration_copies()
    if args.extras_only:
        print(json.dumps({"next_rows": bench_next_rows(args.steps)}), flush=True)
        return

    pcase, vcase = W.LONG, W.VERIFY
    log(f"generating {pcase.name} and {vcase.name}")
    pd = to_dev(W.make_prefill(pcase))
    vd = to_dev(W.make_verify(vcase))
    T, H = pd["q"].shape[0], pd["q"].shape[1]
    N = pd["cu_seqlens"].numel() - 1
    ws = torch.empty(prefill_workspace_bytes(N, T, H), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    B, Tv = vcase.batch, vcase.steps
    vout = torch.empty((B * Tv, H, D), dtype=torch.bfloat16, device="cuda")
    inter = torch.empty((B, Tv, H, D, D), dtype=torch.float32, device="cuda")

    def prefill(phase):
        chunk_prefill(pd["q"], pd["k"], pd["v"], pd["g"], pd["beta_logits"], pd["A_log"],
                      pd["dt_bias"], pd["lower_bound"], pd["cu_seqlens"], out=out, final_state=fin,
                      workspace=ws, scale=pd["scale"], phase=phase)

    def verify():
        recurrent_verify(vd["q"], vd["k"], vd["v"], vd["g"], vd["beta_logits"], vd["A_log"],
                         vd["dt_bias"], vd["lower_bound"], vd["state_pool"], vd["state_idx"], Tv,
                         intermediate=inter, out=vout, scale=vd["scale"])

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        prefill("intra")
        if ev is not None:
            ev[1].record()
        prefill("scan")
        if ev is not None:
            ev[2].record()
        verify()
        if ev is not None:
            ev[3].record()


    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    t_intra = [e[0].elapsed_time(e[1]) * 1e-3 for e in evs]
    t_scan = [e[1].elapsed_time(e[2]) * 1e-3 for e in evs]
    t_ver = [e[2].elapsed_time(e[3]) * 1e-3 for e in evs]
    s_intra, s_scan, s_ver = (float(np.mean(x)) for x in (t_intra, t_scan, t_ver))
    s_prefill = s_intra + s_scan
    log(f"intra {s_intra * 1e6:.1f} us  scan {s_scan * 1e6:.1f} us  verify {s_ver * 1e6:.1f} us")

    # Cold-cache pass: overwrite 1 GiB between iterations (outside the events).
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cold_p, cold_v = [], []
    for _ in range(5):
        flush.fill_(1.0)
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        prefill("both")
        e1.record()
        flush.fill_(2.0)
        torch.cuda.synchronize()
        e1b = torch.cuda.Event(enable_timing=True)
        e1b.record()
        verify()
        e2.record()
        torch.cuda.synchronize()
        cold_p.append(e0.elapsed_time(e1) * 1e-3)
        cold_v.append(e1b.elapsed_time(e2) * 1e-3)
    del flush

    token_heads = T * H
    prefill_bytes = token_heads * BYTES_PER_TOKEN_HEAD + N * H * STATE_BYTES   # + final states
    intra_bytes = token_heads * (3 * 2 * D + 2)                                 # q, k, g, beta logit
    scan_bytes = token_heads * (2 * D + 2 * D) + N * H * STATE_BYTES            # v, out, final states
    verify_bytes = (B * Tv * H * BYTES_PER_TOKEN_HEAD + B * H * STATE_BYTES
                    + B * Tv * H * STATE_BYTES)
    prefill_flops = token_heads * FLOPS_PER_TOKEN_HEAD
    kernels = {
        "kda_prefill_intra": (s_intra, roofline(intra_bytes, 0, s_intra)),
        "kda_prefill_scan": (s_scan, roofline(scan_bytes, 0, s_scan)),
        "kda_verify": (s_ver, roofline(verify_bytes, 0, s_ver)),
    }
    workload = MAIN_WORKLOAD
    for k, (_, rl_k) in kernels.items():
        rl_k["traffic"] = stored_traffic(k, workload)
    dom = max(kernels, key=lambda k: kernels[k][0])
    rl = dict(kernels[dom][1])
    rl["kernel"] = dom

    log("measured ceilings (fill, copy, GEMM)")
    ceil = measured_ceilings()
    rl_p_hbm = roofline(prefill_bytes, 0, s_prefill)
    rl_p_mfma = roofline(0, prefill_flops, s_prefill, bound="mfma")
    vs_measured = {
        "verify_vs_write_only": round(kernels["kda_verify"][1]["achieved"] / ceil["write_only_GBs"], 4),
        "prefill_hbm_vs_copy": round(rl_p_hbm["achieved"] / ceil["copy_GBs"], 4),
        "prefill_mfma_vs_gemm": round(rl_p_mfma["achieved"] / ceil["gemm_bf16_TFs"], 4),
    }

    log("verify latency case (B = 1)")
    lat_b1 = verify_latency_b1(args.steps)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"oracle baseline on {args.cpu_tokens} tokens/sequence")
        cpu = cpu_baseline(pcase, args.cpu_tokens)

    extras = None if args.no_extras else bench_next_rows(args.steps)
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
        "kernel_us": {"kda_prefill_intra": round(s_intra * 1e6, 2),
                      "kda_prefill_scan": round(s_scan * 1e6, 2),
                      "kda_verify": round(s_ver * 1e6, 2)},
        "verify_latency_b1": lat_b1,
        "cold_cache_us": {"prefill": round(float(np.median(cold_p)) * 1e6, 2),
                          "verify": round(float(np.median(cold_v)) * 1e6, 2)},
        "roofline": rl,
        "roofline_by_kernel": {k: v[1] for k, v in kernels.items()},
        "roofline_prefill_call": {
            "hbm": rl_p_hbm,
            "mfma": rl_p_mfma,
            "roofline_frac": round(max(prefill_bytes / (HBM_PEAK_GBS * 1e9),
                                       prefill_flops / (MFMA_BF16_PEAK_TFS * 1e12)) / s_prefill, 4),
        },
        "measured_ceilings": ceil,
        "fraction_of_measured": vs_measured,
        "cpu_baseline": cpu,
        "next_rows": extras,
        "context": {"flashkda_gb300_us_per_layer_8192x4": 146,
                    "note": "the pages' number, other hardware; not a target"},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
