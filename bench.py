"""Throughput of the ReLU linear-attention hot path on one MI355X.

One step = the whole bidirectional path on the 720p-5s latent workload
(B=2, H=32, N=19320 tokens on a 21x23x40 grid, d=64, bf16, 3D RoPE, eps 1e-6):
la_state_reduce (S, z from K, V) then la_apply (O from Q, S, z).  Inputs are
resident in HBM before timing starts; consecutive steps rotate through enough
independent input sets (>= 2 GiB in all) that no step finds its operands in
the 256 MB Infinity Cache or in L2.

Prints one JSON line: tokens/s (value), the roofline of the dominant kernel
(algorithmic bytes per launch / HIP-event duration on the launch stream) and
the fp64 oracle's throughput on the host cores over a bounded sample.

Other workloads (--workload): sana2b (20 heads x d = 112), 720p60s (ten
block-causal steps), tc720p5s (token-causal), cross720p (cross-attention), and
tconv720p -- the Mix-FFN temporal convolution on one 720p-60s block at width
2240, whose roofline is the bf16 MFMA peak (algorithmic flops per launch / its
duration).  --summarize-trace / --summarize-pmc / --summarize-counters turn
rocprofv3 runs into the summaries under profiles/.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "linear-attn tokens/sec and achieved HBM GB/s (% peak), 720p-5s shape, 1 GPU"
HBM_PEAK_GBPS = 8000.0
WORKLOAD = "720p5s"
# The sources each workload's kernels are built from (their hash tags the
# committed counter summaries).
SRC_FILES = {
    "attention": ["la_common.h", "la_state.h", "la_apply.h", "la_causal.h", "la_api.hip"],
    "tconv": ["la_common.h", "la_tconv.h", "la_tconv.hip", "la_api.hip"],
}
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def kernel_source_hash(workload=None):
    h = hashlib.sha256()
    for f in SRC_FILES["tconv" if workload == "tconv720p" else "attention"]:
        with open(os.path.join(ROOT, "linear_attention_video_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# The bf16 state pass is one launch when a head's partials are small (its last
# workgroup per head sums them); otherwise, or with the tuning knob
# state_fused = 0, a separate combine launch follows it.
STATE_KERNELS = ("la_state_bf16_kernel",)
COMBINE_KERNEL = "la_state_combine_kernel"
APPLY_KERNELS = ("la_apply_bf16_kernel",)
CAUSAL_KERNELS = ("la_prefix_kernel", "la_causal_bf16_kernel")  # token-causal pass after the partials
TCONV_KERNELS = ("la_tconv_bf16_kernel",)
OUR_KERNELS = STATE_KERNELS + (COMBINE_KERNEL,) + APPLY_KERNELS + CAUSAL_KERNELS + TCONV_KERNELS
CALIB_KERNEL = "MulFunctor"   # torch's elementwise o = q * 1: a plain copy of known size
LIBGEMM_KERNEL = "Cijk_"      # hipBLASLt's GEMM kernels (context for the temporal convolution)


def traffic_json(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def profile_commands(workload):
    """The profiler runs whose summaries are committed (run from /tmp, with the
    repository at $REPO); the summaries are then written by --summarize-*."""
    wl = "" if workload == WORKLOAD else f" --workload {workload}"
    noextra = " --no-extra" if workload == "overlap720p" else ""
    return {
        "trace": "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d /tmp/la_prof/trace -o trace "
                 f"-- python3 $REPO/bench.py{wl} --steps 50 --warmup 5 --no-cpu-baseline{noextra}",
        "fetch": "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d /tmp/la_prof/fetch -o fetch "
                 f"-- python3 $REPO/bench.py{wl} --steps 10 --warmup 2 --prewarm-ms 0 --no-cpu-baseline",
        "write": "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d /tmp/la_prof/write -o write "
                 f"-- python3 $REPO/bench.py{wl} --steps 10 --warmup 2 --prewarm-ms 0 --no-cpu-baseline",
    }


def load_traffic(kernels, src_hash, workload=WORKLOAD):
    """HBM bytes per launch of a pass from the committed counter summary, or None.

    The summary records the kernel-source hash it was taken with; if the
    kernels changed since, the counters no longer describe them.
    """
    try:
        with open(traffic_json(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    per = t.get("kernels", {})
    if t.get("src_hash") != src_hash or any(k not in per for k in kernels):
        return None
    return sum(per[k]["hbm_bytes_per_launch"] for k in kernels)


def cpu_baseline(q, k, v, spec, budget_s=12.0):
    """Time the fp64 oracle on the workload's (batch, head) slices.

    Whole slices (all N tokens of one head), in order, pass after pass over the
    workload, until about budget_s of oracle time has been spent.
    """
    import numpy as np

    import oracle
    B, H, N, grid, eps = spec["B"], spec["H"], spec["N"], spec["grid"], spec["eps"]
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    slices, t_used = 0, 0.0
    order = [(b, h) for b in range(B) for h in range(H)]
    host = {}
    while t_used < budget_s:
        b, h = order[slices % len(order)]
        if (b, h) not in host:
            host[(b, h)] = tuple(x[b, h].float().cpu().numpy().astype(np.float64) for x in (q, k, v))
        qh, kh, vh = host[(b, h)]
        t0 = time.perf_counter()
        S, z = oracle.state(kh, vh, grid)
        oracle.apply(qh, S, z, grid, eps)
        t_used += time.perf_counter() - t0
        slices += 1
    tokens = slices * N / H  # a token is one grid position across all H heads
    one = _one_thread(lambda qh, kh, vh: oracle.apply(qh, *oracle.state(kh, vh, grid), grid, eps),
                      [host[o] for o in order if o in host], N / H, budget_s / 4)
    return {
        "value": tokens / t_used,
        "unit": "tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "one_thread": one,
        "sample": f"{slices} (batch, head) slices of the {WORKLOAD} workload in order "
                  f"({slices / len(order):.1f} passes over its {len(order)} slices), all {N} "
                  f"tokens each, fp64 numpy, {t_used:.1f} s of oracle time "
                  f"({len(os.sched_getaffinity(0))} host cores visible)",
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _one_thread(fn, samples, tokens_per_sample, budget_s):
    """The same oracle work with BLAS limited to one thread, over the first
    samples again, until about budget_s: tokens/s and what was run."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        return None
    done, t_used = 0, 0.0
    with threadpool_limits(limits=1):
        while t_used < budget_s and samples:
            t0 = time.perf_counter()
            fn(*samples[done % len(samples)])
            t_used += time.perf_counter() - t0
            done += 1
    return {"value": done * tokens_per_sample / t_used, "unit": "tokens/s", "cores": 1,
            "sample": f"{done} of the same samples, {t_used:.1f} s, BLAS limited to 1 thread"}


def cpu_baseline_tconv(X, W, cache, bias, spec, budget_s=12.0):
    """Time the fp64 oracle of the temporal convolution on the block's spatial
    positions, a few at a time (all frames of each), until about budget_s."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    B, T, P = spec["B"], spec["T"], spec["P"]
    Wh = W.float().cpu().numpy().astype(np.float64)
    bh = bias.float().cpu().numpy().astype(np.float64)
    per = 8
    done, t_used = 0, 0.0
    while t_used < budget_s and done < B * P:
        b, p0 = divmod(done, P)
        p1 = min(p0 + per, P)
        Xs = X[b:b + 1, :, p0:p1].float().cpu().numpy().astype(np.float64)
        cs = cache[b:b + 1, p0:p1].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oracle.temporal_conv(Xs, Wh, cs, bh)
        t_used += time.perf_counter() - t0
        done += p1 - p0
    samp = [(X[0:1, :, q0:q0 + per].float().cpu().numpy().astype(np.float64),
             cache[0:1, q0:q0 + per].float().cpu().numpy().astype(np.float64)) for q0 in range(0, min(P, 4 * per), per)]
    one = _one_thread(lambda xs, cs: oracle.temporal_conv(xs, Wh, cs, bh), samp, per * T, budget_s / 4)
    return {
        "value": done * T / t_used,
        "unit": "tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "one_thread": one,
        "sample": f"{done} of the block's {B * P} spatial positions, all {T} frames each "
                  f"({done * T} tokens), fp64 numpy, {t_used:.1f} s of oracle time "
                  f"({len(os.sched_getaffinity(0))} host cores visible)",
    }


class FenceFreeEvents:
    """Timing events without the system-scope fence (hipEventDisableSystemFence).

    A default HIP event makes its recording a system-scope release and acquire:
    L2 write-back and invalidation between the kernels it separates, which
    both adds a gap and slows the next kernel.  Events used only for timing do
    not need it.  Created through the HIP runtime PyTorch already loaded.
    """
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        import torch
        torch.cuda.init()
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime already in the process
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        self.stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.events = []

    def new(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.events.append(ev)
        return ev

    def record(self, ev):
        rc = self.hip.hipEventRecord(ev, self.stream())
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def wait(self, stream, ev):
        """Make `stream` (a torch stream) wait for `ev` (no host synchronisation)."""
        rc = self.hip.hipStreamWaitEvent(self.ct.c_void_p(stream.cuda_stream), ev, 0)
        if rc != 0:
            raise RuntimeError(f"hipStreamWaitEvent failed ({rc})")

    def ms(self, a, b):
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


def _find(path, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {path}")
    return hits[0]


def _short(name):
    for k in OUR_KERNELS:
        if k + "<" in name or name.startswith(k):
            return k
    if CALIB_KERNEL in name:
        return "calibration copy (torch mul by 1)"
    if name.startswith(LIBGEMM_KERNEL):
        return "hipBLASLt GEMM (torch.matmul, context)"
    return None


WORKLOAD_TITLES = {
    WORKLOAD: "720p5s workload (bf16, B=2 H=32 N=19320 d=64, RoPE)",
    "sana2b": "sana2b workload (SANA-Video-2B heads: bf16, B=1 H=20 N=19320 d=112, RoPE)",
    "cross720p": "cross720p workload (cross-attention in one launch: bf16, B=2 H=32, 19320 video queries over "
                 "300 text keys/values, d=64, no RoPE)",
    "tc720p5s": "tc720p5s workload (token-causal: bf16, B=2 H=32 N=19320 d=64, RoPE)",
    "720p60s": "720p60s workload (block-causal: bf16, B=1 H=32 N=220800 in 10 blocks of 22080, d=64, RoPE)",
    "overlap720p": "overlap720p diagnostic (the 720p5s step as its two batch elements on two streams, "
                   "each one's state pass then its apply)",
    "tconv720p": "tconv720p workload (temporal convolution, bf16, one block of 24 frames x 920 "
                 "positions, D=2240, bias)",
}


def summarize_trace(trace_dir, command, out_path, workload=WORKLOAD):
    """Per-kernel durations of the timed steps from a rocprofv3 --kernel-trace run."""
    import csv
    rows = list(csv.DictReader(open(_find(trace_dir, "kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    la = [r for r in rows if _short(r["Kernel_Name"]) in OUR_KERNELS]
    steps = sum(1 for r in la if _short(r["Kernel_Name"]) in APPLY_KERNELS)
    dur = {}
    for r in la:
        dur.setdefault(_short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    stats = list(csv.DictReader(open(_find(trace_dir, "kernel_stats.csv"))))
    lines = [f"# Kernel durations, {WORKLOAD_TITLES[workload]}", "",
             "Command (from the repository root, one MI355X):", "", "```", command, "```", "",
             "rocprofv3 --stats summary, this library's kernels (all launches, warm-up included):", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for st in stats:
        k = _short(st["Name"])
        if k in OUR_KERNELS or (k or "").startswith("hipBLASLt"):
            lines.append(f"| {k} | {st['Calls']} | {float(st['AverageNs']) / 1e3:.1f} | "
                         f"{float(st['MinNs']) / 1e3:.1f} | {float(st['MaxNs']) / 1e3:.1f} |")
    if workload == "overlap720p":
        # every step is 4 launches (state and apply of each batch element, two
        # streams) between a fork and a join: consecutive groups of 4 by start
        t = lambda r, k: int(r[k]) / 1e3
        n = len(la) // 4
        spans, busy, st_us, ap_us, conc = [], [], [], [], []
        for i in range(n):
            g = la[4 * i:4 * i + 4]
            t0, t1 = min(t(r, "Start_Timestamp") for r in g), max(t(r, "End_Timestamp") for r in g)
            spans.append(t1 - t0)
            busy.append(sum(t(r, "End_Timestamp") - t(r, "Start_Timestamp") for r in g))
            for r in g:
                (st_us if _short(r["Kernel_Name"]) in STATE_KERNELS else ap_us).append(
                    t(r, "End_Timestamp") - t(r, "Start_Timestamp"))
            # time two launches of the step run at once: the two state passes, the two
            # applies, and a state pass with the other group's apply
            sts = [r for r in g if _short(r["Kernel_Name"]) in STATE_KERNELS]
            aps = [r for r in g if _short(r["Kernel_Name"]) in APPLY_KERNELS]

            def both(a_, b_):
                return max(0.0, min(t(a_, "End_Timestamp"), t(b_, "End_Timestamp")) -
                           max(t(a_, "Start_Timestamp"), t(b_, "Start_Timestamp")))
            conc.append((both(*sts) if len(sts) == 2 else 0.0, both(*aps) if len(aps) == 2 else 0.0,
                         sum(both(a_, b_) for a_ in sts for b_ in aps)))
        if n:
            lines += ["", f"From the trace, over {n} steps (4 launches each, two streams):", "",
                      f"- step span (first launch start to last launch end): {sum(spans) / n:.1f} us",
                      f"- sum of the 4 launch durations: {sum(busy) / n:.1f} us",
                      f"- state kernel (half batch) average: {sum(st_us) / len(st_us):.1f} us; "
                      f"apply (half batch) average: {sum(ap_us) / len(ap_us):.1f} us",
                      f"- time two launches run at once, per step: the two state passes "
                      f"{sum(c[0] for c in conc) / n:.1f} us, the two applies {sum(c[1] for c in conc) / n:.1f} us, "
                      f"a state pass with an apply {sum(c[2] for c in conc) / n:.1f} us"]
        with open(out_path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return steps

    # per pass, from the trace: state kernel start .. (combine end) .. last kernel's end,
    # the last kernel being the apply (or the causal scan in token-causal mode)
    t = lambda r, k: int(r[k]) / 1e3
    last = CAUSAL_KERNELS[1:] if workload == "tc720p5s" else APPLY_KERNELS
    steps_ = []
    for i, r in enumerate(la):
        if _short(r["Kernel_Name"]) not in STATE_KERNELS:
            continue
        j = i + 1
        while j < len(la) and _short(la[j]["Kernel_Name"]) in (COMBINE_KERNEL, CAUSAL_KERNELS[0]):
            j += 1
        if j < len(la) and _short(la[j]["Kernel_Name"]) in last:
            pass_end = t(la[j - 1], "End_Timestamp")
            steps_.append((pass_end - t(r, "Start_Timestamp"), t(la[j], "Start_Timestamp") - pass_end,
                           t(la[j], "End_Timestamp") - t(r, "Start_Timestamp"), t(r, "Start_Timestamp"),
                           t(la[j], "End_Timestamp")))
    if steps_:
        n = len(steps_)
        what = {"tc720p5s": ("state kernel start to the causal scan's end", "partial states",
                             "partial states -> scan"),
                "720p60s": ("one block step: state kernel start to apply kernel end", "state pass",
                            "state pass -> apply")}.get(
            workload, ("state kernel start to apply kernel end", "state pass", "state pass -> apply"))
        lines += ["", f"From the trace, over {n} passes ({what[0]}):", "",
                  f"- {what[1]} (state kernel start to the end of the launch before the last kernel): "
                  f"{sum(g[0] for g in steps_) / n:.1f} us",
                  f"- gap {what[2]}: {sum(g[1] for g in steps_) / n:.2f} us",
                  f"- whole pass: {sum(g[2] for g in steps_) / n:.1f} us"]
        if workload == "720p60s" and n >= 10:
            # ten block steps make one step of the sequence (every step runs all blocks)
            seq = [steps_[i + 9][4] - steps_[i][3] for i in range(0, n - 9, 10)]
            lines.append(f"- whole 10-block sequence (block 0's state start to block 9's apply end), "
                         f"over {len(seq)} sequences: {sum(seq) / len(seq):.1f} us")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return steps


def summarize_pmc(fetch_dir, write_dir, commands, out_json, out_md, src_hash, tensor_bytes, algo=None,
                  workload=WORKLOAD):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE runs, scaled by a copy kernel.

    Both counters are in KiB per dispatch.  The calibration kernel reads
    `tensor_bytes` and writes `tensor_bytes`; the ratio of those to what the
    counters report for it scales every other kernel's counts.
    """
    import csv

    def per_kernel(d, counter):
        acc = {}
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            k = _short(r["Kernel_Name"])
            if k is None or r["Counter_Name"] != counter:
                continue
            acc.setdefault(k, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    cal = "calibration copy (torch mul by 1)"
    if cal not in fetch or cal not in write:
        raise SystemExit("calibration copy kernel missing from the counter runs")
    f_scale = tensor_bytes / fetch[cal]
    w_scale = tensor_bytes / write[cal]
    if algo is None:
        algo = {"la_state_bf16_kernel": 2 * tensor_bytes, "la_apply_bf16_kernel": 2 * tensor_bytes}
    kernels = {}
    for k in OUR_KERNELS:
        if k in fetch and k in write:
            rd, wr = fetch[k] * f_scale, write[k] * w_scale
            kernels[k] = {"fetch_bytes_raw": fetch[k], "write_bytes_raw": write[k],
                          "read_bytes": rd, "write_bytes": wr, "hbm_bytes_per_launch": rd + wr,
                          "algorithmic_bytes": algo.get(k)}
    out = {"workload": workload, "src_hash": src_hash, "fetch_scale": f_scale, "write_scale": w_scale,
           "calibration": f"{cal}: reads {tensor_bytes} B and writes {tensor_bytes} B per launch",
           "commands": commands, "kernels": kernels}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    lines = [f"# HBM traffic per launch, {workload} workload", "", "Commands (repository root, one MI355X):",
             "", "```", *commands, "```", "",
             f"Scale factors from the calibration copy (reads and writes {tensor_bytes / 1e6:.1f} MB): "
             f"FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f}.", "",
             "| kernel | FETCH_SIZE raw MB | WRITE_SIZE raw MB | read MB (scaled) | write MB (scaled) | "
             "algorithmic MB |", "|---|---|---|---|---|---|"]
    for k, v in kernels.items():
        a = v["algorithmic_bytes"]
        lines.append(f"| {k} | {v['fetch_bytes_raw'] / 1e6:.1f} | {v['write_bytes_raw'] / 1e6:.2f} | "
                     f"{v['read_bytes'] / 1e6:.1f} | {v['write_bytes'] / 1e6:.2f} | "
                     f"{a / 1e6 if a else 0:.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE"


def summarize_counters(dirs, out_path):
    """MFMA utilisation per kernel from rocprofv3 --pmc runs of MFMA_COUNTERS.

    SQ_VALU_MFMA_BUSY_CYCLES sums over the 4 SIMDs of every CU and
    SQ_BUSY_CU_CYCLES over the CUs, so utilisation = busy / (4 * CU cycles).
    """
    import csv
    lines = ["# MFMA utilisation of this library's kernels", "", "Commands (repository root, one MI355X):", "",
             "```"]
    for wl in dirs:
        flag = "" if wl == WORKLOAD else f" --workload {wl}"
        lines.append(f"cd /tmp && rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d /tmp/la_prof/mfma_{wl} "
                     f"-o p -- python3 $REPO/bench.py{flag} --steps 10 --warmup 2 --prewarm-ms 0 --no-cpu-baseline")
    lines += ["python3 bench.py --summarize-counters " + " ".join(f"{w}=/tmp/la_prof/mfma_{w}" for w in dirs),
              "```", "", "utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES), mean over the dispatches "
              "of each kernel (warm-up included).", "",
              "| workload | kernel | dispatches | MFMA instructions | MFMA busy (SIMD cycles) | CU busy cycles | "
              "utilisation |", "|---|---|---|---|---|---|---|"]
    for wl, d in dirs.items():
        acc = {}
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            k = _short(r["Kernel_Name"])
            if k is None or k not in OUR_KERNELS:
                continue
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for k, c in acc.items():
            mean = {n: sum(v) / len(v) for n, v in c.items()}
            busy, cu = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), mean.get("SQ_BUSY_CU_CYCLES", 0.0)
            util = busy / (4 * cu) if cu else 0.0
            lines.append(f"| {wl} | {k} | {len(c.get('SQ_BUSY_CU_CYCLES', []))} | {mean.get('SQ_INSTS_MFMA', 0):.0f} | "
                         f"{busy:.3e} | {cu:.3e} | {100 * util:.1f}% |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-ms", type=float, default=200.0,
                    help="before the warm-up steps, run untimed steps for this long so that the GPU "
                         "reaches its steady clock (from idle it needs tens of ms)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip a workload's extra measurements (library GEMM, stream comparisons)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--workload", default=WORKLOAD, choices=[WORKLOAD, "cross720p", "720p60s", "tc720p5s", "sana2b", "tconv720p", "sweep",
                             "overlap720p"],
                    help="default: the headline 720p-5s bidirectional step")
    ap.add_argument("--event-every", type=int, default=8,
                    help="record per-kernel events on every n-th timed step (each event costs ~2 us)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write the kernel-duration summary of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM-traffic summary of rocprofv3 FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--summarize-counters", nargs="+", metavar="WORKLOAD=DIR",
                    help="write the MFMA-utilisation summary of rocprofv3 --pmc runs of " + MFMA_COUNTERS)
    ap.add_argument("--summarize-sweep", nargs="+", metavar=("JSON", "TRACE_DIR"),
                    help="write profiles/sweep_scaling.md from a --workload sweep JSON line (and its trace)")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"), help="where summaries go")
    args = ap.parse_args()
    if args.summarize_sweep:
        os.makedirs(args.out, exist_ok=True)
        summarize_sweep(args.summarize_sweep[0], args.summarize_sweep[1] if len(args.summarize_sweep) > 1 else None,
                        os.path.join(args.out, "sweep_scaling.md"))
        return
    if args.summarize_counters:
        os.makedirs(args.out, exist_ok=True)
        summarize_counters(dict(x.split("=", 1) for x in args.summarize_counters),
                           os.path.join(args.out, "mfma_utilisation.md"))
        return
    if args.summarize_trace or args.summarize_pmc:
        wlname = args.workload
        if wlname not in WORKLOAD_TITLES:
            raise SystemExit(f"no profile summary for workload {wlname}")
        wlflag = "" if wlname == WORKLOAD else f" --workload {wlname}"
        algo = None
        if wlname == "tconv720p":
            from linear_attention_video_02_amd.inputs import TCONV
            w = TCONV[wlname]
            tensor_bytes = w["B"] * w["T"] * w["P"] * w["D"] * 2  # the calibration copy moves X
            # minimum HBM bytes of one launch: X and W read once, Y written once
            algo = {"la_tconv_bf16_kernel": 2 * tensor_bytes + 3 * w["D"] * w["D"] * 2}
        elif wlname == "cross720p":
            from linear_attention_video_02_amd.inputs import CROSS
            w = CROSS[wlname]
            tensor_bytes = w["B"] * w["H"] * w["Nq"] * w["d"] * 2  # the calibration copy moves Q
            tkv = w["B"] * w["H"] * w["Nkv"] * w["d"] * 2
            algo = {"la_apply_bf16_kernel": 2 * tensor_bytes + 2 * tkv}  # one launch: Q, K, V in, O out
        else:
            from linear_attention_video_02_amd.inputs import WORKLOADS
            w = WORKLOADS["720p5s" if wlname in ("tc720p5s", "overlap720p") else wlname]
            n_tok = w["block"] if wlname == "720p60s" else w["N"]  # per launch: one block
            tensor_bytes = w["B"] * w["H"] * n_tok * w["d"] * 2
            if wlname == "tc720p5s":
                # each kernel's own stream: the partial-state pass reads K and V of every
                # chunk but each head's last (no carry is returned), the scan reads Q, K, V
                # and writes O (the path's minimum is 4 tensors).  Chunks as the library
                # plans them by default: P = 512 / (B H) per head, 128-token aligned.
                P = max(1, min(64, 512 // (w["B"] * w["H"])))
                chunk = -(-w["N"] // P)
                chunk = -(-chunk // 128) * 128
                last = w["N"] - (-(-w["N"] // chunk) - 1) * chunk
                algo = {"la_state_bf16_kernel": 2 * tensor_bytes * (w["N"] - last) // w["N"],
                        "la_causal_bf16_kernel": 4 * tensor_bytes}
        cmds_ = profile_commands(wlname)
        os.makedirs(args.out, exist_ok=True)
        if args.summarize_trace:
            summarize_trace(args.summarize_trace,
                            cmds_["trace"] + f"\npython3 bench.py{wlflag} --summarize-trace /tmp/la_prof/trace",
                            os.path.join(args.out, f"kernels_{wlname}.md"), wlname)
        if args.summarize_pmc:
            cmds = [cmds_["fetch"], cmds_["write"],
                    f"python3 bench.py{wlflag} --summarize-pmc /tmp/la_prof/fetch /tmp/la_prof/write"]
            summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], cmds,
                          os.path.join(args.out, f"traffic_{wlname}.json"),
                          os.path.join(args.out, f"traffic_{wlname}.md"), kernel_source_hash(wlname), tensor_bytes,
                          algo, wlname)
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (got --gpus {args.gpus}); "
              "across GPUs the bidirectional path would shard by (batch, head), with no "
              "communication", file=sys.stderr)
        sys.exit(2)

    if args.workload == "sweep":
        run_sweep(args)
        return

    import torch

    import linear_attention_video_02_amd as la

    if not os.path.exists(la.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    wl = setup_workload(args.workload, la, dev)
    tev = FenceFreeEvents()
    step = wl["step"]

    # clock ramp: untimed steps for about prewarm_ms, then the W warm-up steps
    t_pre, n_pre = time.perf_counter(), 0
    while (time.perf_counter() - t_pre) * 1e3 < args.prewarm_ms:
        for _ in range(8):
            step(n_pre, None, tev)
            n_pre += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i, None, tev)
    torch.cuda.synchronize()
    every = max(1, args.event_every)
    ngroups = len(wl["groups"])
    evs = {i: [tev.new() for _ in range(ngroups + 1)] for i in range(0, args.steps, every)}
    start, stop = tev.new(), tev.new()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tev.record(start)
    for i in range(args.steps):
        step(args.warmup + i, evs.get(i), tev)
    tev.record(stop)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = tev.ms(start, stop) / args.steps
    group_ms = [sum(tev.ms(e[g], e[g + 1]) for e in evs.values()) / len(evs) for g in range(ngroups)]
    keys = sorted(evs)
    step_ms = sorted([tev.ms(evs[a][0], evs[b][0]) / (b - a) for a, b in zip(keys, keys[1:])]) or [ms_step]

    def pct(xs, f):
        return xs[min(len(xs) - 1, int(f * len(xs)))]

    # dominant launch group: algorithmic bytes per launch / its mean event duration
    g = max(range(ngroups), key=lambda i: group_ms[i])
    gname, kernels, nbytes = wl["groups"][g][:3]
    # launches of each kernel in one pass of the group (the counter summary is per launch)
    nlaunch = wl["groups"][g][3] if len(wl["groups"][g]) > 3 else 1
    dur_ms = group_ms[g]
    rf = wl.get("roofline", {"bound": "hbm", "peak": HBM_PEAK_GBPS, "unit": "GB/s", "scale": 1e9})
    achieved = nbytes / (dur_ms * 1e-3) / rf["scale"]
    src_hash = kernel_source_hash(args.workload)
    traffic = load_traffic(kernels, src_hash, args.workload)
    if traffic is not None:
        traffic *= nlaunch

    # Calibration copy o = q * 1 over rotating buffers: a plain elementwise
    # copy of known size (reads and writes copy_bytes), timed as the practical
    # HBM ceiling for a read+write stream and used to scale the byte counters.
    pairs = wl["copy_pairs"]
    copy_bytes = pairs[0][0].numel() * pairs[0][0].element_size()
    for i in range(3):
        torch.mul(pairs[i % len(pairs)][0], 1, out=pairs[i % len(pairs)][1])
    torch.cuda.synchronize()
    c0, c1 = tev.new(), tev.new()
    n_copy = 4 * len(pairs)
    tev.record(c0)
    for i in range(n_copy):
        torch.mul(pairs[i % len(pairs)][0], 1, out=pairs[i % len(pairs)][1])
    tev.record(c1)
    torch.cuda.synchronize()
    copy_gbps = 2 * copy_bytes / (tev.ms(c0, c1) / n_copy * 1e-3) / 1e9
    # the same copy through this library's plain copy kernel (la_stream_copy)
    for i in range(3):
        la.stream_copy(pairs[i % len(pairs)][0], pairs[i % len(pairs)][1])
    torch.cuda.synchronize()
    c2, c3 = tev.new(), tev.new()
    tev.record(c2)
    for i in range(n_copy):
        la.stream_copy(pairs[i % len(pairs)][0], pairs[i % len(pairs)][1])
    tev.record(c3)
    torch.cuda.synchronize()
    copy_repo_gbps = 2 * copy_bytes / (tev.ms(c2, c3) / n_copy * 1e-3) / 1e9
    tev.close()

    out = {
        "metric": wl["metric"],
        "value": wl["tokens_per_step"] / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm": {"ms": args.prewarm_ms, "steps": n_pre,
                    "what": "untimed steps before the warm-up steps, for the GPU clock to ramp up"},
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": wl["config"],
        "roofline": {
            "bound": rf["bound"],
            "achieved": achieved,
            "peak": rf["peak"],
            "unit": rf["unit"],
            "frac": achieved / rf["peak"],
            "traffic": traffic,
            "kernel": "+".join(kernels),
            ("algorithmic_flops" if rf["bound"] == "mfma" else "algorithmic_bytes"): nbytes,
            "duration_us": dur_ms * 1e3,
            "traffic_over_algorithmic": traffic / nbytes if traffic and rf["bound"] == "hbm" else None,
        },
        "step_GBps": wl["step_bytes"] / (ms_step * 1e-3) / 1e9,
        "step_frac_of_peak": wl["step_bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "kernels_us": {wl["groups"][i][0]: group_ms[i] * 1e3 for i in range(ngroups)},
        "step_us_p10_p50_p90": [pct(step_ms, 0.1) * 1e3, pct(step_ms, 0.5) * 1e3, pct(step_ms, 0.9) * 1e3],
        "timing": f"HIP events without system-scope fence on the launch stream; per-group events "
                  f"on every {every}th timed step ({len(evs)} samples)",
        "copy_GBps": copy_gbps,
        "copy_kind": "torch mul by 1 (read + write, rotating buffers)",
        "copy_repo_GBps": copy_repo_gbps,
        "copy_repo_kind": "la_stream_copy: this library's plain 16-byte-per-lane copy, same buffers",
        "wall_s": wall,
        "src_hash": src_hash,
    }
    if "extra" in wl and not args.no_extra:
        out.update(wl["extra"](tev_factory=FenceFreeEvents))
    if not args.no_cpu_baseline and "cpu_baseline" in wl:
        out["cpu_baseline"] = wl["cpu_baseline"](args.cpu_budget)
    print(json.dumps(out), flush=True)


def run_sweep(args):
    """Time the bidirectional step (la_state_reduce + la_apply) over the d x N
    sweep (B1 H32, d in {32, 64, 128}, N in {4096 .. 220800}, grid ceil(N/920)
    x 23 x 40) and check that time grows linearly in N at fixed d (Table 1's
    O(N) claim): a least-squares fit t = a + b N per d, and the time per token
    at the two largest N.  Prints one JSON line."""
    import numpy as np
    import torch

    import linear_attention_video_02_amd as la
    from linear_attention_video_02_amd.inputs import SWEEP_D, SWEEP_N, WORKLOADS, make_qkv_device
    dev = torch.device("cuda:0")
    tev = FenceFreeEvents()
    points = []
    for d in SWEEP_D:
        for N in SWEEP_N:
            w = WORKLOADS[f"sweep_d{d}_n{N}"]
            B, H, grid, eps = w["B"], w["H"], w["grid"], w["eps"]
            q, k, v = make_qkv_device(B, H, N, d, "bf16", w["seed"], dev)
            tb = q.numel() * q.element_size()
            nsets = max(2, math.ceil(2 * 2**30 / (4 * tb)))
            sets = [(q, k, v)] + [tuple(t.clone() for t in (q, k, v)) for _ in range(nsets - 1)]
            outs = [torch.empty_like(q) for _ in range(nsets)]
            S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
            z = torch.empty((B, H, d), dtype=torch.float32, device=dev)
            ws = la.workspace(B, H, N, d, dev)

            def step(i):
                qi, ki, vi = sets[i % nsets]
                la.state_reduce(ki, vi, grid, S=S, z=z, ws=ws)
                la.apply(qi, S, z, grid, eps, out=outs[i % nsets])
            # warm-up: at least 3 steps and about prewarm_ms / 4 (clock ramp)
            t_w, i_w = time.perf_counter(), 0
            while i_w < 3 or (time.perf_counter() - t_w) * 1e3 < args.prewarm_ms / 4:
                step(i_w)
                i_w += 1
                if i_w % 8 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            iters = max(10, min(200, int(50e-3 / max(4 * tb / 5e12, 1e-6))))
            e0, e1 = tev.new(), tev.new()
            tev.record(e0)
            for i in range(iters):
                step(i)
            tev.record(e1)
            torch.cuda.synchronize()
            us = tev.ms(e0, e1) / iters * 1e3
            points.append({"d": d, "N": N, "us": us, "tokens_per_s": B * N / (us * 1e-6),
                           "GBps": 4 * tb / (us * 1e-6) / 1e9, "iters": iters, "input_sets": nsets})
            print(f"sweep d={d} N={N}: {us:.1f} us, {4 * tb / (us * 1e-6) / 1e9:.0f} GB/s", file=sys.stderr,
                  flush=True)
            del sets, outs, q, k, v
            torch.cuda.empty_cache()
    tev.close()
    linear = {}
    for d in SWEEP_D:
        pts = [p_ for p_ in points if p_["d"] == d]
        Ns = np.array([p_["N"] for p_ in pts], dtype=np.float64)
        ts = np.array([p_["us"] for p_ in pts], dtype=np.float64)
        b_, a_ = np.polyfit(Ns, ts, 1)
        pred = a_ + b_ * Ns
        r2 = 1.0 - float(((ts - pred) ** 2).sum() / ((ts - ts.mean()) ** 2).sum())
        per_tok = ts / Ns
        linear[str(d)] = {"fit_us": [float(a_), float(b_) * 1e6], "fit_units": "us = a + b * (N / 1e6)",
                          "r2": r2, "us_per_Mtoken_largest_two": [float(per_tok[-2] * 1e6), float(per_tok[-1] * 1e6)]}
    top = [p_ for p_ in points if p_["d"] == 64][-1]
    out = {
        "metric": "linear-attn tokens/sec over the d x N sweep (B1 H32, bidirectional, RoPE), 1 GPU",
        "value": top["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": None, "warmup": 3,
        "ms_per_step": top["us"] / 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "sweep", "value_point": {"d": 64, "N": top["N"]}},
        "sweep": points, "linearity": linear,
    }
    print(json.dumps(out), flush=True)


SWEEP_TRACE_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d /tmp/la_prof/sweep "
                   "-o tr -- python3 $REPO/bench.py --workload sweep")


def summarize_sweep(json_path, trace_dir, out_path):
    """profiles/sweep_scaling.md from a `bench.py --workload sweep` JSON line and,
    if given, a rocprofv3 kernel trace of the same command (per-kernel rates at
    the largest N: the sweep runs its points in order, so the last launches of
    each kernel instance belong to the largest N of that head size)."""
    import csv
    d_ = json.loads(open(json_path).read().strip().splitlines()[-1])
    pts, lin = d_["sweep"], d_["linearity"]
    lines = ["# d x N sweep: linear scaling of the bidirectional step", "",
             "Commands (repository root, one MI355X):", "", "```",
             "python3 bench.py --workload sweep > /tmp/la_prof/sweep.json"]
    if trace_dir:
        lines.append(SWEEP_TRACE_CMD)
    lines += ["python3 bench.py --summarize-sweep /tmp/la_prof/sweep.json" +
              (" /tmp/la_prof/sweep" if trace_dir else ""), "```", "",
              "B = 1, H = 32, bf16, grid ceil(N/920) x 23 x 40 with RoPE; one step = la_state_reduce + "
              "la_apply, inputs rotating over >= 2 GiB of independent sets, each point warmed for >= 50 ms; "
              "HIP events on the launch stream.", "",
              "| d | N | us per step | tokens/s | GB/s (Q, K, V, O) |", "|---|---|---|---|---|"]
    for p_ in pts:
        lines.append(f"| {p_['d']} | {p_['N']} | {p_['us']:.1f} | {p_['tokens_per_s'] / 1e6:.1f}M | "
                     f"{p_['GBps']:.0f} |")
    lines += ["", "Least-squares fit per head size, t = a + b * (N / 1e6) (Table 1's O(N) claim):", "",
              "| d | a (us) | b (us per M tokens) | R^2 | us per M tokens at the two largest N |",
              "|---|---|---|---|---|"]
    for d, v in lin.items():
        a_, b_ = v["fit_us"]
        t1, t2 = v["us_per_Mtoken_largest_two"]
        lines.append(f"| {d} | {a_:.1f} | {b_:.0f} | {v['r2']:.5f} | {t1:.0f} / {t2:.0f} |")
    lines += ["", "The intercept is the fixed cost of the two launches and their set-up; the slope doubles "
              "with d (bytes per token are proportional to d), and the time per token keeps falling toward "
              "the slope as N grows."]
    if trace_dir:
        rows = list(csv.DictReader(open(_find(trace_dir, "kernel_trace.csv"))))
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        by = {}
        for r in rows:
            k = _short(r["Kernel_Name"])
            if k in STATE_KERNELS + APPLY_KERNELS:
                m = re.search(r"<(\d+)", r["Kernel_Name"])
                dd = int(m.group(1)) if m else 0
                by.setdefault((k, dd), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        nmax = max(p_["N"] for p_ in pts)
        lines += ["", f"Per kernel at N = {nmax} (mean of the last 20 launches of each kernel of that head size):",
                  "", "| d | state kernel | apply kernel | bytes per pass | state | apply |", "|---|---|---|---|---|---|"]
        for d in sorted({p_["d"] for p_ in pts}):
            st = by.get((STATE_KERNELS[0], d), [])[-20:]
            ap = by.get((APPLY_KERNELS[0], d), [])[-20:]
            if not st or not ap:
                continue
            nb = 2 * 32 * nmax * d * 2
            ts, ta = sum(st) / len(st), sum(ap) / len(ap)
            lines.append(f"| {d} | {ts:.1f} us | {ta:.1f} us | {nb / 1e6:.0f} MB | {nb / ts / 1e6:.1f} TB/s | "
                         f"{nb / ta / 1e6:.1f} TB/s |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def setup_workload(name, la, dev):
    """Device inputs, the step function and the launch groups of one workload.

    Every workload rotates through enough independent input sets (>= 2 GiB in
    all) that no step finds its operands in the Infinity Cache or in L2.
    """
    import torch

    from linear_attention_video_02_amd.inputs import CROSS, WORKLOADS, make_cross_device, make_qkv_device

    def rotating(tensors_of_set0, clone_count):
        sets = [tensors_of_set0]
        for _ in range(clone_count - 1):
            sets.append(tuple(t.clone() for t in tensors_of_set0))
        return sets

    def n_sets_for(set_bytes):
        return max(2, math.ceil(2 * 2**30 / set_bytes))

    if name == "720p5s":
        spec = WORKLOADS[name]
        B, H, N, d, grid, eps = spec["B"], spec["H"], spec["N"], spec["d"], spec["grid"], spec["eps"]
        q, k, v = make_qkv_device(B, H, N, d, "bf16", spec["seed"], dev)
        tb = q.numel() * q.element_size()
        base = rotating((q, k, v), n_sets_for(4 * tb))
        sets = [(qi, ki, vi, torch.empty_like(q), torch.empty((B, H, d, d), dtype=torch.float32, device=dev),
                 torch.empty((B, H, d), dtype=torch.float32, device=dev)) for (qi, ki, vi) in base]
        ws = la.workspace(B, H, N, d, dev)

        def step(i, ev, tev):
            qi, ki, vi, oi, S, z = sets[i % len(sets)]
            if ev is not None:
                tev.record(ev[0])
            la.state_reduce(ki, vi, grid, S=S, z=z, ws=ws)
            if ev is not None:
                tev.record(ev[1])
            la.apply(qi, S, z, grid, eps, out=oi)
            if ev is not None:
                tev.record(ev[2])

        return {
            "metric": METRIC, "step": step, "tokens_per_step": B * N, "step_bytes": 4 * tb,
            "config": {"workload": name, "B": B, "H": H, "N": N, "d": d, "grid": list(grid), "eps": eps,
                       "input_sets": len(sets)},
            "groups": [("state", STATE_KERNELS, 2 * tb), ("apply", APPLY_KERNELS, 2 * tb)],
            "copy_pairs": [(s[0], s[3]) for s in sets],
            "cpu_baseline": lambda budget: cpu_baseline(q, k, v, spec, budget),
        }

    if name == "sana2b":
        spec = WORKLOADS[name]
        B, H, N, d, grid, eps = spec["B"], spec["H"], spec["N"], spec["d"], spec["grid"], spec["eps"]
        q, k, v = make_qkv_device(B, H, N, d, "bf16", spec["seed"], dev)
        tb = q.numel() * q.element_size()
        base = rotating((q, k, v), n_sets_for(4 * tb))
        sets = [(qi, ki, vi, torch.empty_like(q), torch.empty((B, H, d, d), dtype=torch.float32, device=dev),
                 torch.empty((B, H, d), dtype=torch.float32, device=dev)) for (qi, ki, vi) in base]
        ws = la.workspace(B, H, N, d, dev)

        def step(i, ev, tev):
            qi, ki, vi, oi, S, z = sets[i % len(sets)]
            if ev is not None:
                tev.record(ev[0])
            la.state_reduce(ki, vi, grid, S=S, z=z, ws=ws)
            if ev is not None:
                tev.record(ev[1])
            la.apply(qi, S, z, grid, eps, out=oi)
            if ev is not None:
                tev.record(ev[2])

        return {
            "metric": "linear-attn tokens/sec and achieved HBM GB/s (% peak), SANA-Video-2B heads "
                      "(H=20, d=112) on the 720p-5s latent, 1 GPU",
            "step": step, "tokens_per_step": B * N, "step_bytes": 4 * tb,
            "config": {"workload": name, "B": B, "H": H, "N": N, "d": d, "grid": list(grid), "eps": eps,
                       "input_sets": len(sets)},
            "groups": [("state", STATE_KERNELS, 2 * tb), ("apply", APPLY_KERNELS, 2 * tb)],
            "copy_pairs": [(s_[0], s_[3]) for s_ in sets],
        }

    if name == "cross720p":
        w = CROSS[name]
        B, H, Nq, Nkv, d, eps = w["B"], w["H"], w["Nq"], w["Nkv"], w["d"], w["eps"]
        q, k, v = make_cross_device(B, H, Nq, Nkv, d, "bf16", w["seed"], dev)
        tq = q.numel() * q.element_size()
        tkv = k.numel() * k.element_size()
        base = rotating((q, k, v), n_sets_for(2 * tq + 2 * tkv))
        sets = [(qi, ki, vi, torch.empty_like(q)) for (qi, ki, vi) in base]
        ws = la.cross_workspace(B, H, Nkv, d, dev)

        def step(i, ev, tev):
            # one library call: at these sizes one launch (each apply workgroup
            # forms its heads' S and z from the 300 keys/values)
            qi, ki, vi, oi = sets[i % len(sets)]
            if ev is not None:
                tev.record(ev[0])
            la.cross_attention(qi, ki, vi, eps, out=oi, ws=ws)
            if ev is not None:
                tev.record(ev[1])

        return {
            "metric": "linear cross-attn video tokens/sec and achieved HBM GB/s (% peak), 720p-5s video "
                      "queries over 300 text tokens, 1 GPU",
            "step": step, "tokens_per_step": B * Nq, "step_bytes": 2 * tq + 2 * tkv,
            "config": {"workload": name, "B": B, "H": H, "N_q": Nq, "N_kv": Nkv, "d": d, "eps": eps,
                       "input_sets": len(sets)},
            "groups": [("cross", APPLY_KERNELS, 2 * tq + 2 * tkv)],
            "copy_pairs": [(s[0], s[3]) for s in sets],
        }

    if name == "overlap720p":
        # Diagnostic, not the headline: the 720p-5s step split into two head
        # groups (its two batch elements), each group's state pass then its
        # apply on a stream of its own, so that one group's pass can drain
        # while the other's ramps up.  The comparison figures in the JSON line
        # time the whole batch on one stream and the two groups on one stream.
        spec = WORKLOADS["720p5s"]
        B, H, N, d, grid, eps = spec["B"], spec["H"], spec["N"], spec["d"], spec["grid"], spec["eps"]
        q, k, v = make_qkv_device(B, H, N, d, "bf16", spec["seed"], dev)
        tb = q.numel() * q.element_size()
        base = rotating((q, k, v), n_sets_for(4 * tb))
        sets = [(qi, ki, vi, torch.empty_like(q), torch.empty((B, H, d, d), dtype=torch.float32, device=dev),
                 torch.empty((B, H, d), dtype=torch.float32, device=dev)) for (qi, ki, vi) in base]
        main = torch.cuda.current_stream()
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
        ws_half = [torch.zeros(la.workspace_bytes(1, H, N, d, grid), dtype=torch.uint8, device=dev)
                   for _ in streams]
        ws_all = la.workspace(B, H, N, d, dev, grid=grid)
        pool = []

        def group(h, i, ws):
            qi, ki, vi, oi, S, z = sets[i % len(sets)]
            sl = slice(h, h + 1)
            la.state_reduce(ki[sl], vi[sl], grid, S=S[sl], z=z[sl], ws=ws)
            la.apply(qi[sl], S[sl], z[sl], grid, eps, out=oi[sl])

        def step(i, ev, tev):
            if not pool:
                pool.extend(tev.new() for _ in range(3))
            if ev is not None:
                tev.record(ev[0])
            tev.record(pool[0])
            for h, st in enumerate(streams):
                tev.wait(st, pool[0])
                with torch.cuda.stream(st):
                    group(h, i, ws_half[h])
                    tev.record(pool[1 + h])
            tev.wait(main, pool[1])
            tev.wait(main, pool[2])
            if ev is not None:
                tev.record(ev[1])

        def compare(tev_factory):
            te = tev_factory()

            def per_step_us(fn, n=100):
                for i in range(10):
                    fn(i)
                torch.cuda.synchronize()
                e0, e1 = te.new(), te.new()
                te.record(e0)
                for i in range(n):
                    fn(i)
                te.record(e1)
                torch.cuda.synchronize()
                return te.ms(e0, e1) / n * 1e3

            def whole(i):
                qi, ki, vi, oi, S, z = sets[i % len(sets)]
                la.state_reduce(ki, vi, grid, S=S, z=z, ws=ws_all)
                la.apply(qi, S, z, grid, eps, out=oi)

            def two_on_one(i):
                group(0, i, ws_half[0])
                group(1, i, ws_half[0])

            out = {"compare_us": {"whole_batch_one_stream": per_step_us(whole),
                                  "two_groups_one_stream": per_step_us(two_on_one)}}
            te.close()
            return out

        return {
            "metric": METRIC + " (diagnostic: two streams)",
            "step": step, "tokens_per_step": B * N, "step_bytes": 4 * tb,
            "config": {"workload": name, "B": B, "H": H, "N": N, "d": d, "grid": list(grid), "eps": eps,
                       "streams": 2, "input_sets": len(sets)},
            # one group: the whole step across both streams (fork to join)
            "groups": [("step_two_streams", STATE_KERNELS + APPLY_KERNELS, 4 * tb)],
            "copy_pairs": [(s_[0], s_[3]) for s_ in sets],
            "extra": compare,
        }

    if name == "tc720p5s":
        spec = WORKLOADS["720p5s"]
        B, H, N, d, grid, eps = spec["B"], spec["H"], spec["N"], spec["d"], spec["grid"], spec["eps"]
        q, k, v = make_qkv_device(B, H, N, d, "bf16", spec["seed"], dev)
        tb = q.numel() * q.element_size()
        base = rotating((q, k, v), n_sets_for(4 * tb))
        sets = [(qi, ki, vi, torch.empty_like(q)) for (qi, ki, vi) in base]
        ws = la.workspace(B, H, N, d, dev)

        def step(i, ev, tev):
            qi, ki, vi, oi = sets[i % len(sets)]
            if ev is not None:
                tev.record(ev[0])
            la.token_causal(qi, ki, vi, grid, eps, out=oi, ws=ws)
            if ev is not None:
                tev.record(ev[1])

        return {
            "metric": "token-causal linear-attn tokens/sec and achieved HBM GB/s (% peak), 720p-5s shape, "
                      "1 GPU",
            "step": step, "tokens_per_step": B * N, "step_bytes": 4 * tb,
            "config": {"workload": name, "B": B, "H": H, "N": N, "d": d, "grid": list(grid), "eps": eps,
                       "input_sets": len(sets)},
            # one call: partial states, then the causal scan, each of whose workgroups
            # forms its chunk's prefix from them (K and V are read twice)
            "groups": [("token_causal", ("la_state_bf16_kernel", "la_causal_bf16_kernel"), 4 * tb)],
            "copy_pairs": [(s_[0], s_[3]) for s_ in sets],
        }

    if name == "720p60s":
        spec = WORKLOADS[name]
        B, H, N, d, grid, eps, L = (spec["B"], spec["H"], spec["N"], spec["d"], spec["grid"], spec["eps"],
                                    spec["block"])
        q, k, v = make_qkv_device(B, H, N, d, "bf16", spec["seed"], dev)
        blocks = [tuple(la.split_blocks(t, L)) for t in (q, k, v)]
        del q, k, v
        outs = [torch.empty_like(x) for x in blocks[0]]
        S = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)
        z = torch.zeros((B, H, d), dtype=torch.float32, device=dev)
        ws = la.workspace(B, H, N, d, dev)
        nb = len(blocks[0])
        blk_bytes = 4 * blocks[0][0].numel() * blocks[0][0].element_size()
        step_bytes = 4 * sum(x.numel() * x.element_size() for x in blocks[0])

        def step(i, ev, tev):
            # one step = the whole 60 s sequence, block after block from an empty cache
            S.zero_()
            z.zero_()
            if ev is not None:
                tev.record(ev[0])
            for b in range(nb):
                la.block_causal_step(blocks[0][b], blocks[1][b], blocks[2][b], S, z, N, grid, L, b, True,
                                     eps, out=outs[b], ws=ws)
            if ev is not None:
                tev.record(ev[1])

        return {
            "metric": "block-causal linear-attn tokens/sec and achieved HBM GB/s (% peak), 720p-60s, "
                      "10 blocks, 1 GPU",
            "step": step, "tokens_per_step": B * N, "step_bytes": step_bytes,
            "config": {"workload": name, "B": B, "H": H, "N": N, "d": d, "grid": list(grid), "block": L,
                       "eps": eps, "input_sets": 1},
            # one group = all block steps (state, combine and apply launches of the nb blocks)
            "groups": [("block_steps", STATE_KERNELS + APPLY_KERNELS, step_bytes, nb)],
            "copy_pairs": [(blocks[0][b], outs[b]) for b in range(nb)],
            "block_bytes": blk_bytes,
        }
    if name == "tconv720p":
        from linear_attention_video_02_amd.inputs import TCONV, make_tconv_device
        w = TCONV[name]
        B, T, P, D = w["B"], w["T"], w["P"], w["D"]
        X, W, cache, bias = make_tconv_device(B, T, P, D, w["seed"], dev)
        xb = X.numel() * X.element_size()
        wb = W.numel() * W.element_size()
        base = rotating((X, W, cache), n_sets_for(2 * xb + wb))
        sets = [(Xi, Wi, ci, torch.empty_like(X)) for (Xi, Wi, ci) in base]
        M = B * T * P
        flops = 2 * M * D * 3 * D  # the GEMM: M tokens x D outputs x 3D inputs

        def step(i, ev, tev):
            Xi, Wi, ci, Yi = sets[i % len(sets)]
            if ev is not None:
                tev.record(ev[0])
            # a denoising step of the block: reads the cache, leaves it (commit = 0)
            la.temporal_conv_step(Xi, Wi, ci, bias, commit=False, out=Yi)
            if ev is not None:
                tev.record(ev[1])

        def library_gemm(tev_factory):
            # context only: hipBLASLt (torch.matmul) on a plain GEMM of the same
            # shape, [M, 3D] x [3D, D], without the frame shifts, shortcut or bias
            A = torch.randn((M, 3 * D), device=dev).to(torch.bfloat16)
            Bm = torch.randn((3 * D, D), device=dev).to(torch.bfloat16)
            Cm = torch.empty((M, D), device=dev, dtype=torch.bfloat16)
            for _ in range(5):
                torch.matmul(A, Bm, out=Cm)
            torch.cuda.synchronize()
            te = tev_factory()
            e0, e1 = te.new(), te.new()
            n = 20
            te.record(e0)
            for _ in range(n):
                torch.matmul(A, Bm, out=Cm)
            te.record(e1)
            torch.cuda.synchronize()
            us = te.ms(e0, e1) / n * 1e3
            te.close()
            return {"library_gemm_same_shape": {"us": us, "tflops": flops / (us * 1e-6) / 1e12,
                                                "what": "torch.matmul bf16 [M,3D]x[3D,D] (hipBLASLt)"}}

        def cpu(budget):
            return cpu_baseline_tconv(X, W, cache, bias, w, budget)

        return {
            "metric": "temporal-conv (Mix-FFN, block-causal) tokens/sec and achieved TFLOP/s (% of bf16 "
                      "MFMA peak), one 720p-60s block at SANA-Video-2B width, 1 GPU",
            "step": step, "tokens_per_step": M, "step_bytes": 2 * xb + wb,
            "config": {"workload": name, "B": B, "T": T, "P": P, "D": D, "bias": True, "commit": 0,
                       "input_sets": len(sets)},
            "groups": [("tconv", ("la_tconv_bf16_kernel",), flops)],
            "roofline": {"bound": "mfma", "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "scale": 1e12},
            "copy_pairs": [(s_[0], s_[3]) for s_ in sets],
            "extra": library_gemm,
            "cpu_baseline": cpu,
        }
    raise SystemExit(f"unknown workload {name}")


if __name__ == "__main__":
    main()
