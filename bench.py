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
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "linear-attn tokens/sec and achieved HBM GB/s (% peak), 720p-5s shape, 1 GPU"
HBM_PEAK_GBPS = 8000.0
WORKLOAD = "720p5s"
SRC_FILES = ["la_common.h", "la_state.h", "la_apply.h", "la_api.hip"]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in SRC_FILES:
        with open(os.path.join(ROOT, "linear_attention_video_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None.

    The summary records the kernel-source hash it was taken with; if the
    kernels changed since, the counters no longer describe them.
    """
    path = os.path.join(ROOT, "profiles", "traffic_720p5s.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("src_hash") != src_hash or kernel not in t.get("kernels", {}):
        return None
    return t["kernels"][kernel].get("hbm_bytes_per_launch")


def cpu_baseline(q, k, v, spec, budget_s=12.0):
    """Time the fp64 oracle on whole (batch, head) slices until ~budget_s."""
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
    for (b, h) in order:
        qh = q[b, h].float().cpu().numpy().astype(np.float64)
        kh = k[b, h].float().cpu().numpy().astype(np.float64)
        vh = v[b, h].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        S, z = oracle.state(kh, vh, grid)
        oracle.apply(qh, S, z, grid, eps)
        t_used += time.perf_counter() - t0
        slices += 1
        if t_used >= budget_s:
            break
    tokens = slices * N / H  # a token is one grid position across all H heads
    return {
        "value": tokens / t_used,
        "unit": "tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{slices} of {B * H} (batch, head) slices of the {WORKLOAD} workload, "
                  f"all {N} tokens each, fp64 numpy, {t_used:.1f} s "
                  f"({len(os.sched_getaffinity(0))} host cores visible)",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); "
              "the path shards by head or by sequence, see the design notes", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_video_02_amd as la
    from linear_attention_video_02_amd.inputs import WORKLOADS, make_qkv_device

    if not os.path.exists(la.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    spec = WORKLOADS[WORKLOAD]
    B, H, N, d, grid, eps = spec["B"], spec["H"], spec["N"], spec["d"], spec["grid"], spec["eps"]
    dev = torch.device("cuda:0")
    q, k, v = make_qkv_device(B, H, N, d, "bf16", spec["seed"], dev)
    tensor_bytes = q.numel() * q.element_size()
    set_bytes = 4 * tensor_bytes
    n_sets = max(2, math.ceil(2 * 2**30 / set_bytes))
    sets = []
    for i in range(n_sets):
        qi, ki, vi = (q, k, v) if i == 0 else (q.clone(), k.clone(), v.clone())
        S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
        z = torch.empty((B, H, d), dtype=torch.float32, device=dev)
        sets.append((qi, ki, vi, torch.empty_like(q), S, z))
    ws = la.workspace(B, H, N, d, dev)

    def step(i, ev=None):
        qi, ki, vi, oi, S, z = sets[i % n_sets]
        if ev is not None:
            ev[0].record()
        la.state_reduce(ki, vi, grid, S=S, z=z, ws=ws)
        if ev is not None:
            ev[1].record()
        la.apply(qi, S, z, grid, eps, out=oi)
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    state_ms = [e[0].elapsed_time(e[1]) for e in evs]
    apply_ms = [e[1].elapsed_time(e[2]) for e in evs]
    st_avg = sum(state_ms) / len(state_ms)
    ap_avg = sum(apply_ms) / len(apply_ms)

    # algorithmic bytes per launch: K + V read (state), Q read + O write (apply)
    kv_bytes = 2 * tensor_bytes
    qo_bytes = 2 * tensor_bytes
    dominant = ("la_state_bf16_kernel", st_avg, kv_bytes) if st_avg >= ap_avg else \
        ("la_apply_bf16_kernel", ap_avg, qo_bytes)
    name, dur_ms, nbytes = dominant
    achieved = nbytes / (dur_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    tokens_per_s = B * N / (ms_step * 1e-3)

    # a plain device copy of the same size, as the practical HBM ceiling
    src = torch.empty(2 * tensor_bytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(20):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 2 / (c0.elapsed_time(c1) / 20 * 1e-3) / 1e9
    del src, dst

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "H": H, "N": N, "d": d, "grid": list(grid),
                   "eps": eps, "input_sets": n_sets},
        "roofline": {
            "bound": "hbm",
            "kernel": name,
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": load_traffic(name, src_hash),
        },
        "step_GBps": 4 * tensor_bytes / (ms_step * 1e-3) / 1e9,
        "step_frac_of_peak": 4 * tensor_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "kernels_us": {"state": st_avg * 1e3, "apply": ap_avg * 1e3},
        "copy_GBps": copy_gbps,
        "wall_s": wall,
        "src_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(q, k, v, spec, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
