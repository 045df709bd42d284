"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the attention arithmetic: it only draws Q, K, V,
rounds them to bf16 when asked, and scales a few columns to mimic activation
outliers.  Both the HIP library and the fp64 oracle are fed from it.

Workloads (latent token grids of the pages' video shapes; DCAE-V compresses
32x in space and 4x in time, a 60 s clip at 16 FPS has 240 latent frames):

  tiny    B1 H2  N256    d32  fp32, no RoPE
  480p    B1 H16 N8190   d64  bf16, grid 21x15x26, 1% of (head, channel) columns x8
  720p5s  B2 H32 N19320  d64  bf16, grid 21x23x40
  720p60s B1 H32 N220800 d64  bf16, grid 240x23x40, 10 blocks of 22080 tokens
  sweep   B1 H32 d in {32,64,128}, N in {4096,16384,65536,220800}, grid ceil(N/920)x23x40
  sana2b  B1 H20 N19320  d112 bf16, grid 21x23x40: SANA-Video-2B's real heads (20 x 112,
          width 2240) on the 720p-5s latent
  cross720p  B2 H32, 19320 video queries over 300 text keys/values, d64 bf16, no RoPE
             (the pages give no text length; 300 is a parameter)
  tconv720p  the Mix-FFN temporal convolution on one block of the 720p-60s clip:
             B1, 24 frames x 920 positions, width D = 2240 (SANA-Video-2B), bf16
"""
from __future__ import annotations

import math

import numpy as np

SWEEP_D = (32, 64, 128)
SWEEP_N = (4096, 16384, 65536, 220800)


def _workload(name, B, H, N, d, dtype, grid, seed, block=None, outliers=False, eps=1e-6):
    return dict(name=name, B=B, H=H, N=N, d=d, dtype=dtype, grid=grid, seed=seed,
                block=block, outliers=outliers, eps=eps)


def sweep_grid(N: int) -> tuple[int, int, int]:
    """Frames of a 23x40 latent plane needed to hold N tokens (last frame partial)."""
    return (math.ceil(N / 920), 23, 40)


WORKLOADS = {
    "tiny": _workload("tiny", 1, 2, 256, 32, "fp32", None, 1001),
    "480p": _workload("480p", 1, 16, 8190, 64, "bf16", (21, 15, 26), 1002, outliers=True),
    "720p5s": _workload("720p5s", 2, 32, 19320, 64, "bf16", (21, 23, 40), 1003),
    "720p60s": _workload("720p60s", 1, 32, 220800, 64, "bf16", (240, 23, 40), 1004,
                         block=22080),
}
WORKLOADS["sana2b"] = _workload("sana2b", 1, 20, 19320, 112, "bf16", (21, 23, 40), 1007)
for _d in SWEEP_D:
    for _n in SWEEP_N:
        WORKLOADS[f"sweep_d{_d}_n{_n}"] = _workload(
            f"sweep_d{_d}_n{_n}", 1, 32, _n, _d, "bf16", sweep_grid(_n), 1005)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    Operates on the bit pattern: add 0x7FFF plus the lowest kept bit, then clear
    the 16 low bits.  Inputs here are finite normal draws, so no NaN handling.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def make_qkv(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
             outliers: bool = False):
    """Draw Q, K, V ~ N(0, 1) of shape [B, H, N, d] as float32 arrays.

    Draw order is Q, K, V from numpy's PCG64 stream of `seed`.  For bf16 the
    values are rounded to bf16 (so they are exactly representable).  With
    `outliers`, for each of Q, K, V in turn, round(0.01 * H * d) distinct
    (head, channel) columns are multiplied by 8 (a power of two, so the bf16
    rounding is unaffected).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(3):
        a = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if dtype == "bf16":
            a = round_to_bf16(a)
        out.append(a)
    if outliers:
        ncols = int(round(0.01 * H * d))
        for a in out:
            cols = rng.choice(H * d, size=ncols, replace=False)
            for c in cols:
                a[:, c // d, :, c % d] *= np.float32(8.0)
    return tuple(out)


def make_workload(name: str):
    """Inputs of a named workload: (q, k, v, spec)."""
    w = WORKLOADS[name]
    q, k, v = make_qkv(w["B"], w["H"], w["N"], w["d"], w["dtype"], w["seed"], w["outliers"])
    return q, k, v, w


def make_qkv_device(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
                    device="cuda:0"):
    """Draw Q, K, V ~ N(0, 1) of shape [B, H, N, d] directly on a GPU.

    Uses torch's device generator seeded with `seed` (draw order Q, K, V) and
    rounds to bf16 with torch's round-to-nearest-even cast.  Used for the large
    workloads, where drawing gigabytes on the host would dominate run time;
    callers copy the heads they check back to the host for the oracle.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for _ in range(3):
        a = torch.randn((B, H, N, d), generator=gen, dtype=torch.float32, device=device)
        out.append(a.to(torch.bfloat16) if dtype == "bf16" else a)
        del a
    return tuple(out)


CROSS = {"cross720p": dict(name="cross720p", B=2, H=32, Nq=19320, Nkv=300, d=64, dtype="bf16",
                           seed=1006, eps=1e-6)}


def make_cross_device(B: int, H: int, Nq: int, Nkv: int, d: int, dtype: str = "bf16", seed: int = 0,
                      device="cuda:0"):
    """Q [B, H, Nq, d] and K, V [B, H, Nkv, d] ~ N(0, 1) drawn on a GPU (order Q, K, V)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for n in (Nq, Nkv, Nkv):
        a = torch.randn((B, H, n, d), generator=gen, dtype=torch.float32, device=device)
        out.append(a.to(torch.bfloat16) if dtype == "bf16" else a)
    return tuple(out)


def make_workload_device(name: str, device="cuda:0"):
    """Device tensors of a named workload: (q, k, v, spec).

    The two small workloads come from the numpy stream (make_qkv) and are
    uploaded; the large ones are drawn on the device (make_qkv_device).
    """
    import torch
    w = WORKLOADS[name]
    if w["name"] in ("tiny", "480p"):
        q, k, v = make_qkv(w["B"], w["H"], w["N"], w["d"], w["dtype"], w["seed"], w["outliers"])
        tdt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
        return tuple(torch.from_numpy(a).to(device=device, dtype=tdt) for a in (q, k, v)) + (w,)
    return make_qkv_device(w["B"], w["H"], w["N"], w["d"], w["dtype"], w["seed"], device) + (w,)


TCONV = {"tconv720p": dict(name="tconv720p", B=1, T=24, P=920, D=2240, seed=1008)}


def make_tconv(B: int, T: int, P: int, D: int, seed: int = 0, bias: bool = True):
    """Inputs of one temporal-convolution block as float32 arrays.

    Draw order from numpy's PCG64 stream of `seed`: X [B, T, P, D] ~ N(0, 1),
    W [3, D, D] ~ N(0, 1/(3D)) (unit-variance output), cache [B, P, D] ~ N(0, 1),
    then bias [D] ~ N(0, 0.01) if asked (else None).  X, W and the cache are
    rounded to bf16; the bias stays float32.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    X = round_to_bf16(rng.standard_normal((B, T, P, D), dtype=np.float32))
    W = round_to_bf16(rng.standard_normal((3, D, D), dtype=np.float32) * np.float32(1.0 / math.sqrt(3 * D)))
    cache = round_to_bf16(rng.standard_normal((B, P, D), dtype=np.float32))
    b = (rng.standard_normal(D, dtype=np.float32) * np.float32(0.1)) if bias else None
    return X, W, cache, b


def make_tconv_device(B: int, T: int, P: int, D: int, seed: int = 0, device="cuda:0"):
    """X, W, cache and bias of the same distributions as make_tconv, drawn on a GPU.

    torch's device generator seeded with `seed`, draw order X, W, cache, bias;
    X, W and the cache in bf16 by torch's round-to-nearest-even cast, the bias
    float32.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    X = torch.randn((B, T, P, D), generator=gen, device=device).to(torch.bfloat16)
    W = (torch.randn((3, D, D), generator=gen, device=device) / math.sqrt(3 * D)).to(torch.bfloat16)
    cache = torch.randn((B, P, D), generator=gen, device=device).to(torch.bfloat16)
    bias = torch.randn(D, generator=gen, device=device) * 0.1
    return X, W, cache, bias
