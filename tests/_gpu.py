"""Helpers shared by the GPU tests (device transfer, oracle comparison)."""
import numpy as np

import oracle

TOL = {"bf16": 2e-2, "fp32": 1e-5}


def say(msg):
    print(msg, flush=True)


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def upload(a, dtype, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=torch_dtype(dtype))


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def row_err(got, ref):
    return oracle.rel_row_error(got, ref)


def state_err(S_got, S_ref):
    """Row-normalised error of a state matrix (rows = key channels)."""
    return oracle.rel_row_error(S_got, S_ref)


def assert_close(got, ref, dtype, what=""):
    e = row_err(got, ref)
    say(f"  {what}: max row-normalised rel err {e:.3e} (tol {TOL[dtype]:.0e})")
    assert e <= TOL[dtype], (what, e)
    return e
