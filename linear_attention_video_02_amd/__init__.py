"""MI355X (gfx950) ReLU linear-attention token mixer.

Python binding of the C-ABI library liblinattn.so (declared in include/la.h).
This module only marshals arguments: every step of the computation runs in the
library's HIP kernels.  PyTorch supplies device memory and the stream.  There
is no fallback: if the library is not built, every call raises.

The method is the ReLU linear attention of the SANA-Video analysis page
(section 3.4: the linear-attention equation, Eq. 2 for RoPE, Eq. 3 and
Algorithm 1 for the block-causal cache), and beside it the block-causal
temporal convolution of the Mix-FFN (section 3.4, "Spatial-Temporal Mix-FFN"
and "Block Causal Mix-FFN": a kernel-3 convolution along time with a shortcut,
last-frame caching and zero padding) -- temporal_conv_step.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblinattn.so")

LA_FP32 = 0
LA_BF16 = 1

STATUS = {
    0: "LA_OK", -1: "LA_E_NULLPTR", -2: "LA_E_SHAPE", -3: "LA_E_UNSUPPORTED",
    -4: "LA_E_ALIGN", -5: "LA_E_WORKSPACE", -6: "LA_E_HIP", -7: "LA_E_ALIAS",
}

_lib = None


class LinAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({strerror(status)})"
        if status == -6 or (status == -5 and where == "la_state_reduce_noalloc"):
            msg += ": " + lib().la_last_hip_error().decode()
        super().__init__(msg)


def lib() -> ctypes.CDLL:
    """Load liblinattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        # PyTorch ships its own HIP/HSA runtime.  It must be the one in the
        # process before the library is loaded, or the library would bring in
        # the system runtime as a second, device-less instance.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, cf, cs = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        common = [ci] * 8 + [cf, ci]  # B H N d gt gh gw block_tokens, eps, dtype
        L.la_workspace_bytes.argtypes = [ci, ci, ci, ci]
        L.la_workspace_bytes.restype = cs
        L.la_workspace_bytes_grid.argtypes = [ci] * 7
        L.la_workspace_bytes_grid.restype = cs
        L.la_state_reduce.argtypes = [vp, vp, vp, vp, vp, vp, vp, cs] + common + [vp]
        L.la_state_reduce.restype = ci
        L.la_state_reduce_noalloc.argtypes = [vp, vp, vp, vp, vp, vp] + common + [vp]
        L.la_state_reduce_noalloc.restype = ci
        L.la_apply.argtypes = [vp, vp, vp, vp, vp, vp, vp, cs] + common + [vp]
        L.la_apply.restype = ci
        L.la_block_causal_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, cs] + common + [ci, ci, vp]
        L.la_block_causal_step.restype = ci
        L.la_cross_attention.argtypes = [vp, vp, vp, vp, vp, cs] + [ci] * 5 + [cf, ci, vp]
        L.la_cross_attention.restype = ci
        L.la_cross_workspace_bytes.argtypes = [ci] * 4
        L.la_cross_workspace_bytes.restype = cs
        L.la_token_causal.argtypes = [vp, vp, vp, vp, vp, vp, vp, cs] + [ci] * 8 + [cf, ci, vp]
        L.la_token_causal.restype = ci
        L.la_temporal_conv_step.argtypes = [vp, vp, vp, vp, vp] + [ci] * 6 + [vp]
        L.la_temporal_conv_step.restype = ci
        L.la_stream_copy.argtypes = [vp, vp, cs, vp]
        L.la_stream_copy.restype = ci
        L.la_strerror.argtypes = [ci]
        L.la_strerror.restype = ctypes.c_char_p
        L.la_last_hip_error.argtypes = []
        L.la_last_hip_error.restype = ctypes.c_char_p
        L.la_set_tuning.argtypes = [ctypes.c_char_p, ci]
        L.la_set_tuning.restype = ci
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().la_strerror(int(status)).decode()


def workspace_bytes(B: int, H: int, N: int, d: int, grid=None) -> int:
    if grid is None:
        return int(lib().la_workspace_bytes(B, H, N, d))
    return int(lib().la_workspace_bytes_grid(B, H, N, d, *_grid(grid)))


def set_tuning(name: str, value: int) -> None:
    """Set one of the library's tuning knobs (measurement only; value < 0 restores the default)."""
    rc = lib().la_set_tuning(name.encode(), int(value))
    if rc:
        raise LinAttnError(rc, f"la_set_tuning({name!r}, {value})")


@contextlib.contextmanager
def tuning(**knobs):
    """Run a block with tuning knobs set, restoring their defaults afterwards."""
    try:
        for name, value in knobs.items():
            set_tuning(name, value)
        yield
    finally:
        for name in knobs:
            lib().la_set_tuning(name.encode(), -1)


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _grid(grid):
    if grid is None:
        return 0, 0, 0
    gt, gh, gw = (int(x) for x in grid)
    return gt, gh, gw


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_qkv(*ts):
    """Q/K/V/O-like tensors: 4-D [B, H, n, d], contiguous, one dtype, on one GPU.

    Shapes are checked before placement, so a mis-sized tensor is reported as
    such (the library trusts the sizes it is given: an undersized buffer would
    be read or written out of bounds).
    """
    ref = ts[0]
    _check_dims(*ts)
    for t in ts:
        if t.dtype != ref.dtype:
            raise ValueError("Q/K/V/O must share one dtype")
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU")
        if t.device != ref.device:
            raise ValueError("Q/K/V/O must be on one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")


def _check_dims(*ts):
    for t in ts:
        if t.dim() != 4:
            raise ValueError(f"tensors must be 4-D [B, H, N, d], got shape {tuple(t.shape)}")


def _check_same_shape(what, *ts):
    _check_dims(*ts)
    shapes = [tuple(t.shape) for t in ts]
    if any(sh != shapes[0] for sh in shapes):
        raise ValueError(f"{what}: shapes must match, got {shapes}")


def _check_state(S, z, B, H, d, device, what):
    """S [B, H, d, d] and z [B, H, d]: contiguous float32 on the inputs' device."""
    torch = _torch()
    if tuple(S.shape) != (B, H, d, d):
        raise ValueError(f"{what}: S must have shape {(B, H, d, d)}, got {tuple(S.shape)}")
    if tuple(z.shape) != (B, H, d):
        raise ValueError(f"{what}: z must have shape {(B, H, d)}, got {tuple(z.shape)}")
    for t in (S, z):
        if t.dtype != torch.float32:
            raise ValueError(f"{what}: S and z must be float32")
        if not t.is_contiguous():
            raise ValueError(f"{what}: S and z must be contiguous")
        if t.device != device:
            raise ValueError(f"{what}: S and z must be on the inputs' device")


_ws_cache: dict = {}


def workspace(B: int, H: int, N: int, d: int, device, stream=None, grid=None):
    """A zero-filled workspace, cached per (device, stream, size).

    The library's calls keep per-head counters and partial states in their
    workspace, so two calls that may run at the same time must not share one:
    the cache hands each stream its own (stream = None: the device's current
    stream).
    """
    torch = _torch()
    nbytes = workspace_bytes(B, H, N, d, grid)
    if nbytes == 0:
        raise ValueError("invalid sizes for a workspace")
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    key = (dev.type, dev.index, int(stream.cuda_stream), nbytes)
    ws = _ws_cache.get(key)
    if ws is None:
        # zero-filled on the stream that will use it, so no other stream's work can race with the fill
        with torch.cuda.stream(stream):
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def _state_tensors(B, H, d, device):
    torch = _torch()
    return (torch.empty((B, H, d, d), dtype=torch.float32, device=device),
            torch.empty((B, H, d), dtype=torch.float32, device=device))


def state_reduce(k, v, grid=None, S=None, z=None, ws=None):
    """S = sum_j RoPE(relu K_j)^T V_j and z = sum_j relu K_j per (batch, head)."""
    _check_same_shape("state_reduce k/v", k, v)
    B, H, N, d = k.shape
    if (S is None) != (z is None):
        raise ValueError("state_reduce: give both S and z, or neither")
    if S is None:
        S, z = _state_tensors(B, H, d, k.device)
    _check_state(S, z, B, H, d, k.device, "state_reduce")
    _check_qkv(k, v)
    if ws is None:
        ws = workspace(B, H, N, d, k.device, grid=grid)
    gt, gh, gw = _grid(grid)
    rc = lib().la_state_reduce(None, _ptr(k), _ptr(v), None, _ptr(S), _ptr(z), _ptr(ws),
                               ws.numel(), B, H, N, d, gt, gh, gw, 0, 0.0,
                               _dtype_code(k), _stream(k))
    if rc:
        raise LinAttnError(rc, "la_state_reduce")
    return S, z


def state_reduce_noalloc(k, v, S, z, grid=None):
    """state_reduce into the caller's S and z through la_state_reduce_noalloc:
    no workspace, the library's static scratch instead (nothing is allocated)."""
    _check_same_shape("state_reduce_noalloc k/v", k, v)
    B, H, N, d = k.shape
    _check_state(S, z, B, H, d, k.device, "state_reduce_noalloc")
    _check_qkv(k, v)
    gt, gh, gw = _grid(grid)
    rc = lib().la_state_reduce_noalloc(None, _ptr(k), _ptr(v), None, _ptr(S), _ptr(z), B, H, N, d,
                                       gt, gh, gw, 0, 0.0, _dtype_code(k), _stream(k))
    if rc:
        raise LinAttnError(rc, "la_state_reduce_noalloc")
    return S, z


def apply(q, S, z, grid=None, eps=1e-6, out=None):
    """O_i = RoPE(relu Q_i) S / (relu Q_i . z + eps)."""
    torch = _torch()
    _check_dims(q)
    B, H, N, d = q.shape
    _check_state(S, z, B, H, d, q.device, "apply")
    if out is not None:
        _check_same_shape("apply q/out", q, out)
    _check_qkv(q)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    gt, gh, gw = _grid(grid)
    rc = lib().la_apply(_ptr(q), None, None, _ptr(out), _ptr(S), _ptr(z), None, 0,
                        B, H, N, d, gt, gh, gw, 0, float(eps), _dtype_code(q), _stream(q))
    if rc:
        raise LinAttnError(rc, "la_apply")
    return out


def bidirectional(q, k, v, grid=None, eps=1e-6, out=None, ws=None):
    """Bidirectional ReLU linear attention with (optional) 3D RoPE."""
    _check_same_shape("bidirectional q/k/v", q, k, v)
    if out is not None:
        _check_same_shape("bidirectional q/out", q, out)
    _check_qkv(q, k, v)
    S, z = state_reduce(k, v, grid, ws=ws)
    return apply(q, S, z, grid, eps, out)


def cross_attention(q, k, v, eps=1e-6, out=None, ws=None):
    """Linear cross-attention: q [B, H, N_q, d] over k, v [B, H, N_kv, d], no RoPE.

    One library call (la_cross_attention): one launch for bf16 at d = 64 with
    N_kv <= 512, otherwise the state pass over the N_kv keys/values and the
    apply pass over the N_q queries.  N_kv = 0 gives zeros.
    """
    torch = _torch()
    _check_dims(q, k, v)
    if k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("k and v must be [B, H, N_kv, d] with q's B, H and d")
    if out is not None:
        _check_same_shape("cross_attention q/out", q, out)
    _check_qkv(q, k, v)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = cross_workspace(B, H, Nkv, d, q.device)
    rc = lib().la_cross_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws), ws.numel(), B, H, Nq, Nkv, d,
                                  float(eps), _dtype_code(q), _stream(q))
    if rc:
        raise LinAttnError(rc, "la_cross_attention")
    return out


def cross_workspace(B, H, Nkv, d, device):
    """A zero-filled workspace for cross_attention over Nkv keys/values, cached like workspace()."""
    torch = _torch()
    nbytes = int(lib().la_cross_workspace_bytes(B, H, Nkv, d))
    if nbytes == 0:
        raise ValueError("invalid sizes for a workspace")
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    stream = torch.cuda.current_stream(dev)
    key = ("cross", dev.type, dev.index, int(stream.cuda_stream), nbytes)
    ws = _ws_cache.get(key)
    if ws is None:
        with torch.cuda.stream(stream):
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def block_causal_step(q, k, v, S_carry, z_carry, N, grid, block_tokens, block_idx,
                      commit=True, eps=1e-6, out=None, ws=None):
    """One block of block-causal mode; q/k/v/out hold only this block."""
    torch = _torch()
    _check_same_shape("block_causal_step q/k/v", q, k, v)
    B, H, Lb, d = q.shape
    N, block_tokens, block_idx = int(N), int(block_tokens), int(block_idx)
    if block_tokens < 1 or block_idx < 0 or block_idx * block_tokens >= N:
        raise ValueError(f"block {block_idx} of {block_tokens} tokens is not inside a sequence of {N}")
    want = min(block_tokens, N - block_idx * block_tokens)
    if Lb != want:
        raise ValueError(f"block {block_idx} holds {want} tokens, but q/k/v hold {Lb}")
    _check_state(S_carry, z_carry, B, H, d, q.device, "block_causal_step carry")
    if out is not None:
        _check_same_shape("block_causal_step q/out", q, out)
    _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    if ws is None:
        ws = workspace(B, H, N, d, q.device, grid=grid)
    gt, gh, gw = _grid(grid)
    rc = lib().la_block_causal_step(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S_carry),
                                    _ptr(z_carry), _ptr(ws), ws.numel(), B, H, N, d,
                                    gt, gh, gw, int(block_tokens), float(eps), _dtype_code(q),
                                    int(block_idx), int(bool(commit)), _stream(q))
    if rc:
        raise LinAttnError(rc, "la_block_causal_step")
    return out


def token_causal(q, k, v, grid=None, eps=1e-6, S_carry=None, z_carry=None, n_offset=0, out=None, ws=None):
    """Token-causal linear attention (Eq. 3): token i sees tokens j <= i.

    q, k, v: [B, H, N, d] bf16 or fp32, d in {32, 64, 112, 128}; token i sits at global position
    n_offset + i.  With S_carry/z_carry ([B, H, d, d] / [B, H, d] fp32) the
    scan starts from that state and leaves the final state in them.
    """
    torch = _torch()
    _check_same_shape("token_causal q/k/v", q, k, v)
    B, H, N, d = q.shape
    if (S_carry is None) != (z_carry is None):
        raise ValueError("token_causal: give both S_carry and z_carry, or neither")
    if S_carry is not None:
        _check_state(S_carry, z_carry, B, H, d, q.device, "token_causal carry")
    if out is not None:
        _check_same_shape("token_causal q/out", q, out)
    _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    if ws is None:
        ws = workspace(B, H, max(N, 1), d, q.device, grid=grid)
    gt, gh, gw = _grid(grid)
    rc = lib().la_token_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S_carry), _ptr(z_carry),
                               _ptr(ws), ws.numel(), B, H, N, d, gt, gh, gw, int(n_offset), float(eps),
                               _dtype_code(q), _stream(q))
    if rc:
        raise LinAttnError(rc, "la_token_causal")
    return out


def split_blocks(x, block_tokens):
    """Per-block contiguous copies [B, H, L_b, d] of a [B, H, N, d] tensor."""
    N = x.shape[2]
    return [x[:, :, b0:b0 + block_tokens].contiguous() for b0 in range(0, N, block_tokens)]


def block_causal(q_blocks, k_blocks, v_blocks, N, grid, block_tokens, eps=1e-6,
                 S_carry=None, z_carry=None, first_block=0):
    """Run blocks first_block, first_block+1, ... in order, committing each.

    q_blocks etc. are lists of per-block [B, H, L_b, d] tensors.  Returns the
    list of outputs and the carry (S, z) after the last block.
    """
    torch = _torch()
    q0 = q_blocks[0]
    B, H, _, d = q0.shape
    if S_carry is None:
        S_carry = torch.zeros((B, H, d, d), dtype=torch.float32, device=q0.device)
        z_carry = torch.zeros((B, H, d), dtype=torch.float32, device=q0.device)
    outs = []
    for i, (qb, kb, vb) in enumerate(zip(q_blocks, k_blocks, v_blocks)):
        outs.append(block_causal_step(qb, kb, vb, S_carry, z_carry, N, grid, block_tokens,
                                      first_block + i, True, eps))
    return outs, S_carry, z_carry


def temporal_conv_step(x, W, cache, bias=None, commit=True, out=None):
    """One block of the block-causal temporal convolution with shortcut.

    x: [B, T, P, D] bf16 (the block's frames; P spatial positions); W: [3, D, D]
    bf16 with W[k][out][in] the weight at time offset k - 1; cache: [B, P, D]
    bf16, the previous block's last frame (zeros before the first block);
    bias: [D] float32 or None.  Returns out = x + conv(x) (+ bias); with commit
    the cache then holds x[:, -1].
    """
    torch = _torch()
    for t in (x, W, cache):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("x, W and cache must be contiguous bf16 GPU tensors")
    if x.dim() != 4:
        raise ValueError("x must be [B, T, P, D]")
    B, T, P, D = x.shape
    if tuple(W.shape) != (3, D, D) or tuple(cache.shape) != (B, P, D):
        raise ValueError("W must be [3, D, D] and cache [B, P, D]")
    if bias is not None and (not bias.is_cuda or bias.dtype != torch.float32 or
                             tuple(bias.shape) != (D,) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [D] GPU tensor")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    rc = lib().la_temporal_conv_step(_ptr(x), _ptr(out), _ptr(W), _ptr(bias), _ptr(cache),
                                     B, T, P, D, int(bool(commit)), LA_BF16, _stream(x))
    if rc:
        raise LinAttnError(rc, "la_temporal_conv_step")
    return out


def stream_copy(src, dst):
    """Plain device copy src -> dst (same size, contiguous): the library's
    reference stream for the practical HBM ceiling (a measurement utility)."""
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous GPU tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    rc = lib().la_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(src))
    if rc:
        raise LinAttnError(rc, "la_stream_copy")
    return dst
