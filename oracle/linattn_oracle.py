"""fp64 CPU oracle for the ReLU linear-attention token mixer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP library: the two are connected
only through the seeded input arrays that a caller hands to both.

Source: "SANA-Video: Efficient Video Generation with Block Linear Diffusion
Transformer" (the paper-graph-ui analysis page of arXiv 2509.24695), section
"3.4 Detailed, Sentence-Based Technical Breakdown":

* "ReLU Linear Attention Mechanism", the unnumbered linear-attention equation:
  O_i = phi(Q_i) (sum_j phi(K_j)^T V_j) / phi(Q_i) (sum_j phi(K_j)^T), phi = ReLU.
* "Integration of 3D Rotary Position Embeddings (RoPE)", Eq. 2: the numerator
  rotates phi(Q_i) and phi(K_j) (RoPE after ReLU); the denominator rotates
  neither.
* "Block Linear Attention with Constant-Memory KV Cache", Eq. 3 and the update
  rule beside it (running sums of phi(K_j)^T V_j and phi(K_j)^T), Table 1
  (O(D^2) state), and Algorithm 1 (a block is denoised against the cache of
  all earlier blocks; the clean block is then folded into the cache).

Readings where the page is silent (each is a stated definition here):

* eps is added to the denominator only (default 1e-6); no 1/sqrt(d) scale.
* RoPE: P = d/2 interleaved pairs (2p, 2p+1).  The t axis takes the first
  P - 2*floor(P/3) pairs, h the next floor(P/3), w the last floor(P/3).  Pair
  k of an axis with P_a pairs turns by angle pos_a * 10000**(-k/P_a)
  (the RoFormer frequency schedule, per axis).  Positions are 0-based integer
  grid coordinates of token n in t-major order:
  t = n // (gh*gw), h = (n // gw) % gh, w = n % gw.
* Block-causal mode: token n belongs to block n // L; a block sees, in full,
  every token of its own block and of all earlier blocks; RoPE uses the
  token's global index n.
* A row whose phi(Q_i) is all zero has output exactly zero (the numerator is
  exactly zero; with eps = 0 the 0/0 is defined as 0).
* Any other row is the IEEE quotient num / den.  Its denominator is zero only
  when eps = 0 and z is zero on every channel where phi(Q_i) is positive (for
  instance cross-attention over no keys): the row is then NaN where the
  numerator is zero and +-inf elsewhere.  Non-finite inputs propagate.

Everything is evaluated in float64 on whatever values the caller passes
(bf16 inputs are passed as their exact float values).
"""
from __future__ import annotations

import numpy as np

ROPE_BASE = 10000.0


# ---------------------------------------------------------------------------
# kernel feature map and 3D rotary embedding
# ---------------------------------------------------------------------------

def phi(x: np.ndarray) -> np.ndarray:
    """ReLU feature map, element-wise ("ReLU Linear Attention Mechanism")."""
    return np.maximum(np.asarray(x, dtype=np.float64), 0.0)


def rope_axis_pairs(d: int) -> tuple[int, int, int]:
    """Number of rotation pairs given to the (t, h, w) axes for head dim d.

    The page says only that 3D RoPE rotates pairs of head dimensions to encode
    temporal and spatial position; the split used here is a stated reading.
    """
    if d % 2:
        raise ValueError("RoPE needs an even head dimension")
    p = d // 2
    ph = pw = p // 3
    return p - 2 * (p // 3), ph, pw


def grid_positions(n: np.ndarray, grid: tuple[int, int, int]):
    """0-based (t, h, w) coordinates of token indices n on a t-major grid."""
    gt, gh, gw = grid
    n = np.asarray(n, dtype=np.int64)
    return n // (gh * gw), (n // gw) % gh, n % gw


def rope_angles(n: np.ndarray, grid: tuple[int, int, int], d: int) -> np.ndarray:
    """Rotation angle of every pair for every token: array [len(n), d/2]."""
    pt, ph, pw = rope_axis_pairs(d)
    t, h, w = grid_positions(n, grid)
    ang = np.empty((len(t), d // 2), dtype=np.float64)
    start = 0
    for pos, npairs in ((t, pt), (h, ph), (w, pw)):
        k = np.arange(npairs, dtype=np.float64)
        omega = ROPE_BASE ** (-k / npairs)
        ang[:, start:start + npairs] = pos[:, None].astype(np.float64) * omega[None, :]
        start += npairs
    return ang


def rope(x: np.ndarray, n: np.ndarray, grid) -> np.ndarray:
    """Rotate each interleaved pair (x_2p, x_2p+1) of rows x[i] by its angle.

    x has shape [len(n), d].  grid=None means no positional encoding.
    """
    x = np.asarray(x, dtype=np.float64)
    if grid is None:
        return x.copy()
    ang = rope_angles(n, grid, x.shape[-1])
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[:, 0::2], x[:, 1::2]
    y = np.empty_like(x)
    y[:, 0::2] = x0 * c - x1 * s
    y[:, 1::2] = x0 * s + x1 * c
    return y


# ---------------------------------------------------------------------------
# one (batch, head) slice: state, apply, full forms
# ---------------------------------------------------------------------------

def state(K: np.ndarray, V: np.ndarray, grid, n0: int = 0):
    """Accumulators of one slice of tokens n0 .. n0+len(K)-1.

    S = sum_j RoPE(phi(K_j))^T V_j   (d x d, row = key channel, col = value channel)
    z = sum_j phi(K_j)               (d, un-rotated: Eq. 2 denominator)
    """
    K = phi(K)
    V = np.asarray(V, dtype=np.float64)
    n = np.arange(n0, n0 + K.shape[0])
    S = rope(K, n, grid).T @ V
    z = K.sum(axis=0)
    return S, z


def apply(Q: np.ndarray, S: np.ndarray, z: np.ndarray, grid, eps: float, n0: int = 0):
    """O_i = RoPE(phi(Q_i)) S / (phi(Q_i) z + eps) for tokens n0 .. n0+len(Q)-1 (Eq. 2)."""
    q = phi(Q)
    n = np.arange(n0, n0 + q.shape[0])
    num = rope(q, n, grid) @ S
    den = q @ z + eps
    out = np.zeros_like(num)
    live = np.any(q > 0.0, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        out[live] = num[live] / den[live, None]
    return out


def bidirectional_head(Q, K, V, grid, eps):
    """Bidirectional linear attention of one (batch, head) slice [N, d]."""
    S, z = state(K, V, grid)
    return apply(Q, S, z, grid, eps)


def block_causal_head(Q, K, V, grid, block_tokens: int, eps, carry=None):
    """Block-causal linear attention of one slice, carrying (S, z) across blocks.

    Follows Eq. 3's running sums taken a block at a time (Algorithm 1): before
    block b the carry holds the sums over blocks < b ("None" = zeros); block b
    adds its own tokens and then applies to its own rows.  Returns (O, S, z)
    with the final carry.
    """
    N, d = np.shape(Q)
    if carry is None:
        S = np.zeros((d, d))
        z = np.zeros(d)
    else:
        S, z = (np.array(c, dtype=np.float64) for c in carry)
    out = np.zeros((N, d))
    for b0 in range(0, N, block_tokens):
        b1 = min(b0 + block_tokens, N)
        Sb, zb = state(K[b0:b1], V[b0:b1], grid, n0=b0)
        S = S + Sb
        z = z + zb
        out[b0:b1] = apply(Q[b0:b1], S, z, grid, eps, n0=b0)
    return out, S, z


def token_causal_head(Q, K, V, grid, eps, n0: int = 0, carry=None):
    """Token-causal linear attention of one slice, Eq. 3 taken literally.

    Section 3.3.1 of the analysis page ("Derivation from causal linear
    attention"): token i sees tokens j <= i.  Before token i the two
    accumulators hold sum_{j<i} RoPE(phi K_j)^T V_j and sum_{j<i} phi(K_j);
    token i first adds its own state S_i and key, then reads them:
    O_i = RoPE(phi Q_i) S_acc / (phi(Q_i) z_acc + eps).  RoPE uses the global
    index n0 + i (the page omits it only for clarity).  `carry` = the
    accumulators before token 0 ("None" = zeros).  Returns (O, S, z) with the
    accumulators after the last token.
    """
    N, d = np.shape(Q)
    if carry is None:
        S = np.zeros((d, d))
        z = np.zeros(d)
    else:
        S, z = (np.array(c, dtype=np.float64) for c in carry)
    q = phi(Q)
    k = phi(K)
    V = np.asarray(V, dtype=np.float64)
    n = np.arange(n0, n0 + N)
    qr = rope(q, n, grid)
    kr = rope(k, n, grid)
    out = np.zeros((N, d))
    for i in range(N):
        S = S + np.outer(kr[i], V[i])
        z = z + k[i]
        if np.any(q[i] > 0.0):
            out[i] = (qr[i] @ S) / (q[i] @ z + eps)
    return out, S, z


def weights_form_head(Q, K, V, grid, eps, block_tokens: int | None = None):
    """O(N^2) form: explicit attention weights, no reassociation.

    O_i = sum_j (RoPE(phi Q_i) . RoPE(phi K_j)) V_j / (sum_j phi Q_i . phi K_j + eps),
    with j restricted to blocks <= block(i) in block-causal mode.  This is the
    kernel-attention reading of the same formula (the page: the weights are
    dot products phi(Q_i) . phi(K_j) instead of softmax scores).
    """
    q, k = phi(Q), phi(K)
    V = np.asarray(V, dtype=np.float64)
    n = np.arange(q.shape[0])
    num_w = rope(q, n, grid) @ rope(k, n, grid).T
    den_w = q @ k.T
    if block_tokens is not None:
        blk = n // block_tokens
        mask = blk[None, :] <= blk[:, None]
        num_w = num_w * mask
        den_w = den_w * mask
    num = num_w @ V
    den = den_w.sum(axis=1) + eps
    out = np.zeros_like(num)
    live = np.any(q > 0.0, axis=1)
    out[live] = num[live] / den[live, None]
    return out


def cross_attention_head(Q, K, V, eps):
    """Linear cross-attention of one slice: N_q queries over N_kv keys/values.

    The analysis page ("How SANA-Video Positions Itself", the architectural
    lens; and the Linear DiT block of section 3.4) replaces cross-attention by
    the same ReLU linear attention as self-attention.  Text tokens carry no
    (t, h, w) grid position, so no RoPE; N_kv is a free parameter (the page
    gives no text length).  N_kv = 0 gives S = 0, z = 0 and all-zero output.
    """
    d = np.shape(Q)[-1]
    if np.shape(K)[0] == 0:
        S, z = np.zeros((d, d)), np.zeros(d)
    else:
        S, z = state(K, V, None)
    return apply(Q, S, z, None, eps)


# ---------------------------------------------------------------------------
# whole [B, H, N, d] tensors
# ---------------------------------------------------------------------------

def bidirectional(Q, K, V, grid=None, eps=1e-6):
    """O[B,H,N,d] of bidirectional ReLU linear attention, per (batch, head)."""
    B, H, N, d = np.shape(Q)
    out = np.empty((B, H, N, d))
    for b in range(B):
        for h in range(H):
            out[b, h] = bidirectional_head(Q[b, h], K[b, h], V[b, h], grid, eps)
    return out


def block_causal(Q, K, V, grid, block_tokens, eps=1e-6):
    """O[B,H,N,d] of block-causal linear attention plus the final carry (S, z)."""
    B, H, N, d = np.shape(Q)
    out = np.empty((B, H, N, d))
    S = np.empty((B, H, d, d))
    z = np.empty((B, H, d))
    for b in range(B):
        for h in range(H):
            out[b, h], S[b, h], z[b, h] = block_causal_head(
                Q[b, h], K[b, h], V[b, h], grid, block_tokens, eps)
    return out, S, z


def cross_attention(Q, K, V, eps=1e-6):
    """O[B,H,N_q,d] of linear cross-attention with K, V of shape [B,H,N_kv,d]."""
    B, H, Nq, d = np.shape(Q)
    out = np.empty((B, H, Nq, d))
    for b in range(B):
        for h in range(H):
            out[b, h] = cross_attention_head(Q[b, h], K[b, h], V[b, h], eps)
    return out


def token_causal(Q, K, V, grid=None, eps=1e-6):
    """O[B,H,N,d] of token-causal linear attention plus the final accumulators."""
    B, H, N, d = np.shape(Q)
    out = np.empty((B, H, N, d))
    S = np.empty((B, H, d, d))
    z = np.empty((B, H, d))
    for b in range(B):
        for h in range(H):
            out[b, h], S[b, h], z[b, h] = token_causal_head(Q[b, h], K[b, h], V[b, h], grid, eps)
    return out, S, z


def rel_row_error(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over rows of ||got_i - ref_i||_inf / ||ref_i||_inf (last axis = row).

    A reference row that is exactly zero demands an exactly zero row: any
    non-zero there counts as infinite error.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.max(np.abs(got - ref), axis=-1)
    scale = np.max(np.abs(ref), axis=-1)
    zero = scale == 0.0
    if np.any(~np.isfinite(got)) or np.any(zero & (err != 0.0)):
        return float("inf")
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, scale))
    return float(ratio.max()) if ratio.size else 0.0
