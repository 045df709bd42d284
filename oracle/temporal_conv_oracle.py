"""fp64 CPU oracle for the block-causal temporal convolution of the Mix-FFN.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library.

Source: the SANA-Video analysis page (arXiv 2509.24695), section "3.4 Detailed,
Sentence-Based Technical Breakdown":

* "Spatial-Temporal Mix-FFN": a 1D convolution of kernel size 3 along the time
  axis (3 x 1 x 1 on the [T, H, W, D] activations) is added to its own input
  through a shortcut: out = x + TemporalConv(x).
* "Block Causal Mix-FFN" (Figure 4(b)): in block-wise generation the frame
  before a block comes from a cache holding the last frame of the previous
  block ("last-frame caching"), and the frame after a block's last frame is an
  all-zero token ("zero padding"), so no block sees a later block.  The cache
  is the third entry of the KV cache [sum S, sum phi(K), conv cache] that
  Algorithm 1 starts as [None, None, None] and updates after the clean block.

Readings where the page is silent (each is a stated definition here):

* The convolution mixes channels: out[f] = x[f] + W_0 x[f-1] + W_1 x[f] +
  W_2 x[f+1] (+ bias), each W_k a D x D matrix (row = output channel).  The
  page calls the spatial 3x3 convolution depthwise but not this one, and three
  D x D matrices per block match the parameter count it gives for the 2B model.
* An empty cache (None) is a zero frame.
* The cache after a block is that block's last input frame x[T_b - 1].
* Activations are token-major [T_b, H*W, D] per batch element (frame-major
  tokens, as the attention's t-major token order); the convolution acts on
  the frame index only, each spatial position separately.

Everything is evaluated in float64 on whatever values the caller passes.
"""
from __future__ import annotations

import numpy as np


def temporal_conv_block(X: np.ndarray, W: np.ndarray, cache=None, bias=None):
    """One block of the block-causal temporal convolution with shortcut.

    X: [T_b, P, D] (frames, spatial positions, channels); W: [3, D, D] with
    W[k][o][i] the weight of input channel i at time offset k - 1 for output
    channel o; cache: [P, D] (the previous block's last frame) or None (zero
    frame); bias: [D] or None.  Returns (Y, new_cache) with Y = X +
    conv(X) and new_cache = X[-1].
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    T, P, D = X.shape
    prev = np.zeros((P, D)) if cache is None else np.asarray(cache, dtype=np.float64)
    # frames -1 .. T: the cached frame, the block, the zero padding frame
    padded = np.concatenate([prev[None], X, np.zeros((1, P, D))], axis=0)
    Y = X.copy()
    for f in range(T):
        for k in range(3):
            Y[f] += padded[f + k] @ W[k].T
    if bias is not None:
        Y += np.asarray(bias, dtype=np.float64)
    return Y, X[-1].copy()


def temporal_conv(X: np.ndarray, W: np.ndarray, cache=None, bias=None):
    """Batched temporal_conv_block: X [B, T_b, P, D], cache [B, P, D] or None."""
    X = np.asarray(X, dtype=np.float64)
    B = X.shape[0]
    Y = np.empty_like(X)
    new = np.empty((B,) + X.shape[2:])
    for b in range(B):
        Y[b], new[b] = temporal_conv_block(X[b], W, None if cache is None else cache[b], bias)
    return Y, new


def temporal_conv_blocks(X: np.ndarray, W: np.ndarray, block_frames: int, bias=None):
    """A whole sequence [T, P, D] in blocks of `block_frames` frames, each block
    taking the cache left by the previous one (Algorithm 1's order)."""
    X = np.asarray(X, dtype=np.float64)
    outs, cache = [], None
    for f0 in range(0, X.shape[0], block_frames):
        Y, cache = temporal_conv_block(X[f0:f0 + block_frames], W, cache, bias)
        outs.append(Y)
    return np.concatenate(outs, axis=0), cache
