"""Pins of the block-causal temporal-convolution oracle (CPU).

The oracle (oracle/temporal_conv_oracle.py) follows the SANA-Video analysis
page, section 3.4, "Spatial-Temporal Mix-FFN" (out = x + TemporalConv(x),
kernel 3 along time) and "Block Causal Mix-FFN" (last-frame cache before a
block, zero padding after it).  Pinned here by:

* hand-worked values (tests/golden/temporal_conv_worked.txt);
* an explicit scalar-loop brute force of the convolution sum;
* zero weights = identity (the zero-initialised shortcut the page describes);
* unit shift kernels fixing the time direction, the cache and the padding;
* an independent whole-sequence formulation with block-masked shift matrices;
* linearity in (x, cache);
* planted mistakes (reversed time offsets, no block padding, cache ignored,
  transposed weights, no shortcut), each of which must fail some pin.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import temporal_conv_oracle as tco

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "temporal_conv_worked.txt")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _case(seed, T=4, P=3, D=5):
    r = _rng(seed)
    return (r.standard_normal((T, P, D)), r.standard_normal((3, D, D)), r.standard_normal((P, D)),
            r.standard_normal(D))


def brute(X, W, cache, bias):
    """The convolution sum with scalar loops and explicit boundary cases."""
    T, P, D = X.shape
    Y = np.zeros_like(X)
    for f in range(T):
        for p in range(P):
            for o in range(D):
                s = X[f, p, o] + (0.0 if bias is None else bias[o])
                for k in range(3):
                    g = f + k - 1
                    for i in range(D):
                        if g < 0:
                            xi = 0.0 if cache is None else cache[p, i]
                        elif g >= T:
                            xi = 0.0
                        else:
                            xi = X[g, p, i]
                        s += W[k, o, i] * xi
                Y[f, p, o] = s
    return Y


def masked_sequence(X, W, L, bias=None):
    """Whole sequence [T, P, D] in blocks of L frames as one linear map: frame g
    feeds frame f through W_k when g = f + k - 1, except g = f + 1 across a
    block boundary (the padding); the previous block's last frame is visible."""
    T = X.shape[0]
    Y = X.copy()
    for k in range(3):
        M = np.zeros((T, T))
        for f in range(T):
            g = f + k - 1
            if 0 <= g < T and not (k == 2 and g // L != f // L):
                M[f, g] = 1.0
        Y += np.einsum("fg,gpi,oi->fpo", M, X, W[k])
    if bias is not None:
        Y += bias
    return Y


def test_golden_worked_examples():
    n = 0
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        name, dims, cache, x, w, y, newc = (s.split() for s in line.split("|"))
        T, P, D = map(int, dims)
        X = np.array(x, float).reshape(T, P, D)
        W = np.array(w, float).reshape(3, D, D)
        c = np.array(cache, float).reshape(P, D)
        Y, nc = tco.temporal_conv_block(X, W, c)
        np.testing.assert_allclose(Y.ravel(), np.array(y, float), rtol=0, atol=1e-12, err_msg=name[0])
        np.testing.assert_allclose(nc.ravel(), np.array(newc, float), rtol=0, atol=0, err_msg=name[0])
        n += 1
    assert n == 2


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("with_cache,with_bias", [(True, True), (False, False), (True, False)])
def test_brute_force(seed, with_cache, with_bias):
    X, W, c, b = _case(seed)
    c = c if with_cache else None
    b = b if with_bias else None
    Y, nc = tco.temporal_conv_block(X, W, c, b)
    np.testing.assert_allclose(Y, brute(X, W, c, b), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(nc, X[-1])


def test_zero_weights_are_identity():
    X, W, c, b = _case(4)
    Y, _ = tco.temporal_conv_block(X, np.zeros_like(W), c)
    np.testing.assert_array_equal(Y, X)


def test_unit_shift_kernels():
    X, _, c, _ = _case(5)
    D = X.shape[2]
    I = np.eye(D)
    Z = np.zeros((D, D))
    Y, _ = tco.temporal_conv_block(X, np.stack([I, Z, Z]), c)      # previous frame
    np.testing.assert_allclose(Y[0], X[0] + c, atol=1e-12)
    np.testing.assert_allclose(Y[1:], X[1:] + X[:-1], atol=1e-12)
    Y, _ = tco.temporal_conv_block(X, np.stack([Z, Z, I]), c)      # next frame, zero padding
    np.testing.assert_allclose(Y[:-1], X[:-1] + X[1:], atol=1e-12)
    np.testing.assert_allclose(Y[-1], X[-1], atol=1e-12)
    Y, _ = tco.temporal_conv_block(X, np.stack([Z, I, Z]), c)      # same frame
    np.testing.assert_allclose(Y, 2 * X, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 3, 7])
def test_blocks_equal_masked_sequence(L):
    r = _rng(6)
    X = r.standard_normal((7, 3, 4))
    W = r.standard_normal((3, 4, 4))
    b = r.standard_normal(4)
    Y, cache = tco.temporal_conv_blocks(X, W, L, b)
    np.testing.assert_allclose(Y, masked_sequence(X, W, L, b), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(cache, X[-1])


def test_linear_in_input_and_cache():
    X1, W, c1, _ = _case(7)
    X2, _, c2, _ = _case(8)
    a, s = 0.75, -1.5
    Y, _ = tco.temporal_conv_block(a * X1 + s * X2, W, a * c1 + s * c2)
    Y1, _ = tco.temporal_conv_block(X1, W, c1)
    Y2, _ = tco.temporal_conv_block(X2, W, c2)
    np.testing.assert_allclose(Y, a * Y1 + s * Y2, rtol=1e-12, atol=1e-12)


def test_batched_matches_blocks():
    r = _rng(9)
    X = r.standard_normal((2, 3, 4, 5))
    W = r.standard_normal((3, 5, 5))
    c = r.standard_normal((2, 4, 5))
    Y, nc = oracle.temporal_conv(X, W, c)
    for bb in range(2):
        Yb, ncb = tco.temporal_conv_block(X[bb], W, c[bb])
        np.testing.assert_array_equal(Y[bb], Yb)
        np.testing.assert_array_equal(nc[bb], ncb)


# -- planted mistakes: each variant must fail at least one pin ---------------

def _variant(kind):
    def f(X, W, cache=None, bias=None):
        X = np.asarray(X, float)
        T, P, D = X.shape
        prev = np.zeros((P, D)) if cache is None or kind == "no_cache" else np.asarray(cache, float)
        padded = np.concatenate([prev[None], X, np.zeros((1, P, D))], axis=0)
        Y = np.zeros_like(X) if kind == "no_shortcut" else X.copy()
        for fr in range(T):
            for k in range(3):
                kk = 2 - k if kind == "reversed" else k
                Wk = W[kk].T if kind == "transposed" else W[kk]
                Y[fr] += padded[fr + k] @ Wk.T
        if bias is not None:
            Y += bias
        return Y, X[-1].copy()
    return f


def _pins_pass(block_fn):
    X, W, c, b = _case(11)
    if not np.allclose(block_fn(X, W, c, b)[0], brute(X, W, c, b), atol=1e-9):
        return False
    D = X.shape[2]
    I, Z = np.eye(D), np.zeros((D, D))
    Y, _ = block_fn(X, np.stack([I, Z, Z]), c)
    return np.allclose(Y[0], X[0] + c) and np.allclose(Y[1:], X[1:] + X[:-1])


def _masked_pin_passes(block_fn, L=2):
    r = _rng(12)
    X = r.standard_normal((5, 2, 3))
    W = r.standard_normal((3, 3, 3))
    outs, cache = [], None
    for f0 in range(0, 5, L):
        Y, cache = block_fn(X[f0:f0 + L], W, cache)
        outs.append(Y)
    return np.allclose(np.concatenate(outs), masked_sequence(X, W, L))


def no_padding_blocks(X, W, L):
    """Plausible mistake: blocks see the next block's first frame (no zero padding)."""
    T = X.shape[0]
    Y = X.copy()
    prev = np.zeros_like(X[0])
    padded = np.concatenate([prev[None], X, np.zeros_like(X[:1])], axis=0)
    for f in range(T):
        for k in range(3):
            Y[f] += padded[f + k] @ W[k].T
    return Y


@pytest.mark.parametrize("kind", ["reversed", "no_cache", "transposed", "no_shortcut"])
def test_planted_mistakes_fail(kind):
    fn = _variant(kind)
    assert not (_pins_pass(fn) and _masked_pin_passes(fn)), kind
    assert _pins_pass(tco.temporal_conv_block) and _masked_pin_passes(tco.temporal_conv_block)


def test_planted_no_padding_fails():
    r = _rng(13)
    X = r.standard_normal((6, 2, 3))
    W = r.standard_normal((3, 3, 3))
    assert not np.allclose(no_padding_blocks(X, W, 2), masked_sequence(X, W, 2))
    assert np.allclose(tco.temporal_conv_blocks(X, W, 2)[0], masked_sequence(X, W, 2))
