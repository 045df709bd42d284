"""Argument checks of the Python binding that need no GPU.

The C library trusts the sizes it is handed (B, H, N, d come from q or k), so
the binding must reject tensors whose shapes disagree before any call: an
undersized output, key, state or carry would otherwise be read or written out
of bounds.  Every case below fails a shape or dtype check, which the binding
runs before it looks at where the tensors live, so CPU tensors suffice.
"""
import pytest
import torch

import linear_attention_video_02_amd as la

B, H, N, d = 1, 2, 16, 64


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def state(b=B, h=H, dd=d, dtype=torch.float32):
    return t(b, h, dd, dd, dtype=dtype), t(b, h, dd, dtype=dtype)


def test_state_reduce_shapes():
    k = t(B, H, N, d)
    with pytest.raises(ValueError, match="shapes must match"):
        la.state_reduce(k, t(B, H, N - 1, d))
    S, z = state()
    with pytest.raises(ValueError, match="S must have shape"):
        la.state_reduce(k, k, S=t(B, H, d, d - 1, dtype=torch.float32), z=z)
    with pytest.raises(ValueError, match="z must have shape"):
        la.state_reduce(k, k, S=S, z=t(B, H + 1, d, dtype=torch.float32))
    with pytest.raises(ValueError, match="float32"):
        la.state_reduce(k, k, S=S.double(), z=z.double())
    with pytest.raises(ValueError, match="both S and z"):
        la.state_reduce(k, k, S=S)
    with pytest.raises(ValueError, match="4-D"):
        la.state_reduce(t(H, N, d), t(H, N, d))


def test_apply_shapes():
    q = t(B, H, N, d)
    S, z = state()
    with pytest.raises(ValueError, match="shapes must match"):
        la.apply(q, S, z, out=t(B, H, N - 8, d))
    with pytest.raises(ValueError, match="S must have shape"):
        la.apply(q, *state(dd=32))
    with pytest.raises(ValueError, match="contiguous"):
        la.apply(q, S.transpose(2, 3), z)
    with pytest.raises(ValueError, match="float32"):
        la.apply(q, S.bfloat16(), z)


def test_bidirectional_and_cross_shapes():
    q = t(B, H, N, d)
    with pytest.raises(ValueError, match="shapes must match"):
        la.bidirectional(q, t(B, H, N + 1, d), t(B, H, N + 1, d))
    with pytest.raises(ValueError, match="shapes must match"):
        la.bidirectional(q, q, t(B, H, N, 32))
    with pytest.raises(ValueError, match="shapes must match"):
        la.bidirectional(q, q, q, out=t(B, H, N, d - 8))
    with pytest.raises(ValueError, match="N_kv"):
        la.cross_attention(q, t(B, H, 7, d), t(B, H, 8, d))
    with pytest.raises(ValueError, match="N_kv"):
        la.cross_attention(q, t(B, H + 1, 7, d), t(B, H + 1, 7, d))
    with pytest.raises(ValueError, match="shapes must match"):
        la.cross_attention(q, t(B, H, 7, d), t(B, H, 7, d), out=t(B, H, 7, d))


def test_block_causal_step_shapes():
    Nseq, L = 1000, 300
    S, z = state()
    qb = t(B, H, L, d)
    last = t(B, H, Nseq - 3 * L, d)
    # the last block of 1000 tokens in blocks of 300 holds 100 tokens
    with pytest.raises(ValueError, match="holds 100 tokens"):
        la.block_causal_step(qb, qb, qb, S, z, Nseq, (10, 10, 10), L, 3)
    with pytest.raises(ValueError, match="holds 300 tokens"):
        la.block_causal_step(last, last, last, S, z, Nseq, (10, 10, 10), L, 0)
    with pytest.raises(ValueError, match="not inside"):
        la.block_causal_step(qb, qb, qb, S, z, Nseq, (10, 10, 10), L, 4)
    with pytest.raises(ValueError, match="not inside"):
        la.block_causal_step(qb, qb, qb, S, z, Nseq, (10, 10, 10), 0, 0)
    with pytest.raises(ValueError, match="shapes must match"):
        la.block_causal_step(qb, qb, last, S, z, Nseq, (10, 10, 10), L, 0)
    with pytest.raises(ValueError, match="S must have shape"):
        la.block_causal_step(qb, qb, qb, *state(h=1), Nseq, (10, 10, 10), L, 0)
    with pytest.raises(ValueError, match="shapes must match"):
        la.block_causal_step(qb, qb, qb, S, z, Nseq, (10, 10, 10), L, 0, out=last)


def test_token_causal_shapes():
    q = t(B, H, N, d)
    S, z = state()
    with pytest.raises(ValueError, match="shapes must match"):
        la.token_causal(q, q, t(B, H, N, d + 64))
    with pytest.raises(ValueError, match="both S_carry and z_carry"):
        la.token_causal(q, q, q, S_carry=S)
    with pytest.raises(ValueError, match="z must have shape"):
        la.token_causal(q, q, q, S_carry=S, z_carry=t(B, H, d + 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="shapes must match"):
        la.token_causal(q, q, q, out=t(B, H, N - 1, d))


def test_well_formed_cpu_tensors_are_refused_for_placement():
    q = t(B, H, N, d)
    S, z = state()
    with pytest.raises(ValueError, match="GPU"):
        la.apply(q, S, z)
    with pytest.raises(ValueError, match="GPU"):
        la.bidirectional(q, q, q)
