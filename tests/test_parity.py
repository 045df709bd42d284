"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance (max over rows of ||got_i - ref_i||_inf / ||ref_i||_inf): 2e-2 for
bf16 inputs, 1e-5 for fp32 inputs; an all-zero reference row needs an exact
zero row.  Workloads: the five latent shapes (tiny, 480p, 720p-5s, 720p-60s
block-causal, the d/N sweep) at full size -- every head for the small ones,
sampled heads (all rows) for the large ones -- plus ragged/odd fuzz shapes.
"""
import numpy as np
import pytest

import oracle
from _gpu import TOL, assert_close, host, say, state_err, upload
from linear_attention_video_02_amd.inputs import (SWEEP_D, SWEEP_N, WORKLOADS, make_qkv,
                                                  make_workload_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    import linear_attention_video_02_amd as m
    m.lib()
    return m


def _oracle_heads(q, k, v, heads, grid, eps):
    out, S, z = [], [], []
    for (b, h) in heads:
        Sh, zh = oracle.state(k[b, h], v[b, h], grid)
        out.append(oracle.apply(q[b, h], Sh, zh, grid, eps))
        S.append(Sh)
        z.append(zh)
    return out, S, z


def _check_bidirectional(la, name, heads=None):
    import torch
    tq, tk, tv, w = make_workload_device(name)
    B, H, N, d, grid, eps, dt = w["B"], w["H"], w["N"], w["d"], w["grid"], w["eps"], w["dtype"]
    say(f"[{name}] B={B} H={H} N={N} d={d} grid={grid} {dt}")
    S, z = la.state_reduce(tk, tv, grid)
    out = la.apply(tq, S, z, grid, eps)
    torch.cuda.synchronize()
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    sel = lambda t: np.stack([host(t[b, h]) for (b, h) in heads])  # noqa: E731
    q, k, v = sel(tq)[:, None], sel(tk)[:, None], sel(tv)[:, None]
    ref_o, ref_S, ref_z = _oracle_heads(q, k, v, [(i, 0) for i in range(len(heads))], grid, eps)
    got_o = sel(out)
    got_S = np.stack([host(S[b, h]) for (b, h) in heads])
    got_z = np.stack([host(z[b, h]) for (b, h) in heads])
    assert_close(got_o, np.stack(ref_o), dt, f"{name} O ({len(heads)} heads)")
    es = state_err(got_S, np.stack(ref_S))
    say(f"  {name} S: {es:.3e}")
    assert es <= TOL[dt]
    np.testing.assert_allclose(got_z, np.stack(ref_z), rtol=1e-4, atol=1e-4)


def test_tiny_fp32(la):
    _check_bidirectional(la, "tiny")


def test_tiny_fp32_against_weights_form(la):
    """The tiny workload also against the O(N^2) explicit-weights form."""
    import torch
    tq, tk, tv, w = make_workload_device("tiny")
    out = la.bidirectional(tq, tk, tv, None, w["eps"])
    torch.cuda.synchronize()
    got = host(out)
    for h in range(w["H"]):
        ref = oracle.weights_form_head(host(tq[0, h]), host(tk[0, h]), host(tv[0, h]), None, w["eps"])
        assert_close(got[0, h], ref, "fp32", f"tiny head {h} vs O(N^2)")


def test_480p(la):
    _check_bidirectional(la, "480p")


def test_720p5s(la):
    _check_bidirectional(la, "720p5s")


def test_sana2b_d112(la):
    """SANA-Video-2B's heads (H = 20, d = 112) on the 720p-5s latent, every head."""
    _check_bidirectional(la, "sana2b")


@pytest.mark.parametrize("d", SWEEP_D)
@pytest.mark.parametrize("N", SWEEP_N)
def test_sweep(la, d, N):
    _check_bidirectional(la, f"sweep_d{d}_n{N}", heads=[(0, 0), (0, 19), (0, 31)])


def test_720p60s_block_causal(la):
    import torch
    tq, tk, tv, w = make_workload_device("720p60s")
    B, H, N, d, grid, L, eps = w["B"], w["H"], w["N"], w["d"], w["grid"], w["block"], w["eps"]
    say(f"[720p60s] B={B} H={H} N={N} d={d} grid={grid} L={L}")
    qb, kb, vb = (la.split_blocks(t, L) for t in (tq, tk, tv))
    del tk, tv
    outs, S, z = la.block_causal(qb, kb, vb, N, grid, L, eps)
    torch.cuda.synchronize()
    out = torch.cat(outs, dim=2)
    for h in (0, 11, 31):
        qh = np.concatenate([host(x[0, h]) for x in qb])
        kh = np.concatenate([host(x[0, h]) for x in kb])
        vh = np.concatenate([host(x[0, h]) for x in vb])
        ref, Sr, zr = oracle.block_causal_head(qh, kh, vh, grid, L, eps)
        assert_close(host(out[0, h]), ref, "bf16", f"720p60s head {h} O")
        es = state_err(host(S[0, h]), Sr)
        say(f"  carry S head {h}: {es:.3e}")
        assert es <= 2e-2
        np.testing.assert_allclose(host(z[0, h]), zr, rtol=1e-4)


FUZZ = [
    # B, H, N, d, dtype, grid, eps
    (1, 1, 1, 64, "bf16", (1, 1, 1), 1e-6),
    (1, 1, 7, 32, "fp32", (2, 2, 2), 1e-6),
    (2, 3, 255, 64, "bf16", (3, 9, 10), 0.0),
    (1, 2, 4097, 128, "bf16", (5, 23, 40), 1e-6),
    (3, 1, 1000, 32, "bf16", None, 1e-6),
    (1, 2, 1000, 64, "fp32", (4, 17, 19), 1e-6),
    (1, 2, 777, 128, "fp32", (2, 20, 20), 1e-3),
    (2, 2, 513, 32, "fp32", None, 0.0),
    (1, 3, 130, 128, "bf16", (130, 1, 1), 1e-6),
    (1, 1, 5000, 64, "bf16", (3, 41, 41), 1e-6),
    (1, 2, 1000, 112, "bf16", (4, 17, 19), 1e-6),
    (2, 1, 333, 112, "fp32", (3, 11, 11), 1e-6),
    (1, 3, 64, 112, "bf16", None, 0.0),
]


@pytest.mark.parametrize("case", FUZZ, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{c[4]}" for c in FUZZ])
def test_fuzz_shapes(la, case):
    import torch
    B, H, N, d, dt, grid, eps = case
    say(f"[fuzz] {case}")
    q, k, v = make_qkv(B, H, N, d, dt, seed=2000 + N + d)
    out = la.bidirectional(upload(q, dt), upload(k, dt), upload(v, dt), grid, eps)
    torch.cuda.synchronize()
    ref = oracle.bidirectional(q, k, v, grid, eps)
    assert_close(host(out), ref, dt, f"fuzz {case}")


BC_FUZZ = [
    # B, H, N, d, dtype, grid, L, eps
    (1, 2, 1000, 64, "bf16", (10, 10, 10), 300, 1e-6),
    (2, 1, 257, 32, "fp32", (3, 9, 10), 64, 1e-6),
    (1, 1, 500, 128, "bf16", (5, 10, 10), 100, 0.0),
    (1, 2, 100, 64, "fp32", (4, 5, 5), 1, 1e-6),
    (1, 1, 640, 64, "bf16", None, 128, 1e-6),
    (1, 2, 900, 112, "bf16", (9, 10, 10), 250, 1e-6),
]


@pytest.mark.parametrize("case", BC_FUZZ, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{c[4]}L{c[6]}" for c in BC_FUZZ])
def test_fuzz_block_causal(la, case):
    import torch
    B, H, N, d, dt, grid, L, eps = case
    say(f"[bc fuzz] {case}")
    q, k, v = make_qkv(B, H, N, d, dt, seed=3000 + N + d)
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    qb, kb, vb = (la.split_blocks(t, L) for t in (tq, tk, tv))
    outs, S, z = la.block_causal(qb, kb, vb, N, grid, L, eps)
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.block_causal(q, k, v, grid, L, eps)
    assert_close(host(torch.cat(outs, dim=2)), ref, dt, f"bc fuzz {case}")
    assert state_err(host(S).reshape(-1, d), Sr.reshape(-1, d)) <= TOL[dt]


def test_state_reduce_empty_sequence(la):
    import torch
    k = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    S, z = la.state_reduce(k, k.clone(), None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S).item() == 0 and torch.count_nonzero(z).item() == 0


CROSS_CASES = [
    # B, H, N_q, N_kv, d, dtype, eps  (video queries over text keys/values, no RoPE)
    (1, 2, 777, 1, 32, "fp32", 1e-6),
    (1, 4, 100, 5000, 128, "bf16", 1e-6),
    (2, 3, 1000, 77, 64, "bf16", 0.0),
    (1, 1, 1, 7, 64, "fp32", 1e-6),
    (1, 2, 64, 0, 64, "bf16", 1e-6),
    (1, 20, 2000, 300, 112, "bf16", 1e-6),
    # one launch (bf16, d = 64, N_kv <= 512): one and two heads a workgroup,
    # ragged and full 128-token chunks of keys/values; 513 takes two launches
    (2, 16, 1500, 300, 64, "bf16", 1e-6),
    (2, 32, 999, 512, 64, "bf16", 1e-6),
    (1, 5, 333, 129, 64, "bf16", 1e-6),
    (1, 2, 64, 1, 64, "bf16", 0.0),
    (1, 3, 500, 513, 64, "bf16", 1e-6),
]


@pytest.mark.parametrize("case", CROSS_CASES, ids=[f"B{c[0]}H{c[1]}Nq{c[2]}Nkv{c[3]}d{c[4]}{c[5]}"
                                                    for c in CROSS_CASES])
def test_cross_attention(la, case):
    import torch
    B, H, Nq, Nkv, d, dt, eps = case
    say(f"[cross] {case}")
    rng = np.random.default_rng(4000 + Nq + Nkv + d)
    q = rng.standard_normal((B, H, Nq, d)).astype(np.float32)
    k = rng.standard_normal((B, H, Nkv, d)).astype(np.float32)
    v = rng.standard_normal((B, H, Nkv, d)).astype(np.float32)
    if dt == "bf16":
        from linear_attention_video_02_amd.inputs import round_to_bf16
        q, k, v = (round_to_bf16(a) for a in (q, k, v))
    out = la.cross_attention(upload(q, dt), upload(k, dt), upload(v, dt), eps)
    torch.cuda.synchronize()
    ref = oracle.cross_attention(q, k, v, eps)
    if Nkv == 0:
        assert torch.count_nonzero(out).item() == 0
    else:
        assert_close(host(out), ref, dt, f"cross {case}")


@pytest.mark.parametrize("B,H,Nkv", [(2, 32, 300), (1, 4, 200), (2, 16, 512)])
def test_cross_attention_one_launch_matches_two(la, B, H, Nkv):
    """The one-launch path against the state + apply launches on the same
    inputs: S and z summed in another order only (max row error 1e-2 of a
    bf16 ulp-scale difference), and bitwise equal over repeated calls."""
    import torch
    from linear_attention_video_02_amd.inputs import round_to_bf16
    rng = np.random.default_rng(4200 + B * H + Nkv)
    q, k, v = (round_to_bf16(rng.standard_normal(s).astype(np.float32))
               for s in ((B, H, 777, 64), (B, H, Nkv, 64), (B, H, Nkv, 64)))
    tq, tk, tv = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16")
    one = la.cross_attention(tq, tk, tv, 1e-6)
    again = la.cross_attention(tq, tk, tv, 1e-6)
    with la.tuning(cross_fused=0):
        two = la.cross_attention(tq, tk, tv, 1e-6)
    # more heads a workgroup than the one-launch instance holds: two launches too
    with la.tuning(apply_heads=4):
        four = la.cross_attention(tq, tk, tv, 1e-6)
    # one launch with one contiguous chunk per workgroup, and with few workgroups
    with la.tuning(apply_ilv=0):
        chunks = la.cross_attention(tq, tk, tv, 1e-6)
    with la.tuning(apply_wgs=7):
        few = la.cross_attention(tq, tk, tv, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(one, again)
    from _gpu import row_err
    e = row_err(host(one), host(two))
    say(f"  one launch vs two: {e:.3e}")
    assert e <= 1e-2
    assert torch.equal(two, four) or row_err(host(four), host(two)) <= 1e-2
    ref = oracle.cross_attention(q, k, v, 1e-6)
    assert_close(host(one), ref, "bf16", "one launch")
    assert_close(host(two), ref, "bf16", "two launches")
    assert_close(host(four), ref, "bf16", "four heads a workgroup")
    assert_close(host(chunks), ref, "bf16", "contiguous chunks")
    assert_close(host(few), ref, "bf16", "seven workgroups")


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 112])
def test_zero_denominator_rows(la, dt, d):
    """eps = 0 with a live query whose denominator is 0: the IEEE quotient.

    Cross-attention over no keys gives NaN rows for live queries and exact
    zeros for dead ones; a RoPE pair that turns keys living only on the
    partner channel of the query's channel gives +-inf (the oracle's
    definition, pinned on the CPU)."""
    import torch
    rng = np.random.default_rng(4100 + d)
    q = rng.standard_normal((1, 2, 40, d)).astype(np.float32)
    q[0, 0, 5] = -np.abs(q[0, 0, 5])  # a dead row
    if dt == "bf16":
        from linear_attention_video_02_amd.inputs import round_to_bf16
        q = round_to_bf16(q)
    k = np.zeros((1, 2, 0, d), np.float32)
    out = host(la.cross_attention(upload(q, dt), upload(k, dt), upload(k, dt), 0.0))
    torch.cuda.synchronize()
    ref = oracle.cross_attention(q, k, k, 0.0)
    assert np.array_equal(np.isnan(out), np.isnan(ref)) and np.isnan(ref).sum() == 79 * d
    assert np.array_equal(out[~np.isnan(ref)], ref[~np.isnan(ref)])
    # pair p = d/2 - floor(d/6) is the first w pair (angle = w); query on its
    # even channel, keys on its odd channel, V = 1, a 1 x 2 x 2 grid
    c = 2 * (d // 2 - d // 6)
    Q = np.zeros((1, 1, 4, d), np.float32)
    Q[..., c] = 1.0
    K = np.zeros((1, 1, 4, d), np.float32)
    K[..., c + 1] = 1.0
    V = np.ones((1, 1, 4, d), np.float32)
    out = host(la.bidirectional(upload(Q, dt), upload(K, dt), upload(V, dt), (1, 2, 2), 0.0))
    torch.cuda.synchronize()
    ref = oracle.bidirectional(Q, K, V, (1, 2, 2), 0.0)
    assert np.isinf(ref).all()
    assert np.array_equal(out, ref), (out[0, 0, :, :4], ref[0, 0, :, :4])


def test_cross720p(la):
    """The cross-attention workload at full size: 19320 video tokens over 300 text tokens."""
    import torch
    from linear_attention_video_02_amd.inputs import CROSS, make_cross_device
    w = CROSS["cross720p"]
    say(f"[cross720p] {w}")
    tq, tk, tv = make_cross_device(w["B"], w["H"], w["Nq"], w["Nkv"], w["d"], w["dtype"], w["seed"])
    out = la.cross_attention(tq, tk, tv, w["eps"])
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (1, 31), (0, 17)):
        ref = oracle.cross_attention_head(host(tq[b, h]), host(tk[b, h]), host(tv[b, h]), w["eps"])
        assert_close(host(out[b, h]), ref, "bf16", f"cross720p head ({b},{h})")


TC_CASES = [
    # B, H, N, d, grid, eps, dtype   (token-causal, Eq. 3 literally)
    (1, 1, 1, 64, (1, 1, 1), 1e-6, "bf16"),
    (1, 2, 1000, 64, (10, 10, 10), 1e-6, "bf16"),
    (2, 3, 300, 64, None, 1e-6, "bf16"),
    (1, 2, 129, 64, (2, 9, 10), 0.0, "bf16"),
    (1, 1, 5000, 64, (3, 41, 41), 1e-6, "bf16"),
    (1, 4, 4097, 64, (5, 23, 40), 1e-6, "bf16"),
    # other head sizes: 32 on the 64-channel kernel, 112 and 128 on the 128-channel one
    (1, 2, 1000, 32, (10, 10, 10), 1e-6, "bf16"),
    (2, 3, 300, 32, None, 1e-6, "bf16"),
    (1, 2, 1000, 112, (10, 10, 10), 1e-6, "bf16"),
    (1, 3, 129, 112, (2, 9, 10), 0.0, "bf16"),
    (1, 1, 4097, 112, (5, 23, 40), 1e-6, "bf16"),
    (1, 2, 1000, 128, (10, 10, 10), 1e-6, "bf16"),
    (2, 2, 2077, 128, None, 1e-6, "bf16"),
    (1, 1, 1, 128, (1, 1, 1), 1e-6, "bf16"),
    # fp32 inputs
    (1, 2, 1000, 64, (10, 10, 10), 1e-6, "fp32"),
    (1, 1, 129, 64, (2, 9, 10), 0.0, "fp32"),
    (2, 2, 300, 32, None, 1e-6, "fp32"),
    (1, 1, 3001, 112, (4, 23, 40), 1e-6, "fp32"),
    (1, 2, 777, 128, (3, 23, 40), 1e-6, "fp32"),
    (1, 1, 1, 32, (1, 1, 1), 1e-6, "fp32"),
]


@pytest.mark.parametrize("case", TC_CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{c[6]}" for c in TC_CASES])
def test_token_causal(la, case):
    import torch
    B, H, N, d, grid, eps, dt = case
    say(f"[token-causal] {case}")
    q, k, v = make_qkv(B, H, N, d, dt, seed=5000 + N + d)
    out = la.token_causal(upload(q, dt), upload(k, dt), upload(v, dt), grid, eps)
    torch.cuda.synchronize()
    ref, _, _ = oracle.token_causal(q, k, v, grid, eps)
    assert_close(host(out), ref, dt, f"token-causal {case}")


def test_token_causal_sana2b(la):
    """SANA-Video-2B heads (H = 20, d = 112) on the 720p-5s latent in
    token-causal mode; sampled heads, every row."""
    import torch
    tq, tk, tv, w = make_workload_device("sana2b")
    grid, eps = w["grid"], w["eps"]
    out = la.token_causal(tq, tk, tv, grid, eps)
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (0, 19), (0, 7)):
        ref, _, _ = oracle.token_causal_head(host(tq[b, h]), host(tk[b, h]), host(tv[b, h]), grid, eps)
        assert_close(host(out[b, h]), ref, "bf16", f"sana2b token-causal head ({b},{h})")


def test_token_causal_720p5s(la):
    """The 720p-5s workload in token-causal mode; sampled heads, every row."""
    import torch
    tq, tk, tv, w = make_workload_device("720p5s")
    grid, eps = w["grid"], w["eps"]
    out = la.token_causal(tq, tk, tv, grid, eps)
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (1, 31), (0, 13)):
        ref, _, _ = oracle.token_causal_head(host(tq[b, h]), host(tk[b, h]), host(tv[b, h]), grid, eps)
        assert_close(host(out[b, h]), ref, "bf16", f"720p5s token-causal head ({b},{h})")


@pytest.mark.parametrize("d,dt", [(64, "bf16"), (112, "bf16"), (32, "bf16"), (64, "fp32"), (128, "fp32")])
def test_token_causal_carry_resume_and_determinism(la, d, dt):
    """Two segments with a carry and a position offset == one call; final carry == total state."""
    import torch
    B, H, N, grid, eps = 1, 2, 2000, (5, 20, 20), 1e-6
    q, k, v = make_qkv(B, H, N, d, dt, seed=5100)
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda:0")
    z = torch.zeros((B, H, d), dtype=torch.float32, device="cuda:0")
    m = 777
    o1 = la.token_causal(tq[:, :, :m].contiguous(), tk[:, :, :m].contiguous(), tv[:, :, :m].contiguous(),
                         grid, eps, S, z, 0)
    o2 = la.token_causal(tq[:, :, m:].contiguous(), tk[:, :, m:].contiguous(), tv[:, :, m:].contiguous(),
                         grid, eps, S, z, m)
    whole = la.token_causal(tq, tk, tv, grid, eps)
    again = la.token_causal(tq, tk, tv, grid, eps)
    torch.cuda.synchronize()
    assert torch.equal(whole, again), "repeated calls differ"
    ref, Sr, zr = oracle.token_causal(q, k, v, grid, eps)
    assert_close(host(torch.cat([o1, o2], dim=2)), ref, dt, "two segments with carry")
    assert state_err(host(S).reshape(-1, d), Sr.reshape(-1, d)) <= 1e-4
    np.testing.assert_allclose(host(z), zr, rtol=1e-5)
    # empty segment: carry unchanged
    S0 = S.clone()
    la.token_causal(tq[:, :, :0].contiguous(), tk[:, :, :0].contiguous(), tv[:, :, :0].contiguous(),
                    grid, eps, S, z, N)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)


@pytest.mark.parametrize("d,dt", [(64, "bf16"), (32, "bf16"), (112, "bf16"), (64, "fp32")])
def test_token_causal_zero_carry_equals_no_carry_bitwise(la, d, dt):
    """Starting from a zero carry is starting from the empty state: the output is
    bitwise the one without a carry.  (Without a carry, bf16 at d <= 64 forms
    each chunk's prefix inside the scan; with one, a separate prefix launch
    does, from the carry's zeros -- the same sums in the same order.)"""
    import torch
    B, H, N, grid, eps = 2, 3, 9000, (10, 30, 30), 1e-6
    q, k, v = make_qkv(B, H, N, d, dt, seed=5300 + d)
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda:0")
    z = torch.zeros((B, H, d), dtype=torch.float32, device="cuda:0")
    with_carry = la.token_causal(tq, tk, tv, grid, eps, S, z, 0)
    without = la.token_causal(tq, tk, tv, grid, eps)
    torch.cuda.synchronize()
    say(f"[token-causal zero carry] d={d} {dt}")
    assert torch.equal(with_carry, without)
    ref, _, _ = oracle.token_causal(q[:, :1], k[:, :1], v[:, :1], grid, eps)
    assert_close(host(without[:, :1]), ref, dt, f"d={d} {dt} batch 0")
