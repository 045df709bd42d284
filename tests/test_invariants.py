"""GPU invariants of the HIP path (through the C ABI).

* bitwise determinism over repeated calls (fixed-order cross-workgroup sums);
* one block covering the whole sequence == bidirectional, bitwise;
* resuming block-causal mode from a carry copied through the host gives
  bitwise the same outputs and carry as the uninterrupted run (the carry is
  the whole cache: Eq. 3's running sums, Algorithm 1);
* commit = 0 leaves the carry untouched and gives the same output as commit = 1;
* the last block's rows match bidirectional attention;
* rows with relu(Q) = 0 are exactly zero, with and without eps;
* constant V without RoPE is reproduced;
* canary words around every output stay untouched.
"""
import numpy as np
import pytest

import oracle
from _gpu import assert_close, host, say, upload
from linear_attention_video_02_amd.inputs import make_qkv, round_to_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    import linear_attention_video_02_amd as m
    m.lib()
    return m


def _inputs(B, H, N, d, dt, seed):
    q, k, v = make_qkv(B, H, N, d, dt, seed=seed)
    return (q, k, v), tuple(upload(a, dt) for a in (q, k, v))


def test_determinism_bidirectional(la):
    import torch
    _, (tq, tk, tv) = _inputs(2, 8, 8190, 64, "bf16", 11)
    grid = (21, 15, 26)
    ref = la.bidirectional(tq, tk, tv, grid)
    S0, z0 = la.state_reduce(tk, tv, grid)
    for i in range(10):
        o = la.bidirectional(tq, tk, tv, grid)
        S, z = la.state_reduce(tk, tv, grid)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), i
        assert torch.equal(S, S0) and torch.equal(z, z0), i


@pytest.mark.parametrize("d", [32, 64, 112, 128])
@pytest.mark.parametrize("N,L", [(5000, 1000), (400, 200)])
def test_fused_combine_matches_separate_launch(la, d, N, L):
    """The bf16 state kernel's in-kernel stage 2 (last workgroup of a head sums
    the partials; with a short sequence, one workgroup per head writing the
    sums directly) and the separate combine launch give bitwise equal S and
    z, also with a carry (block-causal), over repeated calls on one workspace."""
    import torch
    _, (tq, tk, tv) = _inputs(2, 6, N, d, "bf16", 17)
    grid = (6, 23, 40)
    qb, kb, vb = (t[:, :, L:2 * L].contiguous() for t in (tq, tk, tv))
    res = {}
    for fused in (0, 1):
        runs = []
        with la.tuning(state_fused=fused):
            for _ in range(3):
                S, z = la.state_reduce(tk, tv, grid)
                Sc = S.clone() * 0.5
                zc = z.clone() * 0.5
                la.block_causal_step(qb, kb, vb, Sc, zc, N, grid, L, 1, commit=True)
                runs.append((S, z, Sc, zc))
            torch.cuda.synchronize()
        for r in runs[1:]:
            assert all(torch.equal(x, y) for x, y in zip(r, runs[0])), fused
        res[fused] = runs[0]
    say(f"  d={d} N={N}: fused and separate stage 2 bitwise equal")
    assert all(torch.equal(x, y) for x, y in zip(res[0], res[1]))


APPLY_SPLITS = [dict(apply_ilv=0), dict(), dict(apply_heads=1), dict(apply_heads=2),
                dict(apply_heads=3), dict(apply_heads=4), dict(apply_wgs=7),
                dict(apply_spread=0), dict(apply_heads=6), dict(apply_wgs=24, apply_heads=2)]


@pytest.mark.parametrize("d", [32, 64, 112, 128])
@pytest.mark.parametrize("B,H,N", [(2, 6, 4999), (1, 1, 2077), (3, 4, 700)])
def test_apply_work_splits_are_bitwise_equal(la, d, B, H, N):
    """The bf16 apply gives bitwise equal outputs however its work is split:
    one contiguous chunk per workgroup, or interleaved units of whole heads
    with 1, 2, 3, 4 or 6 heads per slot (when B*H allows), few workgroups,
    a slot's workgroups on all XCDs or on few; with and without RoPE, and for a block at a global
    offset (block-causal mode), on ragged token counts."""
    import torch
    _, (tq, tk, tv) = _inputs(B, H, N, d, "bf16", 23)
    grid = (6, 23, 40)
    S, z = la.state_reduce(tk, tv, grid)
    L = N // 3  # block 1 of three: tokens [L, 2L)
    qb, kb, vb = (t[:, :, L:2 * L].contiguous() for t in (tq, tk, tv))
    res = []
    for knobs in APPLY_SPLITS:
        with la.tuning(**knobs):
            o_rope = la.apply(tq, S, z, grid, 1e-6)
            o_plain = la.apply(tq, S, z, None, 1e-6)
            Sc, zc = S.clone() * 0.5, z.clone() * 0.5
            ob = la.block_causal_step(qb, kb, vb, Sc, zc, N, grid, L, 1, commit=False)
            torch.cuda.synchronize()
        res.append((o_rope, o_plain, ob))
    for knobs, r in zip(APPLY_SPLITS[1:], res[1:]):
        assert all(torch.equal(x, y) for x, y in zip(res[0], r)), knobs
    say(f"  d={d} B={B} H={H} N={N}: {len(APPLY_SPLITS)} apply work splits bitwise equal")


def oracle_bf16(x):
    """x rounded to bf16 values (float32 array), as the GPU receives it."""
    return round_to_bf16(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("d", [32, 64, 112, 128])
def test_query_magnitudes(la, d):
    """The bf16 apply rounds RoPE(relu Q) to fp16 after scaling any 16-token
    group that holds a relu(Q) value outside [2^-6, 2^14) by a power of two
    per token.  Queries scaled by 1e-20 .. 1e20, and groups mixing tiny,
    ordinary and huge tokens, must match the oracle like ordinary ones."""
    import torch
    N, grid = 700, (2, 20, 20)
    q, k, v = make_qkv(1, 2, N, d, "bf16", seed=23)
    ref_eps = 1e-6
    for scale in (1e-20, 1e-5, 1e-2, 1.0, 3e4, 1e6, 1e20):
        qs = oracle_bf16(q * scale)
        out = la.bidirectional(upload(qs, "bf16"), upload(k, "bf16"), upload(v, "bf16"), grid, ref_eps)
        torch.cuda.synchronize()
        o = host(out)
        assert np.all(np.isfinite(o)), scale
        assert_close(o, oracle.bidirectional(qs, k, v, grid, ref_eps), "bf16", f"d={d} Q x {scale:g}")
    # every token of a group at its own magnitude
    mags = np.array([1e-30, 1e-9, 1e-3, 0.5, 1.0, 7.0, 2e4, 1e9, 1e30], dtype=np.float64)
    qm = oracle_bf16(q * mags[np.arange(N) % len(mags)][None, None, :, None])
    out = la.bidirectional(upload(qm, "bf16"), upload(k, "bf16"), upload(v, "bf16"), grid, ref_eps)
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(np.isfinite(o))
    assert_close(o, oracle.bidirectional(qm, k, v, grid, ref_eps), "bf16", f"d={d} mixed token magnitudes")


def test_determinism_d128_fp32(la):
    import torch
    _, (tq, tk, tv) = _inputs(1, 4, 3000, 128, "fp32", 12)
    ref = la.bidirectional(tq, tk, tv, (4, 23, 40))
    for _ in range(5):
        assert torch.equal(la.bidirectional(tq, tk, tv, (4, 23, 40)), ref)


def test_single_block_equals_bidirectional_bitwise(la):
    import torch
    _, (tq, tk, tv) = _inputs(1, 4, 2000, 64, "bf16", 13)
    grid = (5, 20, 20)
    ref = la.bidirectional(tq, tk, tv, grid)
    outs, S, z = la.block_causal([tq], [tk], [tv], 2000, grid, 2000)
    S2, z2 = la.state_reduce(tk, tv, grid)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], ref)
    assert torch.equal(S, S2) and torch.equal(z, z2)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_resume_from_host_carry_is_bitwise(la, dt):
    import torch
    N, L, grid = 2200, 220, (10, 11, 20)
    _, (tq, tk, tv) = _inputs(1, 4, N, 64, dt, 14)
    qb, kb, vb = (la.split_blocks(t, L) for t in (tq, tk, tv))
    full, S, z = la.block_causal(qb, kb, vb, N, grid, L)
    first, S5, z5 = la.block_causal(qb[:5], kb[:5], vb[:5], N, grid, L)
    torch.cuda.synchronize()
    S_host, z_host = S5.cpu().numpy().copy(), z5.cpu().numpy().copy()
    del S5, z5
    S_new = torch.from_numpy(S_host).cuda()
    z_new = torch.from_numpy(z_host).cuda()
    rest, S_end, z_end = la.block_causal(qb[5:], kb[5:], vb[5:], N, grid, L, S_carry=S_new,
                                         z_carry=z_new, first_block=5)
    torch.cuda.synchronize()
    for a, b in zip(first + rest, full):
        assert torch.equal(a, b)
    assert torch.equal(S_end, S) and torch.equal(z_end, z)


def test_peek_leaves_carry_untouched(la):
    import torch
    N, L, grid = 1200, 400, (3, 20, 20)
    _, (tq, tk, tv) = _inputs(1, 2, N, 64, "bf16", 15)
    qb, kb, vb = (la.split_blocks(t, L) for t in (tq, tk, tv))
    _, S, z = la.block_causal(qb[:1], kb[:1], vb[:1], N, grid, L)
    S0, z0 = S.clone(), z.clone()
    peek = la.block_causal_step(qb[1], kb[1], vb[1], S, z, N, grid, L, 1, commit=False)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(z, z0)
    commit = la.block_causal_step(qb[1], kb[1], vb[1], S, z, N, grid, L, 1, commit=True)
    torch.cuda.synchronize()
    assert torch.equal(peek, commit)
    assert not torch.equal(S, S0)


def test_last_block_matches_bidirectional(la):
    import torch
    N, L, grid = 3000, 600, (6, 20, 25)
    (q, k, v), (tq, tk, tv) = _inputs(1, 2, N, 64, "bf16", 16)
    qb, kb, vb = (la.split_blocks(t, L) for t in (tq, tk, tv))
    outs, S, z = la.block_causal(qb, kb, vb, N, grid, L)
    bi = la.bidirectional(tq, tk, tv, grid)
    S2, z2 = la.state_reduce(tk, tv, grid)
    torch.cuda.synchronize()
    ref = oracle.bidirectional(q, k, v, grid, 1e-6)
    assert_close(host(outs[-1]), ref[:, :, N - L:], "bf16", "last block vs oracle bidirectional")
    assert_close(host(outs[-1]), host(bi[:, :, N - L:]), "bf16", "last block vs GPU bidirectional")
    np.testing.assert_allclose(host(S), host(S2), rtol=1e-5, atol=1e-3)
    np.testing.assert_allclose(host(z), host(z2), rtol=1e-5)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("eps", [0.0, 1e-6])
def test_zero_query_rows_exact(la, dt, eps):
    import torch
    q, k, v = make_qkv(1, 2, 700, 64, dt, seed=17)
    q[:, :, ::5] = -np.abs(q[:, :, ::5])
    out = la.bidirectional(upload(q, dt), upload(k, dt), upload(v, dt), (2, 20, 20), eps)
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(o[:, :, ::5] == 0.0)
    assert np.all(np.isfinite(o))
    assert_close(o, oracle.bidirectional(q, k, v, (2, 20, 20), eps), dt, f"zero rows {dt} eps={eps}")


def test_constant_v_reproduced(la):
    import torch
    q, k, _ = make_qkv(1, 2, 5000, 64, "bf16", seed=18)
    c = np.linspace(-2, 2, 64).astype(np.float32)
    v = np.broadcast_to(c, (1, 2, 5000, 64)).copy()
    out = la.bidirectional(upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16"), None, 0.0)
    torch.cuda.synchronize()
    o = host(out)
    live = (q > 0).any(axis=-1)
    got = o[live]
    want = np.broadcast_to(host(upload(c, "bf16")), got.shape)
    assert oracle.rel_row_error(got, want) <= 2e-2


def test_canaries_untouched(la):
    import torch
    B, H, N, d, grid = 1, 3, 1001, 64, (3, 20, 20)
    _, (tq, tk, tv) = _inputs(B, H, N, d, "bf16", 19)
    pad = 4096
    n_o = B * H * N * d
    canary = torch.full((n_o + 2 * pad,), -7.0, dtype=torch.bfloat16, device="cuda:0")
    out = canary[pad:pad + n_o].view(B, H, N, d)
    Sbuf = torch.full((B * H * d * d + 2 * pad,), 3.5, dtype=torch.float32, device="cuda:0")
    zbuf = torch.full((B * H * d + 2 * pad,), 3.5, dtype=torch.float32, device="cuda:0")
    S = Sbuf[pad:pad + B * H * d * d].view(B, H, d, d)
    z = zbuf[pad:pad + B * H * d].view(B, H, d)
    la.state_reduce(tk, tv, grid, S=S, z=z)
    la.apply(tq, S, z, grid, 1e-6, out=out)
    torch.cuda.synchronize()
    for buf, val in ((canary, -7.0), (Sbuf, 3.5), (zbuf, 3.5)):
        assert torch.all(buf[:pad] == val) and torch.all(buf[-pad:] == val)
    say("  canaries intact")


def test_token_causal_canaries_untouched(la):
    """Token-causal outputs stay inside their tensor, also when a head's last
    chunk has an odd number of 64-token steps (937 tokens: chunks of 128 and a
    last chunk of 41) and the scan runs one step past the chunk."""
    import torch
    B, H, N, d, grid = 1, 3, 937, 64, (3, 20, 20)
    (q, k, v), (tq, tk, tv) = _inputs(B, H, N, d, "bf16", 29)
    pad = 4096
    n_o = B * H * N * d
    canary = torch.full((n_o + 2 * pad,), -7.0, dtype=torch.bfloat16, device="cuda:0")
    out = canary[pad:pad + n_o].view(B, H, N, d)
    la.token_causal(tq, tk, tv, grid, 1e-6, out=out)
    torch.cuda.synchronize()
    assert torch.all(canary[:pad] == -7.0) and torch.all(canary[-pad:] == -7.0)
    ref, _, _ = oracle.token_causal(q, k, v, grid, 1e-6)
    assert_close(host(out), ref, "bf16", "token-causal, odd last chunk")
    say("  token-causal canaries intact")


def test_stream_copy_is_exact(la):
    """The measurement copy (la_stream_copy) moves every byte, at a size that
    is not a multiple of one workgroup's 4 KB, and writes nothing past the end."""
    import torch
    n = 5 * 1048576 + 20  # 1,310,725 pieces of 16 bytes: the last workgroup holds 5
    src = torch.randint(0, 2**31 - 1, (n + 1024,), dtype=torch.int32, device="cuda:0")
    dst = torch.full((n + 1024,), -7, dtype=torch.int32, device="cuda:0")
    la.stream_copy(src[:n], dst[:n])
    torch.cuda.synchronize()
    assert torch.equal(src[:n], dst[:n])
    assert bool((dst[n:] == -7).all())


def test_stale_counters_heal(la):
    """Counters a call finds from an earlier call that never completed (an
    older epoch, a partial count) restart at zero: the same outputs, bitwise."""
    import torch
    _, (tq, tk, tv) = _inputs(2, 8, 6000, 64, "bf16", 29)
    grid = (7, 23, 40)
    ws = la.workspace(2, 8, 6000, 64, tq.device, grid=grid)
    ref = la.bidirectional(tq, tk, tv, grid, ws=ws).clone()
    S0, z0 = la.state_reduce(tk, tv, grid, ws=ws)
    S0, z0 = S0.clone(), z0.clone()
    torch.cuda.synchronize()
    # epoch 1, count 3: what an interrupted first call could leave
    stale = torch.full((2048,), (1 << 32) | 3, dtype=torch.int64, device=tq.device)
    ws[:16384].copy_(stale.view(torch.uint8))
    out = la.bidirectional(tq, tk, tv, grid, ws=ws)
    ws[:16384].copy_(stale.view(torch.uint8))
    S, z = la.state_reduce(tk, tv, grid, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(S, S0) and torch.equal(z, z0)


def test_graph_replays_match_eager(la):
    """A captured state + apply step replayed with new input contents, with
    eager calls on the same workspace between the replays, gives the eager
    outputs of those inputs on every replay.  The captured state launch keeps
    one counter epoch, so this holds only because the workgroup that completes
    a head puts its counter back to zero."""
    import torch
    B, H, N, d = 2, 32, 3000, 64  # four partials of 16 KB a head: fused stage 2
    grid = (4, 23, 40)
    sets = [_inputs(B, H, N, d, "bf16", 40 + i)[1] for i in range(3)]
    ws = la.workspace(B, H, N, d, sets[0][0].device, grid=grid)
    eager = [la.bidirectional(q, k, v, grid, ws=ws).clone() for q, k, v in sets]
    sq, sk, sv = (t.clone() for t in sets[0])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up call on the capture stream
        la.bidirectional(sq, sk, sv, grid, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = la.bidirectional(sq, sk, sv, grid, ws=ws)
    for rep in range(6):
        i = rep % 3
        for dst, src in zip((sq, sk, sv), sets[i]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[i]), rep
        # eager work on the same workspace between replays
        o2 = la.bidirectional(*sets[(i + 1) % 3], grid, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(o2, eager[(i + 1) % 3]), rep


def test_one_workspace_many_shapes(la):
    """One workspace, zero-filled once, shared by calls of different sizes in
    turn: a call whose partial states cover the bytes another shape's counters
    would sit at must not disturb that shape's next call (the counters have a
    fixed place)."""
    import torch
    shapes = [(1, 16, 4000, 128, (4, 25, 40)), (2, 32, 3000, 64, (3, 25, 40)), (1, 4, 2500, 32, (3, 25, 40))]
    data = [_inputs(B, H, N, d, "bf16", 70 + i)[1] for i, (B, H, N, d, _) in enumerate(shapes)]
    ref = []
    for (B, H, N, d, grid), (q, k, v) in zip(shapes, data):
        ws = torch.zeros(la.workspace_bytes(B, H, N, d, grid), dtype=torch.uint8, device=q.device)
        S, z = la.state_reduce(k, v, grid, ws=ws)
        ref.append((S.clone(), z.clone(), la.bidirectional(q, k, v, grid, ws=ws).clone()))
    nbytes = max(la.workspace_bytes(B, H, N, d, grid) for B, H, N, d, grid in shapes)
    shared = torch.zeros(nbytes, dtype=torch.uint8, device=data[0][0].device)
    for rep in range(3):
        for i in (0, 1, 2, 1, 0):
            q, k, v = data[i]
            grid = shapes[i][4]
            S, z = la.state_reduce(k, v, grid, ws=shared)
            o = la.bidirectional(q, k, v, grid, ws=shared)
            torch.cuda.synchronize()
            assert torch.equal(S, ref[i][0]) and torch.equal(z, ref[i][1]), (rep, i)
            assert torch.equal(o, ref[i][2]), (rep, i)


def test_two_streams_each_get_their_own_workspace(la):
    """Calls on two streams at once: the binding hands each stream its own
    workspace (the in-kernel second stage keeps per-head counters and partial
    states there), so both give bitwise the results of one-stream calls."""
    import torch
    B, H, N, d, grid = 2, 16, 6000, 64, (7, 25, 40)
    (_, _, _), (q1, k1, v1) = _inputs(B, H, N, d, "bf16", 81)
    (_, _, _), (q2, k2, v2) = _inputs(B, H, N, d, "bf16", 82)
    S1, z1 = la.state_reduce(k1, v1, grid)
    S2, z2 = la.state_reduce(k2, v2, grid)
    o1 = la.bidirectional(q1, k1, v1, grid)
    o2 = la.bidirectional(q2, k2, v2, grid)
    torch.cuda.synchronize()
    ref = [(S1.clone(), z1.clone(), o1.clone()), (S2.clone(), z2.clone(), o2.clone())]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(5):
        got = []
        for s, (q, k, v) in zip(streams, ((q1, k1, v1), (q2, k2, v2))):
            with torch.cuda.stream(s):
                S, z = la.state_reduce(k, v, grid)
                o = la.bidirectional(q, k, v, grid)
                got.append((S, z, o))
        torch.cuda.synchronize()
        for i in range(2):
            for a, b in zip(got[i], ref[i]):
                assert torch.equal(a, b), (rep, i)
    ws = {id(la.workspace(B, H, N, d, q1.device, stream=s, grid=grid)) for s in streams}
    assert len(ws) == 2
