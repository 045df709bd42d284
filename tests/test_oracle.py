"""Pins of the fp64 oracle against things other than itself (CPU only).

Each pin ties the oracle to the SANA-Video analysis page's formulas (section
3.4: the ReLU linear-attention equation, Eq. 2, Eq. 3 with its update rule,
Algorithm 1) or to mathematics that holds whatever the implementation:

* an independent O(N^2) brute force written with explicit loops, complex-number
  rotation (the RoFormer form x * e^{i m theta}) and its own nested-loop
  enumeration of grid positions;
* hand-derived worked examples (tests/golden/worked_examples.txt);
* the hand-worked axis split (tests/golden/rope_axis_split.txt);
* invariants: rotation preserves norms and depends only on relative position,
  constant V is reproduced, permutation equivariance without RoPE, scale
  invariance, the last block of block-causal mode equals bidirectional output,
  token-causal Eq. 3 at block size 1.

test_pins_catch_planted_mistakes plants plausible mistakes in the oracle and
checks that some pin fails for each.
"""
import cmath
import math
import os

import numpy as np
import pytest

import oracle
from oracle import linattn_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent helpers (no oracle code)
# ---------------------------------------------------------------------------

def load_axis_split():
    table = {}
    with open(os.path.join(GOLDEN, "rope_axis_split.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                d, pt, ph, pw = map(int, line)
                table[d] = (pt, ph, pw)
    return table


def load_examples():
    examples, cur = [], None
    with open(os.path.join(GOLDEN, "worked_examples.txt")) as f:
        for raw in f:
            line = raw.split("#")[0].strip()
            if not line:
                continue
            key, _, val = line.partition(":")
            if key == "example":
                cur = {"name": val.strip(), "Q": [], "K": [], "V": [], "O": []}
            elif key == "grid":
                cur["grid"] = tuple(int(x) for x in val.split())
            elif key in ("Q", "K", "V", "O"):
                cur[key].append([float(x) for x in val.split()])
            elif key == "end":
                examples.append({k: (np.array(v) if k in "QKVO" else v) for k, v in cur.items()})
    return examples


def enumerate_positions(grid, n_tokens):
    """Token -> (t, h, w) by walking the grid in t, then h, then w order."""
    pos = []
    gt, gh, gw = grid
    for t in range(gt):
        for h in range(gh):
            for w in range(gw):
                pos.append((t, h, w))
    return pos[:n_tokens]


def rotate_loop(x, tpos, split):
    """RoFormer rotation of interleaved pairs, written as complex multiplication."""
    d = len(x)
    out = [0.0] * d
    pair = 0
    for axis, npairs in enumerate(split):
        for k in range(npairs):
            theta = 10000.0 ** (-2.0 * k / (2 * npairs))  # RoFormer: base^(-2i/dim), dim = 2*npairs
            c = complex(x[2 * pair], x[2 * pair + 1]) * cmath.exp(1j * tpos[axis] * theta)
            out[2 * pair], out[2 * pair + 1] = c.real, c.imag
            pair += 1
    return out


def brute_force_loops(Q, K, V, grid, eps, block=None, token_causal=False):
    """O_i = sum_j w_ij V_j / (sum_j u_ij + eps) with explicit double loops."""
    N, d = Q.shape
    relu = lambda row: [max(float(a), 0.0) for a in row]  # noqa: E731
    q = [relu(r) for r in Q]
    k = [relu(r) for r in K]
    if grid is not None:
        split = load_axis_split()[d]
        pos = enumerate_positions(grid, N)
        qr = [rotate_loop(q[i], pos[i], split) for i in range(N)]
        kr = [rotate_loop(k[j], pos[j], split) for j in range(N)]
    else:
        qr, kr = q, k
    out = np.zeros((N, d))
    for i in range(N):
        num = [0.0] * d
        den = 0.0
        for j in range(N):
            if block is not None and j // block > i // block:
                continue
            if token_causal and j > i:
                continue
            w = sum(qr[i][c] * kr[j][c] for c in range(d))
            u = sum(q[i][c] * k[j][c] for c in range(d))
            for c in range(d):
                num[c] += w * float(V[j][c])
            den += u
        if any(a > 0.0 for a in q[i]):
            out[i] = [a / (den + eps) for a in num]
    return out


def brute_force_cross_loops(Q, K, V, eps):
    """Cross-attention O_i = sum_j (q.k_j) V_j / (sum_j q.k_j + eps), explicit loops, N_q != N_kv."""
    Nq, d = Q.shape
    out = np.zeros((Nq, d))
    for i in range(Nq):
        q = [max(float(a), 0.0) for a in Q[i]]
        num = [0.0] * d
        den = 0.0
        for j in range(K.shape[0]):
            k = [max(float(a), 0.0) for a in K[j]]
            w = sum(q[c] * k[c] for c in range(d))
            for c in range(d):
                num[c] += w * float(V[j][c])
            den += w
        if any(a > 0.0 for a in q):
            out[i] = [a / (den + eps) for a in num]
    return out


def brute_force_state_loops(K, V, grid):
    """S[c_in][c_out] = sum_j RoPE(relu K_j)[c_in] V_j[c_out], z = sum_j relu K_j, with loops."""
    N, d = K.shape
    split = load_axis_split()[d] if grid is not None else None
    pos = enumerate_positions(grid, N) if grid is not None else None
    S = np.zeros((d, d))
    z = np.zeros(d)
    for j in range(N):
        k = [max(float(a), 0.0) for a in K[j]]
        kr = rotate_loop(k, pos[j], split) if grid is not None else k
        for a in range(d):
            z[a] += k[a]
            for b in range(d):
                S[a][b] += kr[a] * float(V[j][b])
    return S, z


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# pin checks (raise AssertionError on failure); reused by the mutation test
# ---------------------------------------------------------------------------

def check_worked_examples():
    for ex in load_examples():
        got = oracle.bidirectional_head(ex["Q"], ex["K"], ex["V"], ex["grid"], 0.0)
        np.testing.assert_allclose(got, ex["O"], rtol=1e-13, atol=1e-13, err_msg=ex["name"])


def check_brute_force_bidirectional():
    cases = [(24, 8, (2, 3, 4), 1), (20, 12, (3, 2, 5), 2), (16, 32, (2, 2, 4), 3),
             (17, 8, (2, 3, 3), 4), (12, 6, None, 5), (30, 64, (2, 3, 5), 6)]
    for N, d, grid, seed in cases:
        Q, K, V = rand((3, N, d), seed)
        for eps in (0.0, 1e-6):
            ref = brute_force_loops(Q, K, V, grid, eps)
            got = oracle.bidirectional_head(Q, K, V, grid, eps)
            np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12,
                                       err_msg=f"N={N} d={d} grid={grid}")


def check_brute_force_block_causal():
    for N, d, grid, L, seed in [(24, 8, (4, 2, 3), 6, 7), (23, 12, (2, 3, 4), 5, 8),
                                (18, 8, (3, 2, 3), 18, 9), (10, 8, (2, 1, 5), 1, 10)]:
        Q, K, V = rand((3, N, d), seed)
        ref = brute_force_loops(Q, K, V, grid, 1e-6, block=L)
        got, _, _ = oracle.block_causal_head(Q, K, V, grid, L, 1e-6)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12, err_msg=f"N={N} L={L}")


def check_brute_force_cross():
    for Nq, Nkv, d, seed in [(13, 5, 8, 21), (7, 19, 16, 22), (9, 1, 8, 23), (4, 0, 8, 24)]:
        rng = np.random.default_rng(seed)
        Q = rng.standard_normal((Nq, d))
        K = rng.standard_normal((Nkv, d))
        V = rng.standard_normal((Nkv, d))
        for eps in (1e-6, 1e-3):  # eps > 0: a live query with no overlapping key has den = eps
            ref = brute_force_cross_loops(Q, K, V, eps)
            got = oracle.cross_attention_head(Q, K, V, eps)
            np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12, err_msg=f"Nq={Nq} Nkv={Nkv}")


def check_brute_force_token_causal():
    for N, d, grid, seed in [(20, 8, (2, 2, 5), 41), (17, 12, (3, 2, 3), 42), (9, 6, None, 43)]:
        Q, K, V = rand((3, N, d), seed)
        ref = brute_force_loops(Q, K, V, grid, 1e-6, token_causal=True)
        got, _, _ = oracle.token_causal_head(Q, K, V, grid, 1e-6)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12, err_msg=f"N={N} d={d}")


def check_batched_wrappers():
    """The [B, H, N, d] entry points route every argument to every (batch, head) slice.

    Each wrapper runs on B = 2, H = 3 with a large, non-default eps (so that an
    eps that falls back to its default shows), a grid and a block size, and is
    compared slice by slice with the loop brute force of that slice.
    """
    B, H, N, d, grid, L, eps = 2, 3, 14, 8, (2, 2, 4), 5, 0.37
    rng = np.random.default_rng(61)
    Q, K, V = rng.standard_normal((3, B, H, N, d))
    got = oracle.bidirectional(Q, K, V, grid, eps)
    got_bc, S_bc, z_bc = oracle.block_causal(Q, K, V, grid, L, eps)
    got_tc, S_tc, z_tc = oracle.token_causal(Q, K, V, grid, eps)
    Kc, Vc = rng.standard_normal((2, B, H, 5, d))
    got_x = oracle.cross_attention(Q, Kc, Vc, eps)
    for b in range(B):
        for h in range(H):
            where = f"slice ({b}, {h})"
            q, k, v = Q[b, h], K[b, h], V[b, h]
            np.testing.assert_allclose(got[b, h], brute_force_loops(q, k, v, grid, eps),
                                       rtol=1e-10, atol=1e-12, err_msg="bidirectional " + where)
            np.testing.assert_allclose(got_bc[b, h], brute_force_loops(q, k, v, grid, eps, block=L),
                                       rtol=1e-10, atol=1e-12, err_msg="block_causal " + where)
            np.testing.assert_allclose(got_tc[b, h], brute_force_loops(q, k, v, grid, eps, token_causal=True),
                                       rtol=1e-10, atol=1e-12, err_msg="token_causal " + where)
            np.testing.assert_allclose(got_x[b, h], brute_force_cross_loops(q, Kc[b, h], Vc[b, h], eps),
                                       rtol=1e-10, atol=1e-12, err_msg="cross_attention " + where)
            S_ref, z_ref = brute_force_state_loops(k, v, grid)
            for S_got, z_got, what in ((S_bc, z_bc, "block_causal"), (S_tc, z_tc, "token_causal")):
                np.testing.assert_allclose(S_got[b, h], S_ref, rtol=1e-10, atol=1e-12,
                                           err_msg=f"{what} final S " + where)
                np.testing.assert_allclose(z_got[b, h], z_ref, rtol=1e-12, atol=1e-13,
                                           err_msg=f"{what} final z " + where)


def check_axis_split():
    for d, split in load_axis_split().items():
        assert oracle.rope_axis_pairs(d) == split, d


def check_rotation_axes_and_frequencies():
    """Unit vectors in each pair, moved along one axis, turn by pos * omega_k."""
    for d, (pt, ph, pw) in load_axis_split().items():
        grid = (5, 6, 7)
        P = d // 2
        owner = ["t"] * pt + ["h"] * ph + ["w"] * pw
        local = list(range(pt)) + list(range(ph)) + list(range(pw))
        count = {"t": pt, "h": ph, "w": pw}
        for axis, coord in (("t", (3, 0, 0)), ("h", (0, 4, 0)), ("w", (0, 0, 5))):
            n = np.array([coord[0] * 42 + coord[1] * 7 + coord[2]])
            x = np.zeros((1, d))
            x[0, 0::2] = 1.0
            y = oracle.rope(x, n, grid)[0]
            for p in range(P):
                ang = math.atan2(y[2 * p + 1], y[2 * p])
                if owner[p] == axis:
                    pos = {"t": 3, "h": 4, "w": 5}[axis]
                    want = pos * 10000.0 ** (-2.0 * local[p] / (2 * count[axis]))
                    want = math.remainder(want, 2 * math.pi)
                else:
                    want = 0.0
                assert abs(ang - want) < 1e-12, (d, axis, p, ang, want)


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------

def test_worked_examples():
    check_worked_examples()


def test_brute_force_bidirectional():
    check_brute_force_bidirectional()


def test_brute_force_block_causal():
    check_brute_force_block_causal()


def test_brute_force_cross():
    check_brute_force_cross()


def test_cross_attention_closed_forms():
    """One key/value token: O_i = V_0 a/(a + eps), a = relu(q_i).relu(k_0); none: zeros."""
    rng = np.random.default_rng(30)
    Q = rng.standard_normal((50, 16))
    K = np.abs(rng.standard_normal((1, 16)))
    V = rng.standard_normal((1, 16))
    got = oracle.cross_attention_head(Q, K, V, 1e-3)
    a = np.maximum(Q, 0) @ K[0]
    want = np.where((np.maximum(Q, 0) > 0).any(axis=1)[:, None], a[:, None] * V[0] / (a[:, None] + 1e-3), 0.0)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)
    assert not np.any(oracle.cross_attention_head(Q, K[:0], V[:0], 1e-6))
    # text-token order does not matter
    K2, V2 = rng.standard_normal((2, 40, 16))
    perm = rng.permutation(40)
    np.testing.assert_allclose(oracle.cross_attention_head(Q, K2, V2, 1e-6),
                               oracle.cross_attention_head(Q, K2[perm], V2[perm], 1e-6), rtol=1e-12)


def test_brute_force_token_causal():
    check_brute_force_token_causal()


def test_token_causal_identities():
    """Block size 1 is token-causal; the last row sees everything; carry + offset resume."""
    Q, K, V = rand((3, 40, 8), 44)
    grid = (4, 2, 5)
    o_tc, S_tc, z_tc = oracle.token_causal_head(Q, K, V, grid, 1e-6)
    o_bc, S_bc, z_bc = oracle.block_causal_head(Q, K, V, grid, 1, 1e-6)
    np.testing.assert_allclose(o_tc, o_bc, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S_tc, S_bc, rtol=1e-12, atol=1e-13)
    bi = oracle.bidirectional_head(Q, K, V, grid, 1e-6)
    np.testing.assert_allclose(o_tc[-1], bi[-1], rtol=1e-12, atol=1e-14)
    S_all, z_all = oracle.state(K, V, grid)
    np.testing.assert_allclose(S_tc, S_all, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z_tc, z_all, rtol=1e-12)
    m = 23
    o1, S1, z1 = oracle.token_causal_head(Q[:m], K[:m], V[:m], grid, 1e-6)
    o2, S2, z2 = oracle.token_causal_head(Q[m:], K[m:], V[m:], grid, 1e-6, n0=m, carry=(S1, z1))
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_tc, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2, S_tc, rtol=1e-12, atol=1e-13)


def test_batched_wrappers():
    check_batched_wrappers()


def test_axis_split():
    check_axis_split()


def test_rotation_axes_and_frequencies():
    check_rotation_axes_and_frequencies()


def test_linear_form_equals_weights_form():
    """Reassociation: O(N) state form == O(N^2) explicit-weights form."""
    for N, d, grid, seed in [(256, 32, None, 11), (200, 64, (3, 8, 9), 12), (97, 128, (2, 7, 7), 13)]:
        Q, K, V = rand((3, N, d), seed)
        for eps in (0.0, 1e-6):
            a = oracle.bidirectional_head(Q, K, V, grid, eps)
            b = orc.weights_form_head(Q, K, V, grid, eps)
            np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)
            for L in (1, 17, 64):
                a, _, _ = oracle.block_causal_head(Q, K, V, grid, L, eps)
                b = orc.weights_form_head(Q, K, V, grid, eps, block_tokens=L)
                np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)


def test_rotation_norm_and_origin():
    x = rand((50, 64), 20)
    n = np.arange(1000, 1050)
    y = oracle.rope(x, n, (30, 23, 40))
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    z = oracle.rope(x[:1], np.array([0]), (30, 23, 40))
    np.testing.assert_array_equal(z, x[:1])


def test_rotation_relative_position():
    """RoPE(x, p) . RoPE(y, p') depends only on p - p' (shift all three axes)."""
    grid = (40, 23, 40)
    enc = lambda t, h, w: np.array([t * 23 * 40 + h * 40 + w])  # noqa: E731
    rng = np.random.default_rng(21)
    for d in (32, 64, 128):
        for _ in range(5):
            x, y = rng.standard_normal((2, 1, d))
            p = rng.integers(0, [20, 11, 20])
            pp = rng.integers(0, [20, 11, 20])
            s = rng.integers(0, [20, 12, 20])
            a = oracle.rope(x, enc(*p), grid) @ oracle.rope(y, enc(*pp), grid).T
            b = oracle.rope(x, enc(*(p + s)), grid) @ oracle.rope(y, enc(*(pp + s)), grid).T
            np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)


def test_constant_v_is_reproduced():
    """No RoPE, eps = 0: every weight sum cancels, O_i = c (rows with phi Q_i != 0)."""
    Q, K = rand((2, 300, 64), 30)
    c = rand((64,), 31)
    V = np.tile(c, (300, 1))
    O = oracle.bidirectional_head(Q, K, V, None, 0.0)
    live = (Q > 0).any(axis=1)
    np.testing.assert_allclose(O[live], np.tile(c, (live.sum(), 1)), rtol=1e-12, atol=1e-13)


def test_permutation_equivariance_without_rope():
    Q, K, V = rand((3, 128, 32), 40)
    perm = np.random.default_rng(41).permutation(128)
    a = oracle.bidirectional_head(Q, K, V, None, 1e-6)
    b = oracle.bidirectional_head(Q[perm], K[perm], V[perm], None, 1e-6)
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-14)


def test_scaling():
    Q, K, V = rand((3, 100, 64), 50)
    g = (4, 5, 5)
    a = oracle.bidirectional_head(Q, K, V, g, 0.0)
    np.testing.assert_allclose(oracle.bidirectional_head(3.0 * Q, 0.5 * K, V, g, 0.0), a, rtol=1e-11)
    np.testing.assert_allclose(oracle.bidirectional_head(Q, K, -2.5 * V, g, 0.0), -2.5 * a, rtol=1e-11)


def test_zero_query_rows_are_exactly_zero():
    Q, K, V = rand((3, 64, 32), 60)
    Q[::3] = -np.abs(Q[::3])
    for eps in (0.0, 1e-6):
        O = oracle.bidirectional_head(Q, K, V, (2, 4, 8), eps)
        assert np.all(O[::3] == 0.0)
        assert np.all(np.isfinite(O))


def test_denominator_nonnegative():
    Q, K, V = rand((3, 200, 64), 70)
    _, z = oracle.state(K, V, (5, 5, 8))
    assert np.all(z >= 0)
    assert np.all(oracle.phi(Q) @ z >= 0)


def test_block_causal_last_block_and_carry_equal_bidirectional():
    Q, K, V = rand((3, 250, 32), 80)
    g = (10, 5, 5)
    full = oracle.bidirectional_head(Q, K, V, g, 1e-6)
    O, S, z = oracle.block_causal_head(Q, K, V, g, 60, 1e-6)
    np.testing.assert_allclose(O[240:], full[240:], rtol=1e-11, atol=1e-14)
    S_ref, z_ref = oracle.state(K, V, g)
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(z, z_ref, rtol=1e-12)
    O1, _, _ = oracle.block_causal_head(Q, K, V, g, 250, 1e-6)
    np.testing.assert_allclose(O1, full, rtol=1e-12, atol=1e-15)


def test_block_causal_resume_from_carry():
    Q, K, V = rand((3, 200, 32), 90)
    g = (8, 5, 5)
    O, S, z = oracle.block_causal_head(Q, K, V, g, 50, 1e-6)
    _, S1, z1 = oracle.block_causal_head(Q[:100], K[:100], V[:100], g, 50, 1e-6)
    # second half continues at global positions 100.., so shift via a padded call
    Oc = np.zeros((200, 32))
    Sc, zc = S1, z1
    for b0 in (100, 150):
        Sb, zb = oracle.state(K[b0:b0 + 50], V[b0:b0 + 50], g, n0=b0)
        Sc, zc = Sc + Sb, zc + zb
        Oc[b0:b0 + 50] = oracle.apply(Q[b0:b0 + 50], Sc, zc, g, 1e-6, n0=b0)
    np.testing.assert_allclose(Oc[100:], O[100:], rtol=1e-12, atol=1e-15)


def test_block_size_one_is_token_causal_eq3():
    """Eq. 3 literally (j <= i) is the block-causal mode with one token per block."""
    Q, K, V = rand((3, 20, 8), 100)
    ref = brute_force_loops(Q, K, V, (2, 2, 5), 1e-6, token_causal=True)
    got, _, _ = oracle.block_causal_head(Q, K, V, (2, 2, 5), 1, 1e-6)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_rel_row_error_metric():
    ref = np.array([[1.0, -2.0], [0.0, 0.0]])
    assert oracle.rel_row_error(ref, ref) == 0.0
    assert oracle.rel_row_error(ref + [[0.02, 0.0], [0.0, 0.0]], ref) == pytest.approx(0.01)
    assert oracle.rel_row_error(ref + [[0.0, 0.0], [1e-30, 0.0]], ref) == float("inf")
    assert oracle.rel_row_error(ref * np.nan, ref) == float("inf")


# ---------------------------------------------------------------------------
# planted mistakes: every one must make some pin fail
# ---------------------------------------------------------------------------

def _mut_rope_sign(x, n, grid):
    y = _ORIG["rope"](x, n, grid)
    if grid is not None:
        xx = np.asarray(x, dtype=np.float64)
        ang = orc.rope_angles(n, grid, xx.shape[-1])
        c, s = np.cos(ang), -np.sin(ang)
        y = np.empty_like(xx)
        y[:, 0::2] = xx[:, 0::2] * c - xx[:, 1::2] * s
        y[:, 1::2] = xx[:, 0::2] * s + xx[:, 1::2] * c
    return y


def _mut_rope_half(x, n, grid):
    xx = np.asarray(x, dtype=np.float64)
    if grid is None:
        return xx.copy()
    d = xx.shape[1]
    perm = np.concatenate([np.arange(0, d // 2), np.arange(d // 2, d)]).reshape(2, -1).T.ravel()
    inv = np.argsort(perm)
    return _ORIG["rope"](xx[:, perm], n, grid)[:, inv]


def _mut_axis_swap(d):
    pt, ph, pw = _ORIG["rope_axis_pairs"](d)
    return (pw, ph, pt)


def _mut_positions_w_major(n, grid):
    gt, gh, gw = grid
    n = np.asarray(n, dtype=np.int64)
    return n % gt, (n // gt) % gh, n // (gt * gh)


def _mut_state_rotated_z(K, V, grid, n0=0):
    S, _ = _ORIG["state"](K, V, grid, n0)
    k = orc.phi(K)
    z = orc.rope(k, np.arange(n0, n0 + len(k)), grid).sum(axis=0)
    return S, z


def _mut_state_no_relu(K, V, grid, n0=0):
    K = np.asarray(K, dtype=np.float64)
    n = np.arange(n0, n0 + K.shape[0])
    return orc.rope(K, n, grid).T @ np.asarray(V, dtype=np.float64), orc.phi(K).sum(axis=0)


def _mut_state_rope_before_relu(K, V, grid, n0=0):
    K = np.asarray(K, dtype=np.float64)
    n = np.arange(n0, n0 + K.shape[0])
    kr = orc.phi(orc.rope(K, n, grid))
    return kr.T @ np.asarray(V, dtype=np.float64), orc.phi(K).sum(axis=0)


def _mut_apply_transposed(Q, S, z, grid, eps, n0=0):
    return _ORIG["apply"](Q, np.asarray(S).T, z, grid, eps, n0)


def _mut_apply_eps_numerator(Q, S, z, grid, eps, n0=0):
    return _ORIG["apply"](Q, np.asarray(S) + 1e-3, z, grid, eps, n0)


def _mut_block_exclusive(Q, K, V, grid, block_tokens, eps, carry=None):
    N, d = np.shape(Q)
    S, z = np.zeros((d, d)), np.zeros(d)
    out = np.zeros((N, d))
    for b0 in range(0, N, block_tokens):
        b1 = min(b0 + block_tokens, N)
        Sb, zb = orc.state(K[b0:b1], V[b0:b1], grid, n0=b0)
        out[b0:b1] = orc.apply(Q[b0:b1], S, z, grid, eps, n0=b0)
        S, z = S + Sb, z + zb
    return out, S, z


def _mut_token_exclusive(Q, K, V, grid, eps, n0=0, carry=None):
    N, d = np.shape(Q)
    S, z = np.zeros((d, d)), np.zeros(d)
    q, k = orc.phi(Q), orc.phi(K)
    n = np.arange(n0, n0 + N)
    qr, kr = orc.rope(q, n, grid), orc.rope(k, n, grid)
    out = np.zeros((N, d))
    for i in range(N):
        if np.any(q[i] > 0.0):
            out[i] = (qr[i] @ S) / (q[i] @ z + eps)
        S = S + np.outer(kr[i], np.asarray(V[i], dtype=np.float64))
        z = z + k[i]
    return out, S, z


def _mut_freq(n, grid, d):
    ang = _ORIG["rope_angles"](n, grid, d)
    return ang * 1.0001


def _mut_wrap_bidir_eps_default(Q, K, V, grid=None, eps=1e-6):
    return _ORIG["bidirectional"](Q, K, V, grid)


def _mut_wrap_block_eps_default(Q, K, V, grid, block_tokens, eps=1e-6):
    return _ORIG["block_causal"](Q, K, V, grid, block_tokens)


def _mut_wrap_token_no_grid(Q, K, V, grid=None, eps=1e-6):
    return _ORIG["token_causal"](Q, K, V, None, eps)


def _mut_wrap_cross_k_for_v(Q, K, V, eps=1e-6):
    return _ORIG["cross_attention"](Q, K, K, eps)


def _mut_wrap_bidir_head_shift(Q, K, V, grid=None, eps=1e-6):
    """Slice (b, h) reads K and V of head h + 1: an indexing slip in the loop."""
    B, H, N, d = np.shape(Q)
    out = np.empty((B, H, N, d))
    for b in range(B):
        for h in range(H):
            hh = (h + 1) % H
            out[b, h] = orc.bidirectional_head(Q[b, h], K[b, hh], V[b, hh], grid, eps)
    return out


def _mut_wrap_block_carry_batch0(Q, K, V, grid, block_tokens, eps=1e-6):
    """Every batch element reports the carry of batch element 0."""
    out, S, z = _ORIG["block_causal"](Q, K, V, grid, block_tokens, eps)
    return out, np.broadcast_to(S[:1], S.shape).copy(), np.broadcast_to(z[:1], z.shape).copy()


_ORIG = {}
MUTANTS = [
    ("rope", _mut_rope_sign),
    ("rope", _mut_rope_half),
    ("rope_axis_pairs", _mut_axis_swap),
    ("grid_positions", _mut_positions_w_major),
    ("state", _mut_state_rotated_z),
    ("state", _mut_state_no_relu),
    ("state", _mut_state_rope_before_relu),
    ("apply", _mut_apply_transposed),
    ("apply", _mut_apply_eps_numerator),
    ("block_causal_head", _mut_block_exclusive),
    ("rope_angles", _mut_freq),
    ("token_causal_head", _mut_token_exclusive),
    ("bidirectional", _mut_wrap_bidir_eps_default),
    ("block_causal", _mut_wrap_block_eps_default),
    ("token_causal", _mut_wrap_token_no_grid),
    ("cross_attention", _mut_wrap_cross_k_for_v),
    ("bidirectional", _mut_wrap_bidir_head_shift),
    ("block_causal", _mut_wrap_block_carry_batch0),
]
PIN_CHECKS = [check_worked_examples, check_axis_split, check_rotation_axes_and_frequencies,
              check_brute_force_bidirectional, check_brute_force_block_causal, check_brute_force_cross,
              check_brute_force_token_causal, check_batched_wrappers]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_pins_catch_planted_mistakes(monkeypatch, name, mutant):
    for key in ("rope", "rope_axis_pairs", "state", "apply", "rope_angles", "bidirectional",
                "block_causal", "token_causal", "cross_attention"):
        _ORIG[key] = getattr(orc, key)
    monkeypatch.setattr(orc, name, mutant)
    # the package namespace re-exports the functions; patch it too
    monkeypatch.setattr(oracle, name, mutant, raising=False)
    failed = []
    for check in PIN_CHECKS:
        try:
            check()
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {mutant.__name__}"


def test_zero_denominator_rows():
    """eps = 0 and a live query whose channels meet no key mass: the IEEE quotient.

    With no keys at all, S = 0 and z = 0: a live row is 0/0 = NaN in every
    channel, a dead row (relu(Q_i) = 0) is exactly zero.  With keys that are
    zero on every channel where the query is positive, the denominator is 0
    while RoPE can still give the numerator a non-zero value (+-inf there).
    """
    rng = np.random.default_rng(62)
    Q = rng.standard_normal((9, 8))
    Q[3] = -np.abs(Q[3])  # a dead row
    got = oracle.cross_attention_head(Q, np.zeros((0, 8)), np.zeros((0, 8)), 0.0)
    live = (Q > 0).any(axis=1)
    assert np.isnan(got[live]).all() and not np.any(got[~live])
    # d = 8 on a 1x2x2 grid: pair 3 (channels 6, 7) turns with w by angle w.  The
    # query is positive on channel 6 only, the keys on channel 7 only, so z is
    # zero where the query lives, but keys one w step away contribute -+sin(1)
    Qp = np.zeros((4, 8))
    Qp[:, 6] = 1.0
    Kp = np.zeros((4, 8))
    Kp[:, 7] = 1.0
    Vp = np.ones((4, 8))
    out = oracle.bidirectional_head(Qp, Kp, Vp, (1, 2, 2), 0.0)
    assert np.isinf(out).all()
    assert (np.sign(out[:, 0]) == [-1, 1, -1, 1]).all()
