"""Pins of the fp64 oracle against facts outside itself (CPU only).

Each test names the fact it checks: a closed form, a special case that
reduces to a library routine, finite differences, an invariant of the
mathematics, or a statistical property of the dropout generator.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _mask(N, causal):
    return np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 4), (7, 3), (33, 8)])
def test_softmax_rows_sum_to_one(N, d, causal):
    """Softmax rows are normalised ("Tiling": the normaliser l)."""
    q, k = _rand((N, d), 1), _rand((N, d), 2)
    P, Pd = oracle.probs(q, k, 0.7, causal)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(P, Pd)  # p = 0 drops nothing
    if causal:
        assert np.all(P[~_mask(N, True)] == 0.0)
    # V = all ones and p = 0 -> every output is exactly a sum of probabilities = 1.
    v = np.ones((1, 1, N, d))
    o, _ = oracle.fwd(q[None, None], k[None, None], v, 0.7, causal)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_values(causal):
    """Q = 0: every score is 0, so O_i is the mean of the visible V rows and
    LSE_i = ln(number of visible keys)."""
    N, d = 37, 5
    q = np.zeros((1, 1, N, d))
    k, v = _rand((1, 1, N, d), 3), _rand((1, 1, N, d), 4)
    o, lse = oracle.fwd(q, k, v, 0.3, causal)
    vv = v[0, 0]
    if causal:
        counts = np.arange(1, N + 1)
        expect = np.cumsum(vv, axis=0) / counts[:, None]
    else:
        counts = np.full(N, N)
        expect = np.broadcast_to(vv.mean(axis=0), (N, d))
    np.testing.assert_allclose(o[0, 0], expect, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(counts), rtol=0, atol=1e-13)


def test_single_key_returns_value():
    """N = 1: the only probability is exp(0) = 1, so O = V, LSE = scale q.k,
    dV = dO and dQ = dK = 0."""
    d = 6
    q, k, v, do = (_rand((2, 3, 1, d), s) for s in range(4))
    for p in (0.0,):
        o, lse = oracle.fwd(q, k, v, 0.41, causal=True, dropout_p=p)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse[..., 0], 0.41 * np.sum(q * k, axis=-1)[..., 0],
                                   rtol=0, atol=1e-15)
    dq, dk, dv, o2, _ = oracle.bwd(q, k, v, do, 0.41, causal=False)
    np.testing.assert_array_equal(dv, do)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_array_equal(o2, v)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_one_hot_values_select_probabilities(causal, p):
    """V = [I_N | 0] with d >= N: O[:, :N] is exactly the (dropped) probability
    matrix; with p = 0 it equals scipy's softmax of the masked scores."""
    N, d = 9, 12
    q, k = _rand((N, d), 5), _rand((N, d), 6)
    v = np.zeros((N, d))
    v[:, :N] = np.eye(N)
    o, _ = oracle.fwd(q[None, None], k[None, None], v[None, None], 0.5, causal, p, seed=77)
    _, Pd = oracle.probs(q, k, 0.5, causal, p, seed=77)
    np.testing.assert_allclose(o[0, 0, :, :N], Pd, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(o[0, 0, :, N:], 0.0)
    if p == 0.0:
        s = 0.5 * q @ k.T
        s[~_mask(N, causal)] = -np.inf
        np.testing.assert_allclose(Pd, scipy.special.softmax(s, axis=1), rtol=0, atol=1e-14)


# ------------------------------------------------------- library routine

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 8), (17, 8), (64, 16), (130, 32)])
def test_matches_torch_cpu_fp64_sdpa_and_autograd(N, d, causal):
    """p = 0: the whole forward and backward against PyTorch's CPU float64
    scaled_dot_product_attention and autograd (the library entry point named
    on the chipfoundryservices page, "Adoption")."""
    B, H = 2, 3
    q, k, v, do = (_rand((B, H, N, d), 10 + s) for s in range(4))
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.fwd(q, k, v, scale, causal)
    dq, dk, dv, o2, lse2 = oracle.bwd(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           scale=scale)
    ref.backward(torch.tensor(do))
    s = scale * torch.tensor(q) @ torch.tensor(k).transpose(-1, -2)
    if causal:
        s = s.masked_fill(~torch.tensor(_mask(N, True)), float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    tol = dict(rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, ref.detach().numpy(), **tol)
    np.testing.assert_allclose(o2, ref.detach().numpy(), **tol)
    np.testing.assert_allclose(lse, ref_lse, **tol)
    np.testing.assert_allclose(lse2, ref_lse, **tol)
    np.testing.assert_allclose(dq, tq.grad.numpy(), **tol)
    np.testing.assert_allclose(dk, tk.grad.numpy(), **tol)
    np.testing.assert_allclose(dv, tv.grad.numpy(), **tol)


# ---------------------------------------------------- finite differences

def _loss(q, k, v, do, scale, causal, p, seed):
    o, _ = oracle.fwd(q, k, v, scale, causal, p, seed)
    return float(np.sum(o * do))


@pytest.mark.parametrize("p", [0.0, 0.5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 1), (2, 2), (3, 4), (5, 2), (8, 4)])
def test_gradients_match_finite_differences(N, d, causal, p):
    """Analytic dQ, dK, dV agree with central differences of L = sum(O * dO);
    the dropout mask is fixed by the seed, so L is smooth."""
    seed = 1234
    scale = 0.8
    q, k, v, do = (_rand((1, 1, N, d), 20 + s) for s in range(4))
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, do, scale, causal, p, seed)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, scale, causal, p, seed)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, scale, causal, p, seed)
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7, err_msg=name)


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("p", [0.0, 0.2])
@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sum_identities(causal, p):
    """sum_j dK_j = 0 (each row of dS sums to zero); with p = 0 also
    sum_j dV_j = sum_i dO_i (each row of P sums to one)."""
    N, d = 23, 6
    q, k, v, do = (_rand((1, 2, N, d), 30 + s) for s in range(4))
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, do, 0.6, causal, p, seed=5)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    if p == 0.0:
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    """K -> K + 1 c^T leaves O unchanged and shifts LSE_i by scale q_i . c."""
    N, d = 19, 7
    q, k, v = (_rand((1, 1, N, d), 40 + s) for s in range(3))
    c = _rand((d,), 44)
    scale = 0.45
    o1, l1 = oracle.fwd(q, k, v, scale, causal)
    o2, l2 = oracle.fwd(q, k + c, v, scale, causal)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, scale * (q[0, 0] @ c)[None, None], atol=1e-12)


def test_joint_key_value_permutation_invariance():
    """Non-causal: permuting the rows of K and V together leaves O and LSE."""
    N, d = 21, 5
    q, k, v = (_rand((1, 1, N, d), 50 + s) for s in range(3))
    perm = np.random.default_rng(51).permutation(N)
    o1, l1 = oracle.fwd(q, k, v, 0.5, False)
    o2, l2 = oracle.fwd(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_bounds_hull_and_first_row(causal):
    """m_i <= LSE_i <= m_i + ln n_i; O_i lies in the coordinate-wise hull of
    the visible V rows (p = 0); causal row 0 is O_0 = V_0, LSE_0 = s_00."""
    N, d = 31, 4
    q, k, v = (_rand((1, 1, N, d), 60 + s) for s in range(3))
    scale = 1.3
    o, lse = oracle.fwd(q, k, v, scale, causal)
    s = scale * q[0, 0] @ k[0, 0].T
    vis = _mask(N, causal)
    s_masked = np.where(vis, s, -np.inf)
    m = s_masked.max(axis=1)
    n = vis.sum(axis=1)
    assert np.all(lse[0, 0] >= m - 1e-12)
    assert np.all(lse[0, 0] <= m + np.log(n) + 1e-12)
    for i in range(N):
        rows = v[0, 0][vis[i]]
        assert np.all(o[0, 0, i] >= rows.min(axis=0) - 1e-12)
        assert np.all(o[0, 0, i] <= rows.max(axis=0) + 1e-12)
    if causal:
        np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])
        np.testing.assert_allclose(lse[0, 0, 0], s[0, 0], atol=1e-15)


def test_selected_rows_equal_full_evaluation():
    """Evaluating a subset of rows gives the same values as all rows (the
    forward has no coupling between rows)."""
    N, d = 40, 8
    q, k, v = (_rand((2, 2, N, d), 70 + s) for s in range(3))
    o, lse = oracle.fwd(q, k, v, 0.35, True, 0.25, seed=9)
    rows = [0, 5, 39, 17]
    orow, lrow = oracle.fwd_rows(q, k, v, 1, 1, rows, 0.35, True, 0.25, seed=9)
    np.testing.assert_array_equal(orow, o[1, 1, rows])
    np.testing.assert_array_equal(lrow, lse[1, 1, rows])


# --------------------------------------------------------------- dropout

def test_dropout_threshold_and_scale():
    """T = round(p * 65536) and c = float(1 / (1 - p))."""
    assert oracle.drop_threshold(0.1) == 6554
    assert oracle.drop_threshold(0.0) == 0
    assert oracle.drop_threshold(0.5) == 32768
    assert oracle.keep_scale(0.1) == float(np.float32(1.0 / 0.9))
    assert oracle.keep_scale(0.5) == 2.0


def test_dropout_kept_fraction_within_five_sigma():
    """The kept fraction over >= 1e7 draws is 1 - T/65536 within 5 sigma."""
    N, p = 1024, 0.1
    kept = 0
    total = 0
    for b, h in [(0, 0), (1, 3), (2, 7), (3, 31), (0, 9), (5, 1), (2, 2), (7, 12), (1, 1), (6, 6)]:
        m = oracle.dropout_mask(N, p, 0xABCDEF0123456789, b, h)
        kept += int(m.sum())
        total += m.size
    assert total >= 10_000_000
    q = 1.0 - oracle.drop_threshold(p) / 65536.0
    sigma = math.sqrt(q * (1 - q) / total)
    assert abs(kept / total - q) < 5 * sigma


def test_dropout_mask_depends_on_every_key_field():
    """Changing the seed, b, h or the row changes the mask."""
    N, p = 64, 0.5
    base = oracle.dropout_mask(N, p, 1, 0, 0)
    for other in (oracle.dropout_mask(N, p, 2, 0, 0), oracle.dropout_mask(N, p, 1 << 40, 0, 0),
                  oracle.dropout_mask(N, p, 1, 1, 0), oracle.dropout_mask(N, p, 1, 0, 1)):
        frac_same = float((other == base).mean())
        assert 0.45 < frac_same < 0.55
    rows_same = float((base[1:] == base[:-1]).mean())
    cols_same = float((base[:, 1:] == base[:, :-1]).mean())
    assert 0.45 < rows_same < 0.55 and 0.45 < cols_same < 0.55


def test_dropout_neighbour_pairs_are_independent():
    """2x2 chi-square on horizontally and vertically adjacent keep bits."""
    N, p = 512, 0.3
    m = oracle.dropout_mask(N, p, 0x1234, 2, 5).astype(np.int64)
    for a, b in ((m[:, :-1], m[:, 1:]), (m[:-1, :], m[1:, :])):
        table = np.zeros((2, 2))
        for x in (0, 1):
            for y in (0, 1):
                table[x, y] = np.sum((a == x) & (b == y))
        chi2 = scipy.stats.chi2_contingency(table, correction=False)[0]
        assert chi2 < 20.0  # 1 d.o.f.; p-value ~ 1e-5


def test_dropout_is_unbiased():
    """E over seeds of O with dropout equals O without dropout."""
    N, d, p = 12, 3, 0.4
    q, k, v = (_rand((1, 1, N, d), 80 + s) for s in range(3))
    o_ref, _ = oracle.fwd(q, k, v, 0.5, True)
    acc = np.zeros_like(o_ref)
    n = 400
    for s in range(n):
        o, _ = oracle.fwd(q, k, v, 0.5, True, p, seed=s * 7919 + 1)
        acc += o
    mean = acc / n
    # Per-element standard error is below ~0.1 for these sizes.
    assert np.abs(mean - o_ref).max() < 0.25
    assert np.abs(mean - o_ref).mean() < 0.05


def test_dropout_zero_probability_is_identity():
    """p = 0 keeps everything and evaluates no generator."""
    m = oracle.dropout_mask(50, 0.0, 99, 0, 0)
    assert m.all()


# ----------------------------------------------------------- the generator

def test_philox_output_bits_are_balanced_and_avalanche():
    """Each output bit is 1 about half the time, and flipping one counter or
    key bit flips about half of the 128 output bits."""
    rng = np.random.default_rng(90)
    flips = []
    ones = np.zeros(128)
    n = 2000
    for _ in range(n):
        ctr = rng.integers(0, 2**32, size=4, dtype=np.uint64).astype(np.uint32)
        key = rng.integers(0, 2**32, size=2, dtype=np.uint64).astype(np.uint32)
        out = oracle.philox4x32_10(ctr, key)
        bits = np.unpackbits(out.view(np.uint8))
        ones += bits
        which = rng.integers(0, 6 * 32)
        c2, k2 = ctr.copy(), key.copy()
        if which < 128:
            c2[which // 32] ^= np.uint32(1 << (which % 32))
        else:
            k2[(which - 128) // 32] ^= np.uint32(1 << ((which - 128) % 32))
        out2 = oracle.philox4x32_10(c2, k2)
        flips.append(int(np.unpackbits((out ^ out2).view(np.uint8)).sum()))
    assert np.all(np.abs(ones / n - 0.5) < 0.06)
    assert abs(np.mean(flips) - 64) < 1.0
    assert min(flips) > 30


def test_philox_distinct_counters_distinct_outputs():
    """A keyed bijection: distinct counters never collide."""
    outs = set()
    for c0 in range(2000):
        out = oracle.philox4x32_10([c0, 3, 0, 0], [11, 22])
        outs.add(tuple(int(x) for x in out))
    assert len(outs) == 2000


def test_mask_uses_eight_lanes_of_one_block():
    """Columns 8c..8c+7 of a row read the eight 16-bit lanes of one block,
    counter (c, row, h, b): the mask equals lane >= T lane by lane."""
    seed, b, h, row = 0x0123456789ABCDEF, 3, 5, 17
    p = 0.37
    T = oracle.drop_threshold(p)
    m = oracle.dropout_mask(32, p, seed, b, h)
    for c in range(4):
        out = oracle.philox4x32_10([c, row, h, b], [seed & 0xFFFFFFFF, seed >> 32])
        lanes = []
        for w in out:
            lanes += [int(w) & 0xFFFF, int(w) >> 16]
        expect = [int(x >= T) for x in lanes]
        assert list(m[row, 8 * c:8 * c + 8]) == expect


# ------------------------------------------- queries and keys of two lengths

def _cross_mask(Nq, Nk, causal):
    """Visible (i, j): every key, or (causal) j <= i + (Nk - Nq)."""
    if not causal:
        return np.ones((Nq, Nk), dtype=bool)
    return np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)


@pytest.mark.parametrize("Nq,Nk", [(1, 9), (5, 23), (23, 5), (16, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_cross_matches_torch_cpu_fp64_sdpa(Nq, Nk, causal):
    """Nq != Nk: torch's fp64 scaled_dot_product_attention with the same
    visibility as an explicit mask (rows with no visible key are compared
    through the closed form O = 0, LSE = -inf instead)."""
    d, scale = 6, 0.45
    q, k, v = _rand((1, 2, Nq, d), 50), _rand((1, 2, Nk, d), 51), _rand((1, 2, Nk, d), 52)
    o, lse = oracle.fwd(q, k, v, scale, causal)
    m = _cross_mask(Nq, Nk, causal)
    live = m.any(axis=1)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(m), scale=scale).numpy()
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    s = np.where(m, s, -np.inf)
    with np.errstate(divide="ignore"):
        ref_lse = scipy.special.logsumexp(s, axis=-1)
    np.testing.assert_allclose(o[:, :, live], ref[:, :, live], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[:, :, live], ref_lse[:, :, live], rtol=1e-12, atol=1e-13)
    assert np.all(o[:, :, ~live] == 0.0) and np.all(lse[:, :, ~live] == -np.inf)


@pytest.mark.parametrize("Nq,Nk", [(1, 40), (7, 40), (40, 40)])
def test_cross_causal_is_the_tail_of_the_square_problem(Nq, Nk):
    """Causal with the last query aligned to the last key: the Nq queries
    see exactly what the last Nq rows of the square problem over the Nk
    keys see (decoding), so their O and LSE are those rows."""
    d, scale = 5, 0.6
    qf = _rand((1, 1, Nk, d), 60)
    k, v = _rand((1, 1, Nk, d), 61), _rand((1, 1, Nk, d), 62)
    o_sq, l_sq = oracle.fwd(qf, k, v, scale, True)
    o, lse = oracle.fwd(np.ascontiguousarray(qf[:, :, Nk - Nq:]), k, v, scale, True)
    np.testing.assert_allclose(o, o_sq[:, :, Nk - Nq:], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, l_sq[:, :, Nk - Nq:], rtol=0, atol=1e-14)


@pytest.mark.parametrize("Nq,Nk", [(9, 30), (30, 9)])
def test_cross_zero_query_gives_mean_of_visible_values(Nq, Nk):
    """Q = 0, causal: O_i is the mean of V_0 .. V_{i + Nk - Nq} and LSE_i the
    log of their count; queries with no visible key give O = 0, LSE = -inf."""
    d = 4
    q = np.zeros((1, 1, Nq, d))
    k, v = _rand((1, 1, Nk, d), 63), _rand((1, 1, Nk, d), 64)
    o, lse = oracle.fwd(q, k, v, 0.5, True)
    for i in range(Nq):
        n = i + 1 + Nk - Nq
        if n <= 0:
            assert np.all(o[0, 0, i] == 0.0) and lse[0, 0, i] == -np.inf
        else:
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[0, 0, i] - math.log(n)) < 1e-13


def test_cross_dropout_uses_the_square_counters():
    """With dropout, entry (i, j) of an Nq x Nk problem is kept iff entry
    (i, j) of the plane's keep mask is: one-hot V (d >= Nk) exposes the
    dropped, rescaled probabilities, which must be the undropped ones times
    mask times c."""
    Nq, Nk, d, p, seed = 6, 11, 12, 0.4, 0xABCDEF
    q, k = _rand((1, 1, Nq, d), 65), _rand((1, 1, Nk, d), 66)
    v = np.zeros((1, 1, Nk, d))
    v[0, 0, :, :Nk] = np.eye(Nk)
    pd, _ = oracle.fwd(q, k, v, 0.8, True, p, seed)
    prob, _ = oracle.fwd(q, k, v, 0.8, True, 0.0, seed)
    keep = oracle.dropout_mask(max(Nq, Nk), p, seed, 0, 0)[:Nq, :Nk]
    c = oracle.keep_scale(p)
    np.testing.assert_allclose(pd[0, 0, :, :Nk], prob[0, 0, :, :Nk] * keep * c, rtol=0, atol=1e-15)


@pytest.mark.parametrize("p", [0.0, 0.5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,d", [(1, 3, 2), (4, 2, 3), (3, 6, 2)])
def test_cross_gradients_match_finite_differences(Nq, Nk, d, causal, p):
    """Nq != Nk: analytic dQ, dK, dV agree with central differences of
    L = sum(O * dO) (rows with no visible key contribute nothing)."""
    seed, scale, eps = 77, 0.7, 1e-6
    q, do = _rand((1, 1, Nq, d), 70), _rand((1, 1, Nq, d), 71)
    k, v = _rand((1, 1, Nk, d), 72), _rand((1, 1, Nk, d), 73)
    dq, dk, dv, o, lse = oracle.bwd(q, k, v, do, scale, causal, p, seed)
    o_f, lse_f = oracle.fwd(q, k, v, scale, causal, p, seed)
    np.testing.assert_array_equal(o, o_f)
    np.testing.assert_array_equal(lse, lse_f)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args[name] = xp
            lp = float(np.sum(oracle.fwd(args["q"], args["k"], args["v"], scale, causal, p, seed)[0] * do))
            args[name] = xm
            lm = float(np.sum(oracle.fwd(args["q"], args["k"], args["v"], scale, causal, p, seed)[0] * do))
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("Nq,Nk", [(5, 23), (23, 5)])
@pytest.mark.parametrize("causal", [False, True])
def test_cross_gradients_match_torch_fp64_autograd(Nq, Nk, causal):
    """Nq != Nk: torch's fp64 SDPA with the same visibility, differentiated by
    autograd (rows with no visible key are left out of the loss)."""
    d, scale = 6, 0.45
    q, do = _rand((1, 2, Nq, d), 80), _rand((1, 2, Nq, d), 81)
    k, v = _rand((1, 2, Nk, d), 82), _rand((1, 2, Nk, d), 83)
    m = _cross_mask(Nq, Nk, causal)
    live = m.any(axis=1)
    do_live = do * live[None, None, :, None]
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, do_live, scale, causal)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(m),
                                                         scale=scale)
    o = torch.where(torch.from_numpy(live)[None, None, :, None], o, torch.zeros_like(o))
    (o * torch.from_numpy(do_live)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-12, atol=1e-13)
