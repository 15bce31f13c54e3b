"""Pins for the fp64 oracle against what the pages and mathematics fix.

None of these re-types the oracle's own formulas: each check is a closed form,
an invariant, a printed value from the pages, a finite difference or an
independent library routine, chosen so that a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- worked example
def test_worked_example_matches_printed_values():
    """Video page, transcript 05:49-06:52: the online softmax on scores 1, 2, 3, 0."""
    with open(os.path.join(GOLDEN, "worked_example_online_softmax.json")) as f:
        g = json.load(f)
    m, l, steps = orc.online_softmax_row(g["scores"], g["blocks"])
    (m1, l1, _, _, bs1), (m2, l2, alpha, beta, bs2) = steps
    got = {
        "m1": m1,
        "exp_minus_1": math.exp(-1.0),  # the page's 0.368 is e^-1; checked against the block-one term below
        "l1": l1,
        "m2": m2,
        "alpha": alpha,
        "alpha_l1": alpha * l1,
        "block2_sum": bs2,
        "l2": l2,
        "textbook_denominator": float(np.exp(np.array(g["scores"])).sum()),
        "textbook_scaled": float(np.exp(np.array(g["scores"])).sum()) * math.exp(-3.0),
    }
    for key, spec in g["printed"].items():
        tol = 0.5 * 10 ** (-spec["decimals"]) + 1e-12
        assert abs(got[key] - spec["value"]) <= tol, (key, got[key], spec)
    # block one's sum scaled to its own max is e^-1 + e^0 (video page, transcript 05:49, worked example)
    assert abs(bs1 - (math.exp(-1) + 1.0)) < 1e-15
    # the online result equals the textbook softmax denominator scaled to the final max
    assert m == 3.0 and abs(l - float(np.exp(np.array(g["scores"]) - 3.0).sum())) < 1e-15
    # and the full attention row agrees: P from the forward oracle on a one-query problem
    q = np.array([[1.0, 0.0]])
    k = np.array([[1.0, 0.0], [2.0, 0.0], [3.0, 0.0], [0.0, 0.0]])
    v = np.arange(8, dtype=float).reshape(4, 2)
    o, lse, p = orc.forward_head(q, k, v, 1.0, False)
    assert abs(lse[0] - (3.0 + math.log(l))) < 1e-14
    textbook = np.exp(np.array(g["scores"])) / np.exp(np.array(g["scores"])).sum()
    np.testing.assert_allclose(p[0], textbook, rtol=0, atol=1e-15)
    o_online, lse_online = orc.online_attention_row(g["scores"], v, g["blocks"])
    np.testing.assert_allclose(o_online, o[0], rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    r = rng(1)
    q, k, v = r.standard_normal((3, 37, 8))
    _, _, p = orc.forward_head(q, k, v, 0.7, causal)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (p >= 0).all()
    if causal:
        assert (np.triu(p, 1) == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_give_mean_of_v(causal):
    """Q = 0 makes every allowed score equal: O_i is the mean of the allowed V rows."""
    r = rng(2)
    n, d = 23, 6
    q = np.zeros((n, d))
    k = r.standard_normal((n, d))
    v = r.standard_normal((n, d))
    o, lse, _ = orc.forward_head(q, k, v, 0.5, causal)
    for i in range(n):
        allowed = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[:allowed].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[i] - math.log(allowed)) < 1e-14
    # same with all K rows equal and a nonzero Q: constant score s per row
    k2 = np.tile(r.standard_normal((1, d)), (n, 1))
    q2 = r.standard_normal((n, d))
    o2, lse2, _ = orc.forward_head(q2, k2, v, 0.5, causal)
    for i in range(n):
        allowed = i + 1 if causal else n
        s = 0.5 * float(q2[i] @ k2[0])
        np.testing.assert_allclose(o2[i], v[:allowed].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse2[i] - (s + math.log(allowed))) < 1e-13


def test_one_hot_dominant_score_picks_v_row():
    """k_j = e_j, q_i = t e_{j*}: the score of key j* exceeds the others by scale*t >= 40."""
    r = rng(3)
    n, d = 8, 8
    k = np.eye(n, d)
    v = r.standard_normal((n, d))
    t, scale = 80.0, 0.5
    targets = r.integers(0, n, size=n)
    q = np.stack([t * np.eye(d)[j] for j in targets])
    o, lse, _ = orc.forward_head(q, k, v, scale, False)
    bound = (n - 1) * math.exp(-scale * t) * np.abs(v).max() * 2
    for i, j in enumerate(targets):
        assert np.abs(o[i] - v[j]).max() <= bound
        assert abs(lse[i] - scale * t) < 1e-12


def test_causal_row_zero_and_future_independence():
    r = rng(4)
    n, d = 16, 4
    q, k, v, do = r.standard_normal((4, n, d))
    scale = 0.3
    o, lse, _ = orc.forward_head(q, k, v, scale, True)
    np.testing.assert_array_equal(o[0], v[0])
    assert abs(lse[0] - scale * float(q[0] @ k[0])) < 1e-15
    dq, dk, dv, _ = orc.backward_head(q, k, v, do, scale, True)
    np.testing.assert_array_equal(dq[0], np.zeros(d))
    # changing keys/values after row i leaves rows <= i unchanged
    i = 6
    k2, v2 = k.copy(), v.copy()
    k2[i + 1:] += 5.0
    v2[i + 1:] -= 3.0
    o2, lse2, _ = orc.forward_head(q, k2, v2, scale, True)
    np.testing.assert_array_equal(o2[: i + 1], o[: i + 1])
    np.testing.assert_array_equal(lse2[: i + 1], lse[: i + 1])
    # the last key only receives gradient from the last query
    np.testing.assert_allclose(dv[-1], _p_last(q, k, scale) * do[-1], rtol=1e-13, atol=1e-14)


def _p_last(q, k, scale):
    s = scale * (q[-1] @ k.T)
    e = np.exp(s - s.max())
    return e[-1] / e.sum()


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("n,d", [(1, 2), (3, 4), (5, 2), (8, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(n, d, causal):
    r = rng(100 + n * 10 + d + (1 if causal else 0))
    q, k, v, gup = r.standard_normal((4, n, d))
    scale = 0.6

    def loss(qq, kk, vv):
        o, _, _ = orc.forward_head(qq, kk, vv, scale, causal)
        return float((o * gup).sum())

    dq, dk, dv, _ = orc.backward_head(q, k, v, gup, scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-7, (name, err)


def test_library_autograd_cross_check():
    """torch CPU fp64 autograd of softmax(scale Q K^T + mask) V on small inputs."""
    g = torch.Generator().manual_seed(7)
    for causal in (False, True):
        n, d = 11, 5
        q, k, v, do = (torch.randn(n, d, generator=g, dtype=torch.float64) for _ in range(4))
        qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
        s = 0.4 * qq @ kk.T
        if causal:
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ vv
        o.backward(do)
        o_ref, lse_ref, _ = orc.forward_head(q.numpy(), k.numpy(), v.numpy(), 0.4, causal)
        np.testing.assert_allclose(o_ref, o.detach().numpy(), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse_ref, torch.logsumexp(s, dim=-1).detach().numpy(), rtol=1e-13, atol=1e-14)
        dq, dk, dv, _ = orc.backward_head(q.numpy(), k.numpy(), v.numpy(), do.numpy(), 0.4, causal)
        for a, b in ((dq, qq.grad), (dk, kk.grad), (dv, vv.grad)):
            np.testing.assert_allclose(a, b.numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- online vs untiled
@pytest.mark.parametrize("seed", range(6))
def test_online_equals_untiled_on_random_splits(seed):
    r = rng(200 + seed)
    n, d = 41, 7
    q, k, v = r.standard_normal((3, n, d)) * 2
    scale = 0.8
    for causal in (False, True):
        o, lse, _ = orc.forward_head(q, k, v, scale, causal)
        s = orc.scores_head(q, k, scale, causal)
        for i in range(n):
            # random contiguous blocks, including size-1 blocks and the whole row
            cuts = sorted(set(r.integers(1, n, size=r.integers(0, 8)).tolist()))
            if seed == 0:
                cuts = []
            if seed == 1:
                cuts = list(range(1, n))
            sizes = np.diff([0] + cuts + [n]).tolist()
            oi, li = orc.online_attention_row(s[i], v, sizes)
            np.testing.assert_allclose(oi, o[i], rtol=1e-12, atol=1e-13)
            assert abs(li - lse[i]) < 1e-12


def test_online_skips_fully_masked_first_block():
    """A causal row whose first visited block is entirely masked must not produce NaN."""
    x = [-np.inf, -np.inf, 0.5, -1.0, 2.0]
    v = np.arange(10.0).reshape(5, 2)
    o, lse = orc.online_attention_row(x, v, [2, 3])
    w = np.exp(np.array(x[2:]) - 2.0)
    np.testing.assert_allclose(o, (w / w.sum()) @ v[2:], rtol=1e-14)
    m, l, _ = orc.online_softmax_row(x, [2, 1, 2])
    assert m == 2.0 and abs(l - w.sum()) < 1e-14


# ---------------------------------------------------------------- invariances
def test_permutation_and_shift_invariance():
    r = rng(5)
    n, d = 19, 6
    q, k, v = r.standard_normal((3, n, d))
    o, lse, p = orc.forward_head(q, k, v, 0.9, False)
    perm = r.permutation(n)
    o2, lse2, _ = orc.forward_head(q, k[perm], v[perm], 0.9, False)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-14)
    o3, lse3, _ = orc.forward_head(q[perm], k, v, 0.9, False)
    np.testing.assert_allclose(o3, o[perm], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse3, lse[perm], rtol=1e-13, atol=1e-14)
    # adding c * u to every key adds scale * c * (q_i . u) to all scores of row i: P unchanged
    u = r.standard_normal(d)
    k4 = k + 3.0 * u[None, :]
    o4, lse4, p4 = orc.forward_head(q, k4, v, 0.9, False)
    np.testing.assert_allclose(p4, p, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse4, lse + 0.9 * 3.0 * (q @ u), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- gradient identities
@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identities(causal):
    r = rng(6)
    n, d = 64, 16
    q, k, v, do = r.standard_normal((4, n, d))
    o, _, _ = orc.forward_head(q, k, v, 0.25, causal)
    dq, dk, dv, delta = orc.backward_head(q, k, v, do, 0.25, causal)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(delta, (do * o).sum(axis=1), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- row-local helpers
@pytest.mark.parametrize("causal", [False, True])
def test_row_local_helpers_agree_with_full(causal):
    r = rng(8)
    n, d = 50, 8
    q, k, v, do = r.standard_normal((4, n, d))
    o, lse, _ = orc.forward_head(q, k, v, 0.35, causal)
    dq, _, _, _ = orc.backward_head(q, k, v, do, 0.35, causal)
    rows = [0, 7, 31, 49]
    o_r, lse_r = orc.forward_rows(q[rows], rows, k, v, 0.35, causal)
    np.testing.assert_allclose(o_r, o[rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse_r, lse[rows], rtol=1e-13, atol=1e-14)
    dq_r = orc.dq_rows(q[rows], do[rows], rows, k, v, 0.35, causal)
    np.testing.assert_allclose(dq_r, dq[rows], rtol=1e-12, atol=1e-13)


def test_batched_wrappers_match_heads():
    r = rng(9)
    q, k, v, do = r.standard_normal((4, 2, 3, 9, 4))
    o, lse = orc.attention_forward(q, k, v, 0.5, True)
    dq, dk, dv = orc.attention_backward(q, k, v, do, 0.5, True)
    o1, l1, _ = orc.forward_head(q[1, 2], k[1, 2], v[1, 2], 0.5, True)
    g1 = orc.backward_head(q[1, 2], k[1, 2], v[1, 2], do[1, 2], 0.5, True)
    np.testing.assert_array_equal(o[1, 2], o1)
    np.testing.assert_array_equal(lse[1, 2], l1)
    np.testing.assert_array_equal(dq[1, 2], g1[0])
    np.testing.assert_array_equal(dk[1, 2], g1[1])
    np.testing.assert_array_equal(dv[1, 2], g1[2])
