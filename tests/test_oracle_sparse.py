"""Pins of the oracle's block-sparse attention (CPU only).

Block-sparse attention keeps the (query, key) pairs whose 128 x 128 block is
on in a block mask, on top of the causal mask ([talk], questions after the
method part: the tiled method also takes imposed sparsity).  Each pin checks
the oracle against something other than itself: dense attention on separate
blocks, torch's own masked attention and its autograd, finite differences,
and the defined behaviour of rows with no allowed key.
"""
import numpy as np
import pytest
import torch

from oracle import attention as orc

B = orc.BLOCK


def rng(seed):
    return np.random.default_rng(seed)


def test_block_diagonal_mask_is_attention_on_each_block():
    """With only the diagonal blocks on, each 128-row block attends to its own
    128 keys: the result is dense attention on each block separately."""
    r = rng(1)
    n, d = 2 * B + 40, 8  # three blocks, the last one ragged
    q, k, v, do = r.standard_normal((4, n, d))
    nb = 3
    mask = np.eye(nb, dtype=np.uint8)
    for causal in (False, True):
        o, lse, _ = orc.forward_head(q, k, v, 0.5, causal, mask)
        dq, dk, dv, _ = orc.backward_head(q, k, v, do, 0.5, causal, mask)
        for b in range(nb):
            sl = slice(b * B, min(n, (b + 1) * B))
            o_b, lse_b, _ = orc.forward_head(q[sl], k[sl], v[sl], 0.5, causal)
            dq_b, dk_b, dv_b, _ = orc.backward_head(q[sl], k[sl], v[sl], do[sl], 0.5, causal)
            np.testing.assert_allclose(o[sl], o_b, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[sl], lse_b, rtol=1e-12, atol=1e-13)
            for a, bb in ((dq[sl], dq_b), (dk[sl], dk_b), (dv[sl], dv_b)):
                np.testing.assert_allclose(a, bb, rtol=1e-11, atol=1e-12)


def _random_mask(r, nb, causal):
    """A random block mask with at least one allowed key in every row."""
    m = (r.random((nb, nb)) < 0.5).astype(np.uint8)
    for i in range(nb):
        if causal:
            m[i, i] = 1  # the diagonal block holds the row's own key
        elif not m[i].any():
            m[i, r.integers(nb)] = 1
    return m


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_masked_attention_and_autograd(causal):
    """torch.nn.functional.scaled_dot_product_attention (fp64, CPU) with the
    element mask expanded from the blocks, and its autograd gradients."""
    r = rng(10 + causal)
    n, d, scale = 3 * B + 17, 6, 0.35
    nb = -(-n // B)
    mask = _random_mask(r, nb, causal)
    q, k, v, do = (torch.from_numpy(x) for x in r.standard_normal((4, n, d)))
    allowed = torch.from_numpy(orc.allowed_pairs(n, n, causal, mask))
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    o_t = torch.nn.functional.scaled_dot_product_attention(qq[None], kk[None], vv[None], attn_mask=allowed[None],
                                                           scale=scale)[0]
    o_t.backward(do)
    o, lse, _ = orc.forward_head(q.numpy(), k.numpy(), v.numpy(), scale, causal, mask)
    np.testing.assert_allclose(o, o_t.detach().numpy(), rtol=1e-12, atol=1e-13)
    s = (scale * q @ k.T).masked_fill(~allowed, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-13)
    dq, dk, dv, _ = orc.backward_head(q.numpy(), k.numpy(), v.numpy(), do.numpy(), scale, causal, mask)
    for a, b in ((dq, qq.grad), (dk, kk.grad), (dv, vv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-11, atol=1e-12)


def test_rows_without_allowed_keys():
    """A row block with every block off: O = 0, L = -inf, dQ = 0; keys in a
    column block that no row attends get dK = dV = 0; other rows unchanged."""
    r = rng(3)
    n, d = 3 * B, 4
    q, k, v, do = r.standard_normal((4, n, d))
    mask = np.array([[1, 0, 1], [0, 0, 0], [1, 0, 1]], dtype=np.uint8)
    o, lse, p = orc.forward_head(q, k, v, 0.7, False, mask)
    dq, dk, dv, delta = orc.backward_head(q, k, v, do, 0.7, False, mask)
    dead = slice(B, 2 * B)
    assert np.all(o[dead] == 0) and np.all(lse[dead] == -np.inf) and np.all(p[dead] == 0)
    assert np.all(dq[dead] == 0) and np.all(delta[dead] == 0)
    assert np.all(dk[dead] == 0) and np.all(dv[dead] == 0)  # column block 1 is never attended
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(dq)) and np.all(np.isfinite(dk))
    # the live rows see keys of blocks 0 and 2 only: attention on those keys alone
    keep = np.r_[0:B, 2 * B:3 * B]
    o_ref, lse_ref, _ = orc.forward_head(q[keep], k[keep], v[keep], 0.7, False)
    np.testing.assert_allclose(o[keep], o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[keep], lse_ref, rtol=1e-12, atol=1e-13)


def test_causal_and_block_mask_can_empty_a_row():
    """Causal with the diagonal block off: the first row of that block has no
    allowed key when the blocks to its left are off too."""
    r = rng(4)
    n, d = 2 * B, 4
    q, k, v = r.standard_normal((3, n, d))
    mask = np.array([[0, 0], [0, 1]], dtype=np.uint8)
    o, lse, _ = orc.forward_head(q, k, v, 0.5, True, mask)
    assert np.all(o[:B] == 0) and np.all(lse[:B] == -np.inf)
    o_ref, lse_ref, _ = orc.forward_head(q[B:], k[B:], v[B:], 0.5, True)
    np.testing.assert_allclose(o[B:], o_ref, rtol=1e-12, atol=1e-13)


def test_masked_gradients_match_central_differences():
    r = rng(5)
    n, d, scale = B + 72, 2, 0.6
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    q, k, v, gup = r.standard_normal((4, n, d))

    def loss(qq, kk, vv):
        o, _, _ = orc.forward_head(qq, kk, vv, scale, False, mask)
        return float((o * gup).sum())

    dq, dk, dv, _ = orc.backward_head(q, k, v, gup, scale, False, mask)
    h = 1e-6
    pick = r.integers(0, n * d, size=24)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for flat in pick:
            idx = np.unravel_index(flat, x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a_p = {"q": q, "k": k, "v": v, name: xp}
            a_m = {"q": q, "k": k, "v": v, name: xm}
            num = (loss(a_p["q"], a_p["k"], a_p["v"]) - loss(a_m["q"], a_m["k"], a_m["v"])) / (2 * h)
            assert abs(num - g[idx]) < 1e-7 * max(1.0, np.abs(g).max()), (name, idx, num, g[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_row_helpers_and_batched_wrappers_with_mask(causal):
    r = rng(6 + causal)
    Bb, H, n, d = 1, 2, 2 * B + 9, 4
    q, k, v, do = r.standard_normal((4, Bb, H, n, d))
    nb = 3
    mask = np.stack([_random_mask(r, nb, causal) for _ in range(Bb * H)])
    mask[1, 1, :] = 0  # a dead row block in head 1
    o, lse = orc.attention_forward(q, k, v, 0.5, causal, mask)
    dq, dk, dv = orc.attention_backward(q, k, v, do, 0.5, causal, mask)
    rows = [0, 5, B, B + 3, 2 * B + 8]
    for h in range(H):
        o_r, lse_r = orc.forward_rows(q[0, h, rows], rows, k[0, h], v[0, h], 0.5, causal, mask[h])
        np.testing.assert_allclose(o_r, o[0, h, rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_array_equal(np.isinf(lse_r), np.isinf(lse[0, h, rows]))
        fin = np.isfinite(lse_r)
        np.testing.assert_allclose(lse_r[fin], lse[0, h, rows][fin], rtol=1e-12, atol=1e-13)
        dq_r = orc.dq_rows(q[0, h, rows], do[0, h, rows], rows, k[0, h], v[0, h], 0.5, causal, mask[h])
        np.testing.assert_allclose(dq_r, dq[0, h, rows], rtol=1e-11, atol=1e-12)
    # a shared mask ([1, nb, nb]) is the same as repeating it per head
    o1, _ = orc.attention_forward(q, k, v, 0.5, causal, mask[:1])
    o2, _ = orc.attention_forward(q, k, v, 0.5, causal, np.repeat(mask[:1], H, axis=0))
    np.testing.assert_array_equal(o1, o2)
