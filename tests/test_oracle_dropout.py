"""Pins of the oracle's dropout (CPU only).

The generator is pinned to the published known-answer values of
Philox4x32-10 (Salmon et al., SC 2011, and the known-answer tests that ship
with its reference implementation).  The keep decisions are checked for
rate, uniformity and independence of the sequence length; the dropped
attention and its gradients against torch autograd with the same decisions,
against finite differences, and against the no-dropout oracle at rate 0.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as orc
from oracle import dropout as drp


@pytest.mark.parametrize("ctr,key,expected", [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
])
def test_philox_known_answers(ctr, key, expected):
    out = drp.philox4x32_10(*ctr, *key)
    assert tuple(int(x) for x in out) == expected


def test_philox_output_bytes_are_uniform():
    """Chi-square of the 256 byte values over 2^14 generator calls (2^16 bytes)."""
    c = np.arange(1 << 14, dtype=np.uint32)
    words = drp.philox4x32_10(c, c >> 7, np.full_like(c, 5), np.zeros_like(c), 123, 456)
    b = np.concatenate([(w[:, None] >> np.array([0, 8, 16, 24], dtype=np.uint32)[None, :]) & 0xFF
                        for w in words]).ravel()
    hist = np.bincount(b.astype(np.int64), minlength=256)
    e = b.size / 256
    chi2 = ((hist - e) ** 2 / e).sum()
    assert chi2 < 255 + 6 * math.sqrt(2 * 255), chi2  # mean 255, sd sqrt(510)


@pytest.mark.parametrize("t", [0, 26, 128, 255])
def test_keep_rate(t):
    n = 512
    z = drp.keep_mask(seed=0x1234567890AB, t=t, bh=3, n_q=n, n_k=n)
    frac = z.mean()
    keep = 1 - t / 256
    if t == 0:
        assert z.all()
    else:
        sd = math.sqrt(keep * (1 - keep) / z.size)
        assert abs(frac - keep) < 5 * sd, (frac, keep)


def test_keep_mask_depends_only_on_seed_head_and_position():
    a = drp.keep_mask(seed=77, t=100, bh=2, n_q=64, n_k=64)
    b = drp.keep_mask(seed=77, t=100, bh=2, n_q=200, n_k=131)
    assert np.array_equal(a, b[:64, :64])
    assert not np.array_equal(a, drp.keep_mask(seed=77, t=100, bh=3, n_q=64, n_k=64))
    assert not np.array_equal(a, drp.keep_mask(seed=78, t=100, bh=2, n_q=64, n_k=64))
    assert not np.array_equal(a, drp.keep_mask(seed=77 + (1 << 32), t=100, bh=2, n_q=64, n_k=64))


def test_keep_mask_uses_the_stated_byte():
    """Element (i, j) is byte 4 (i % 4) + (j % 4) of the call for counter (j // 4, i // 4, bh, 0)."""
    seed, bh, t = 0xDEADBEEF12345678, 9, 90
    z = drp.keep_mask(seed, t, bh, 12, 12)
    for i, j in [(0, 0), (3, 1), (5, 9), (11, 11), (7, 4)]:
        w = drp.philox4x32_10(j // 4, i // 4, bh, 0, seed & 0xFFFFFFFF, seed >> 32)
        byte = (int(w[i % 4]) >> (8 * (j % 4))) & 0xFF
        assert z[i, j] == (byte >= t)


def test_threshold_rounding():
    assert drp.threshold(0.0) == 0
    assert drp.threshold(0.1) == 26
    assert drp.threshold(0.5) == 128
    with pytest.raises(ValueError):
        drp.threshold(1.0)


@pytest.mark.parametrize("causal", [False, True])
def test_rate_zero_is_plain_attention(causal):
    r = np.random.default_rng(1)
    q, k, v, do = r.standard_normal((4, 37, 8))
    o, lse, _, z = drp.forward_head_dropout(q, k, v, 0.4, causal, seed=5, t=0, bh=0)
    o_ref, lse_ref, _ = orc.forward_head(q, k, v, 0.4, causal)
    assert z.all()
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(lse, lse_ref)
    g = drp.backward_head_dropout(q, k, v, do, 0.4, causal, seed=5, t=0, bh=0)
    g_ref = orc.backward_head(q, k, v, do, 0.4, causal)
    for a, b in zip(g, g_ref):
        np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_with_the_same_decisions(causal):
    n, d, scale, seed, t, bh = 45, 6, 0.5, 0xABCDEF, 51, 4
    g = torch.Generator().manual_seed(2)
    q, k, v, do = (torch.randn(n, d, generator=g, dtype=torch.float64) for _ in range(4))
    z = torch.from_numpy(drp.keep_mask(seed, t, bh, n, n))
    qq, kk, vv = (x.clone().requires_grad_(True) for x in (q, k, v))
    s = scale * qq @ kk.T
    if causal:
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    o_t = (torch.softmax(s, dim=-1) * z / (1 - t / 256)) @ vv
    o_t.backward(do)
    o, lse, _, _ = drp.forward_head_dropout(q.numpy(), k.numpy(), v.numpy(), scale, causal, seed, t, bh)
    np.testing.assert_allclose(o, o_t.detach().numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).detach().numpy(), rtol=1e-13, atol=1e-14)
    dq, dk, dv, delta = drp.backward_head_dropout(q.numpy(), k.numpy(), v.numpy(), do.numpy(), scale, causal,
                                                  seed, t, bh)
    for a, b in ((dq, qq.grad), (dk, kk.grad), (dv, vv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-12, atol=1e-13)
    # Delta is still rowsum(dO * O)
    np.testing.assert_allclose(delta, (do.numpy() * o).sum(axis=1), rtol=1e-12, atol=1e-13)


def test_dropout_gradients_match_central_differences():
    r = np.random.default_rng(3)
    n, d, scale, seed, t = 9, 3, 0.7, 99, 64
    q, k, v, gup = r.standard_normal((4, n, d))

    def loss(qq, kk, vv):
        o, _, _, _ = drp.forward_head_dropout(qq, kk, vv, scale, True, seed, t, 1)
        return float((o * gup).sum())

    dq, dk, dv, _ = drp.backward_head_dropout(q, k, v, gup, scale, True, seed, t, 1)
    h = 1e-6
    for name, x, gr in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a_p = {"q": q, "k": k, "v": v, name: xp}
            a_m = {"q": q, "k": k, "v": v, name: xm}
            num[idx] = (loss(a_p["q"], a_p["k"], a_p["v"]) - loss(a_m["q"], a_m["k"], a_m["v"])) / (2 * h)
        assert np.abs(num - gr).max() < 1e-7 * max(1.0, np.abs(gr).max()), name


def test_batched_wrappers_use_head_index():
    r = np.random.default_rng(4)
    q, k, v, do = r.standard_normal((4, 2, 3, 20, 4))
    o, lse = drp.attention_forward_dropout(q, k, v, 0.5, False, seed=7, t=40)
    dq, dk, dv = drp.attention_backward_dropout(q, k, v, do, 0.5, False, seed=7, t=40)
    for b in range(2):
        for h in range(3):
            o_h, lse_h, _, _ = drp.forward_head_dropout(q[b, h], k[b, h], v[b, h], 0.5, False, 7, 40, b * 3 + h)
            np.testing.assert_array_equal(o[b, h], o_h)
            g = drp.backward_head_dropout(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, False, 7, 40, b * 3 + h)
            np.testing.assert_array_equal(dq[b, h], g[0])
