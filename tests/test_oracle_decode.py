"""Pins of the oracle's decode attention (CPU only).

Decode is pinned to the square attention oracle (itself pinned elsewhere):
with Nq = Nk it is plain attention, and its causal rows are the last rows of
causal attention over the whole sequence.  The chunk merge rule is pinned to
the unsplit softmax on random splits, including chunks with no allowed key.
"""
import numpy as np
import pytest

from oracle import attention as orc
from oracle import decode as dec


@pytest.mark.parametrize("causal", [False, True])
def test_square_decode_is_attention(causal):
    r = np.random.default_rng(1)
    q, k, v = r.standard_normal((3, 40, 8))
    o, lse = dec.decode_head(q, k, v, 0.3, causal)
    o_ref, lse_ref, _ = orc.forward_head(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("n_q", [1, 3, 8])
def test_causal_decode_rows_are_the_last_rows_of_causal_attention(n_q):
    """The new queries are the last n_q positions: their rows of causal attention
    over all n_k positions are the decode result."""
    r = np.random.default_rng(2 + n_q)
    n_k, d = 57, 6
    q_all, k, v = r.standard_normal((3, n_k, d))
    o_full, lse_full, _ = orc.forward_head(q_all, k, v, 0.45, True)
    o, lse = dec.decode_head(q_all[n_k - n_q:], k, v, 0.45, True)
    np.testing.assert_allclose(o, o_full[n_k - n_q:], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_full[n_k - n_q:], rtol=1e-13, atol=1e-14)


def test_non_causal_decode_ignores_query_position():
    r = np.random.default_rng(3)
    q, k, v = r.standard_normal((3, 30, 5))
    o, _ = dec.decode_head(q[:4], k, v, 0.5, False)
    o2, _ = dec.decode_head(q[2:3], k, v, 0.5, False)
    np.testing.assert_allclose(o[2:3], o2, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("seed", range(5))
def test_merge_of_random_chunks_equals_unsplit(seed):
    r = np.random.default_rng(10 + seed)
    n, d = 97, 4
    s = 3 * r.standard_normal(n)
    v = r.standard_normal((n, d))
    s[r.random(n) < 0.3] = -np.inf          # some masked keys
    s[20:35] = -np.inf                      # a chunk that may be empty
    cuts = np.sort(r.choice(np.arange(1, n), size=6, replace=False))
    parts = [dec.chunk_partial(s[a:b], v[a:b]) for a, b in zip(np.r_[0, cuts], np.r_[cuts, n])]
    o, lse = dec.merge_partials(parts)
    p = np.exp(s - s.max())
    np.testing.assert_allclose(o, (p / p.sum()) @ v, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, s.max() + np.log(p.sum()), rtol=1e-13, atol=1e-14)


def test_merge_with_every_chunk_empty():
    parts = [dec.chunk_partial(np.full(5, -np.inf), np.ones((5, 3))) for _ in range(3)]
    o, lse = dec.merge_partials(parts)
    assert np.all(o == 0) and lse == -np.inf


def test_batched_decode_matches_heads():
    r = np.random.default_rng(4)
    q = r.standard_normal((2, 3, 2, 8))
    k, v = r.standard_normal((2, 2, 3, 50, 8))
    o, lse = dec.attention_decode(q, k, v, 0.35, True)
    for b in range(2):
        for h in range(3):
            o_h, lse_h = dec.decode_head(q[b, h], k[b, h], v[b, h], 0.35, True)
            np.testing.assert_array_equal(o[b, h], o_h)
            np.testing.assert_array_equal(lse[b, h], lse_h)
