"""Pins of the oracle's FP8 (e4m3) attention (CPU only).

* e4m3 decoding against values fixed by the OFP8 definition (zero, the
  smallest subnormal, the smallest normal, one, the largest finite value,
  NaN) and against torch's float8_e4m3fn reinterpretation of all 256 codes;
* e4m3 rounding against torch's float8_e4m3fn cast on random magnitudes
  across the whole range and on every exact midpoint (ties to even);
* the attention itself: a hand-computed three-key case, and invariants of
  the per-tensor scales (only the product dq dk enters S; dv scales O);
* the error model of rounding P to e4m3: its bound holds for a CPU emulation
  of that rounding at any reference-max offset sigma in [1, 2^8], it is
  attained to within 6% on a constructed worst case (so its
  constant is not too large either), and the error scale is within a small
  factor of the emulated root-mean-square error.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as orc
from oracle import fp8


def torch_decode(codes):
    t = torch.as_tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_round(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_fixed_values():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x80: 0.0}
    for c, v in cases.items():
        assert fp8.e4m3_decode(np.uint8(c)) == v, hex(c)
    assert np.isnan(fp8.e4m3_decode(np.uint8(0x7F))) and np.isnan(fp8.e4m3_decode(np.uint8(0xFF)))


def test_decode_structure():
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)                                   # codes 0..126 increase
    neg = fp8.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    np.testing.assert_array_equal(neg, -pos)                          # sign bit only flips the sign
    assert np.isfinite(fp8.e4m3_decode(np.arange(256, dtype=np.uint8))).sum() == 254


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    np.testing.assert_array_equal(fp8.e4m3_decode(codes), torch_decode(codes))


def test_round_matches_torch_on_random_values():
    r = np.random.default_rng(0)
    mag = np.exp2(r.uniform(-12, math.log2(460), 200000))
    x = (mag * r.choice([-1.0, 1.0], mag.size)).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(fp8.e4m3_round(x), torch_round(x))


def test_round_ties_go_to_even_like_torch():
    vals = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                                  # exact in fp32
    got = fp8.e4m3_round(mids)
    np.testing.assert_array_equal(got, torch_round(mids))
    # the even neighbour: the code of the result has mantissa bit 0 clear
    idx = np.searchsorted(vals, got)
    assert np.all(idx % 2 == 0)
    assert fp8.e4m3_round(464.0) == 448.0 and np.isnan(fp8.e4m3_round(470.0))


def test_round_is_nearest_and_idempotent():
    vals = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    np.testing.assert_array_equal(fp8.e4m3_round(vals), vals)
    r = np.random.default_rng(1)
    x = r.uniform(0, 448, 10000)
    got = fp8.e4m3_round(x)
    best = np.min(np.abs(vals[None, :] - x[:, None]), axis=1)
    np.testing.assert_array_equal(np.abs(got - x), best)


def test_three_key_case_by_hand():
    # q = [1, 0], keys [1,0], [0,1], [2,0] (all exact e4m3 codes), scale 1,
    # dq = dk = dv = 1: scores 1, 0, 2
    q8 = np.array([[0x38, 0x00]], dtype=np.uint8)
    k8 = np.array([[0x38, 0x00], [0x00, 0x38], [0x40, 0x00]], dtype=np.uint8)
    v8 = np.array([[0x38, 0x40], [0x30, 0x00], [0xB8, 0x38]], dtype=np.uint8)  # [1,2], [0.5,0], [-1,1]
    o, lse = fp8.forward_head_fp8(q8, k8, v8, 1.0, 1.0, 1.0, 1.0, False)
    e = [math.e, 1.0, math.e ** 2]
    z = sum(e)
    want = [(e[0] * 1 + e[1] * 0.5 - e[2]) / z, (e[0] * 2 + e[2] * 1) / z]
    np.testing.assert_allclose(o[0], want, rtol=1e-15)
    assert abs(lse[0] - math.log(z)) < 1e-15


def random_codes(r, shape):
    c = r.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)   # no NaN codes


def test_scale_invariants():
    r = np.random.default_rng(2)
    q8, k8, v8 = (random_codes(r, (40, 16)) for _ in range(3))
    s = 0.002
    o1, l1 = fp8.forward_head_fp8(q8, k8, v8, 1.0, 1.0, 1.0, s, True)
    o2, l2 = fp8.forward_head_fp8(q8, k8, v8, 4.0, 0.25, 1.0, s, True)        # dq dk = 1
    o3, l3 = fp8.forward_head_fp8(q8, k8, v8, 2.0, 1.0, 1.0, s / 2, True)     # scale dq dk = s
    o4, l4 = fp8.forward_head_fp8(q8, k8, v8, 1.0, 1.0, 3.0, s, True)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)
    np.testing.assert_allclose(o3, o1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l3, l1, rtol=1e-13)
    np.testing.assert_allclose(o4, 3 * o1, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(l4, l1)


def test_forward_is_attention_of_dequantized_values():
    r = np.random.default_rng(3)
    q8, k8, v8 = (random_codes(r, (1, 2, 30, 8)) for _ in range(3))
    o, lse = fp8.attention_forward_fp8(q8, k8, v8, 0.01, 0.02, 0.5, 0.3, False)
    for h in range(2):
        q = fp8.e4m3_decode(q8[0, h]) * 0.01
        k = fp8.e4m3_decode(k8[0, h]) * 0.02
        v = fp8.e4m3_decode(v8[0, h]) * 0.5
        s = 0.3 * q @ k.T
        p = np.exp(s - s.max(axis=1, keepdims=True))
        np.testing.assert_allclose(o[0, h], (p / p.sum(axis=1, keepdims=True)) @ v, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[0, h], s.max(axis=1) + np.log(p.sum(axis=1)), rtol=1e-13)


def emulate(q8, k8, v8, dq, dk, dv, scale, causal, log_sigma, tile=64):
    """O with P rounded to e4m3 in the units of a reference max sigma below
    the row max (log2 sigma = log_sigma[row, tile]); l from the unrounded p."""
    q, k, v = fp8.dequantize(q8, dq), fp8.dequantize(k8, dk), fp8.dequantize(v8, dv)
    s = orc.scores_head(q, k, scale, causal)
    p_t = np.where(np.isfinite(s), np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
    sig = np.exp2(np.repeat(log_sigma, tile, axis=1)[:, : s.shape[1]])
    p_hat = fp8.e4m3_round(sig * p_t) / sig
    return (p_hat @ v) / p_t.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sigma_mode", ["one", "max", "random"])
def test_error_model_against_emulation(causal, sigma_mode):
    r = np.random.default_rng(4 + causal)
    n, d = 300, 64
    x = r.standard_normal((3, n, d))
    codes = [torch.as_tensor(t / (np.abs(t).max() / 448), dtype=torch.float32).to(torch.float8_e4m3fn)
             .view(torch.uint8).numpy() for t in x]
    descale = [float(np.abs(t).max() / 448) for t in x]
    args = (*codes, *descale, 1 / math.sqrt(d), causal)
    n_tiles = (n + 63) // 64
    ls = {"one": np.zeros((n, n_tiles)), "max": np.full((n, n_tiles), 8.0),
          "random": r.uniform(0, 8, (n, n_tiles))}[sigma_mode]
    o, _ = fp8.forward_head_fp8(*args)
    bound, sigma, _ = fp8.error_model_head(*args)
    err = np.abs(emulate(*args, ls) - o)
    assert np.all(err <= bound)
    z = np.sqrt(np.mean((err / sigma) ** 2))
    assert 0.2 <= z <= 1.0, z


def test_error_bound_is_nearly_attained():
    # one key with p_t just below the first midpoint of a binade, 1 + 2^-4:
    # it rounds down to 1 and O = p_hat v / p misses v by (p - 1) / p, which
    # approaches 2^-4 / (1 + 2^-4) = 1/17, the largest relative rounding
    # error of a normal e4m3 value.  The bound uses 2^-4 = 17/16 of that.
    x = 1.0 + 2.0 ** -4 - 2.0 ** -20
    p_t = np.array([[x]])
    v = np.array([[1.0]])
    bound, _ = fp8._error_model(p_t, v)
    err = abs(fp8.e4m3_round(x) - x) / x
    assert err <= bound[0, 0] and err >= 0.999 * (16 / 17) * bound[0, 0]


def test_rows_match_head():
    r = np.random.default_rng(5)
    n, d = 150, 32
    q8, k8, v8 = (random_codes(r, (n, d)) for _ in range(3))
    args = (0.01, 0.01, 0.1, 0.2, True)
    o, lse = fp8.forward_head_fp8(q8, k8, v8, *args)
    bound, sigma, eps = fp8.error_model_head(q8, k8, v8, *args, s_rel=2.0 ** -13)
    rows = [0, 7, 64, 149]
    o_r, l_r, b_r, s_r, e_r = fp8.forward_rows_fp8(q8[rows], rows, k8, v8, *args, s_rel=2.0 ** -13)
    np.testing.assert_allclose(o_r, o[rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l_r, lse[rows], rtol=1e-13)
    np.testing.assert_allclose(b_r, bound[rows], rtol=1e-12)
    np.testing.assert_allclose(s_r, sigma[rows], rtol=1e-12)
    np.testing.assert_allclose(e_r, eps[rows], rtol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_score_error_terms_against_perturbation(seed):
    """Scores perturbed by at most eps (here the eps of a contraction with
    relative precision 2^-10 of the product magnitudes, chosen at its extreme
    +-eps per entry): L moves by at most eps and O by at most the bound's
    score term (no P rounding in this check: the perturbed result is exact)."""
    r = np.random.default_rng(20 + seed)
    n, d = 120, 16
    q8, k8, v8 = (random_codes(r, (n, d)) for _ in range(3))
    args = (0.01, 0.02, 0.1, 0.3, bool(seed % 2))
    o, lse = fp8.forward_head_fp8(q8, k8, v8, *args)
    b0, _, _ = fp8.error_model_head(q8, k8, v8, *args, s_rel=0.0)
    b1, _, eps = fp8.error_model_head(q8, k8, v8, *args, s_rel=2.0 ** -10)
    assert np.all(eps > 0)
    q, k, v = fp8.dequantize(q8, 0.01), fp8.dequantize(k8, 0.02), fp8.dequantize(v8, 0.1)
    s = orc.scores_head(q, k, 0.3, args[-1])
    s2 = s + eps[:, None] * r.choice([-1.0, 1.0], s.shape)
    p, m, l = orc._safe_softmax(s2)
    o2 = p @ v
    lse2 = m + np.log(l)
    assert np.all(np.abs(lse2 - lse) <= eps * (1 + 1e-12))
    # the score part of the bound: b1 - e^(2 eps) b0 = (e^(2 eps) - 1) sum p_t |v| / l_t
    score_term = b1 - np.exp(2 * eps)[:, None] * b0
    assert np.all(np.abs(o2 - o) <= score_term * (1 + 1e-9) + 1e-15)
