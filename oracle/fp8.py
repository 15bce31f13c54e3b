"""FP8 (e4m3) attention forward in fp64 on the CPU (test infrastructure only).

Nothing in the GPU library may import or call this module; only tests and
the benchmark's CPU-baseline leg do.  It shares no code with the HIP path.

Sources:
  * "What is Flash Attention?" (iania.ai video page, English), 09:29: the
    third generation of the method adds an FP8 path to the forward.  The
    pages give no format, no scaling rule and no accuracy figure.
  * OCP 8-bit Floating Point Specification (OFP8), E4M3: one sign bit, four
    exponent bits with bias 7, three mantissa bits; exponent field 0 holds
    the subnormals (m / 8) 2^-6; S.1111.111 is NaN; there are no infinities,
    and the largest finite magnitude is 1.75 * 2^8 = 448.

Readings (where the pages say no more):
  * inputs: Q, K, V are e4m3 codes with one fp32 scale per tensor
    (dq, dk, dv): the value of code x in tensor Q is dq * e4m3(x);
  * what is computed: exact attention of the dequantized tensors,
    S = scale * (dq Q8)(dk K8)^T, P = softmax(S), O = P (dv V8), L = logsumexp;
    that is the oracle;
  * a kernel may round P to e4m3 before P V.  In the kernel's own units a
    probability is p = 2^(s - m) with a reference max m that lies within
    2^8 of the row max, so p <= 256 (inside the e4m3 range), and the row sum
    l is taken from the unrounded p.  `error_model_*` turn that rounding
    into an elementwise bound and an error scale (see there).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from . import attention as orc

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9


def e4m3_decode(codes) -> np.ndarray:
    """Values of OCP e4m3 codes (uint8) as fp64; S.1111.111 gives NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    sub = (m / 8.0) * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    val = sign * np.where(e == 0, sub, nor)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_round(x) -> np.ndarray:
    """Round fp64 values to the nearest e4m3 value, ties to even (the mode of
    the OFP8 conversions); magnitudes that round past 448 give NaN (there is
    no infinity)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                       # a = f 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                # binade exponent, subnormals share 2^-6
    quantum = np.exp2(e - 3.0)                # spacing of the 3-bit mantissa in that binade
    r = np.round(a / quantum) * quantum       # np.round: half to even
    r = np.where(a == 0, 0.0, r)
    r = np.where(r > E4M3_MAX, np.nan, r)
    return np.copysign(r, x)


def dequantize(codes, descale: float) -> np.ndarray:
    return e4m3_decode(codes) * float(descale)


def forward_head_fp8(q8, k8, v8, dq: float, dk: float, dv: float, scale: float, causal: bool):
    """O [n, d] and L [n] of one head from e4m3 codes and per-tensor scales."""
    q, k, v = dequantize(q8, dq), dequantize(k8, dk), dequantize(v8, dv)
    o, lse, _ = orc.forward_head(q, k, v, scale, causal)
    return o, lse


def attention_forward_fp8(q8, k8, v8, dq: float, dk: float, dv: float, scale: float, causal: bool):
    """Over all (batch, head) pairs of [B, H, N, d] code arrays; fp64 O, L."""
    q8, k8, v8 = (np.asarray(t) for t in (q8, k8, v8))
    B, H, n, d = q8.shape
    o = np.empty((B, H, n, d))
    lse = np.empty((B, H, n))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head_fp8(q8[b, h], k8[b, h], v8[b, h], dq, dk, dv, scale, causal)
    return o, lse


# sigma of a rounding error spread evenly over one quantum: quantum / sqrt(12)
_U = 1.0 / np.sqrt(12.0)


def _error_model(p_t: np.ndarray, v: np.ndarray, eps=None):
    """Bound and scale of the O error caused by rounding P to e4m3, and by
    score errors of at most eps per row (eps [r, 1]; None = exact scores).

    p_t [r, n]: row-normalised probabilities e^(S - max S) (masked = 0),
    v [n, d]: dequantized V.  A kernel rounds p = sigma p_t with 1 <= sigma
    <= 2^8 (its reference max lies at most 2^8 below the row max).  In the
    normal range (p >= 2^-6) the rounding error is at most 2^-4 p (half of
    a 3-bit mantissa step); below it at most 2^-10 (half the subnormal
    step).  O = sum p v / sum p, so dividing by sigma l_t:

        |dO| <= [2^-4 sum p_t |v| + 2^-10 sum_{p_t < 2^-6} |v|] / l_t,

    and p < 2^-6 implies p_t < 2^-6 since sigma >= 1.  Scores off by at
    most eps scale each p by a factor in [e^-eps, e^eps]: the rounding term
    grows by at most e^(2 eps) and the weights of the convex combination
    O = sum p v / sum p move by at most (e^(2 eps) - 1) sum p_t |v| / l_t;
    L moves by at most eps (logsumexp is 1-Lipschitz in the max norm).  The
    error scale covers the P rounding only.  It
treats each rounding error as spread evenly over its quantum
    (sigma_abs = quantum / sqrt 12), with the largest relative quantum of a
    binade (2^-3 p) and sigma = 1 for the subnormals, so it tends to
    overstate the error.
    """
    l_t = p_t.sum(axis=1, keepdims=True)
    av = np.abs(v)
    tiny = ((p_t < E4M3_MIN_NORMAL) & (p_t > 0)).astype(np.float64)
    pv = (p_t @ av) / l_t
    bound = 2.0 ** -4 * pv + 2.0 ** -10 * (tiny @ av) / l_t
    if eps is not None:
        grow = np.expm1(2.0 * np.asarray(eps, dtype=np.float64).reshape(-1, 1))
        bound = (1.0 + grow) * bound + grow * pv
    var = (2.0 ** -3 * _U) ** 2 * ((p_t * p_t) @ (v * v)) + (E4M3_SUBNORMAL_STEP * _U) ** 2 * (tiny @ (v * v))
    return bound, np.sqrt(var) / l_t


def _score_eps(q, k, scale: float, allowed, s_rel: float):
    """Per-row bound s_rel * max over allowed keys of scale * sum_k |q_k k_k|:
    the error of scores formed by a contraction whose rounding error is at
    most s_rel times the sum of the magnitudes of its products."""
    mag = scale * (np.abs(q) @ np.abs(k).T)
    mag = np.where(allowed, mag, 0.0)
    return s_rel * mag.max(axis=1, keepdims=True)


def error_model_head(q8, k8, v8, dq: float, dk: float, dv: float, scale: float, causal: bool,
                     s_rel: float = 0.0):
    """(bound [n, d], sigma [n, d], eps [n]) for one head's O and L with P
    rounded to e4m3 and scores formed with relative precision s_rel (of the
    sum of product magnitudes); see _error_model.  |L - L_ref| <= eps."""
    q, k, v = dequantize(q8, dq), dequantize(k8, dk), dequantize(v8, dv)
    s = orc.scores_head(q, k, scale, causal)
    m = np.max(s, axis=1, keepdims=True)
    p_t = np.where(np.isfinite(s), np.exp(s - m), 0.0)
    eps = _score_eps(q, k, scale, np.isfinite(s), s_rel)
    bound, sigma = _error_model(p_t, v, eps)
    return bound, sigma, eps[:, 0]


def forward_rows_fp8(q8_rows, rows: Sequence[int], k8, v8, dq: float, dk: float, dv: float, scale: float,
                     causal: bool, s_rel: float = 0.0):
    """O, L, bound, sigma and eps for the listed query rows of one head:
    q8_rows [r, d] holds the codes of rows `rows` (their positions, for the
    causal mask); k8, v8 are the head's [n, d] codes."""
    q = dequantize(q8_rows, dq)
    k, v = dequantize(k8, dk), dequantize(v8, dv)
    o, lse = orc.forward_rows(q, rows, k, v, scale, causal)
    n = k.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.arange(n)[None, :] <= np.asarray(rows)[:, None], s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    p_t = np.where(np.isfinite(s), np.exp(s - m), 0.0)
    eps = _score_eps(q, k, scale, np.isfinite(s), s_rel)
    bound, sigma = _error_model(p_t, v, eps)
    return o, lse, bound, sigma, eps[:, 0]
