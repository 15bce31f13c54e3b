"""Attention with dropout on P, in fp64 on the CPU (test infrastructure only).

Nothing in the GPU library may import or call this module; only tests, the
smoke check and the benchmark's CPU-baseline leg do.  It shares no code with
the HIP path.

Source (the pages, by title and section): the FlashAttention talk transcript
(youtube-distilled.com, FThvfkXWqtE).  Its background on standard attention
applies an optional dropout to the softmax output before the product with V;
its questions after the method part note that the fused kernel drops entries
without writing them out, while the gradients still need the same decisions.

Readings (where the pages say no more):
  * inverted dropout: O = (Z * P / (1 - p)) V, with Z_ij in {0, 1}; L is the
    logsumexp of the scores without dropout (the backward recomputes P from
    it and applies the same Z);
  * Z comes from the counter-based generator Philox4x32-10 (Salmon, Moraes,
    Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011),
    keyed by a 64-bit seed.  Element (i, j) of head bh (= b * H + h) takes
    the generator output for counter (j // 4, i // 4, bh, 0), byte
    4 * (i % 4) + (j % 4) of its 16 little-endian bytes, and is kept iff
    that byte is >= t, where t = round(256 p) in [0, 255]: the rate applied
    is exactly t / 256;
  * backward: dV = (Z * P / (1 - p))^T dO, dP = Z * (dO V^T) / (1 - p),
    Delta_i = sum_j P_ij dP_ij (= rowsum(dO * O)), dS = P * (dP - Delta),
    dQ = scale dS K, dK = scale dS^T Q.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, forward_head

# Philox4x32 constants (Salmon et al. 2011): round multipliers and the Weyl
# increments of the key schedule.
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint32(0x9E3779B9)
_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on uint32 arrays (broadcast); returns four uint32 arrays.

    One round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as 64-bit
    products; the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).
    The key advances by (W0, W1) before every round after the first.
    """
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint32) for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint32)
    k1 = np.asarray(k1, dtype=np.uint32)
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd > 0:
                k0 = (k0 + _W0).astype(np.uint32)
                k1 = (k1 + _W1).astype(np.uint32)
            p0 = c0.astype(np.uint64) * _M0
            p1 = c2.astype(np.uint64) * _M1
            hi0, lo0 = (p0 >> np.uint64(32)).astype(np.uint32), (p0 & _MASK32).astype(np.uint32)
            hi1, lo1 = (p1 >> np.uint64(32)).astype(np.uint32), (p1 & _MASK32).astype(np.uint32)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def threshold(p_drop: float) -> int:
    """The byte threshold t = round(256 p) used for a requested dropout rate p in [0, 1)."""
    t = int(np.floor(256.0 * p_drop + 0.5))
    if not 0 <= t <= 255:
        raise ValueError(f"dropout rate {p_drop} gives threshold {t} outside [0, 255]")
    return t


def keep_mask(seed: int, t: int, bh: int, n_q: int, n_k: int) -> np.ndarray:
    """Boolean [n_q, n_k]: True where element (i, j) of head bh is kept."""
    qi = np.arange(n_q)
    kj = np.arange(n_k)
    gi, gj = np.meshgrid(np.arange((n_q + 3) // 4), np.arange((n_k + 3) // 4), indexing="ij")
    words = philox4x32_10(gj, gi, np.full(gi.shape, bh), np.zeros(gi.shape), seed & 0xFFFFFFFF,
                          (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(words, axis=-1)  # [n_q/4, n_k/4, 4]
    word = w[qi[:, None] // 4, kj[None, :] // 4, qi[:, None] % 4]
    byte = (word >> (8 * (kj[None, :] % 4)).astype(np.uint32)) & np.uint32(0xFF)
    return byte >= t


def forward_head_dropout(q, k, v, scale: float, causal: bool, seed: int, t: int, bh: int):
    """O = (Z * P / (1 - p)) V and L = logsumexp of the undropped scores, for one head.

    Returns (O, L, P, Z) with p = t / 256.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _, lse, p = forward_head(q, k, v, scale, causal)
    z = keep_mask(seed, t, bh, q.shape[0], k.shape[0])
    pd = np.where(z, p, 0.0) / (1.0 - t / 256.0)
    return pd @ v, lse, p, z


def backward_head_dropout(q, k, v, do, scale: float, causal: bool, seed: int, t: int, bh: int):
    """Exact gradients of O = (Z * softmax(scale Q K^T + mask) / (1 - p)) V for one head.

    Returns (dQ, dK, dV, Delta).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _, _, p, z = forward_head_dropout(q, k, v, scale, causal, seed, t, bh)
    keep = 1.0 - t / 256.0
    pd = np.where(z, p, 0.0) / keep
    dv = pd.T @ do
    dp = np.where(z, do @ v.T, 0.0) / keep
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv, delta


def attention_forward_dropout(q, k, v, scale: float, causal: bool, seed: int, t: int):
    """Forward with dropout over all (batch, head) pairs of [B, H, N, d] inputs."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h], _, _ = forward_head_dropout(q[b, h], k[b, h], v[b, h], scale, causal, seed, t,
                                                            b * H + h)
    return o, lse


def attention_backward_dropout(q, k, v, do, scale: float, causal: bool, seed: int, t: int):
    """Backward with dropout over all (batch, head) pairs; returns dQ, dK, dV."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], _ = backward_head_dropout(q[b, h], k[b, h], v[b, h], do[b, h], scale,
                                                                    causal, seed, t, b * H + h)
    return dq, dk, dv
