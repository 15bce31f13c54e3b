"""Decode attention against a KV cache, in fp64 on the CPU (test infrastructure only).

Nothing in the GPU library may import or call this module; only tests and
the benchmark's CPU-baseline leg do.  It shares no code with the HIP path.

Source (the pages, by title and section): "What is Flash Attention?" (iania.ai
video page, English).  10:00 lists memory-bound inference with long prompts
among the uses; 11:02-11:33 names the KV cache for fast generation as the
next step; 04:46-05:17 gives the rule that merges softmax statistics of
separate blocks of keys (running max, rescaled sums and accumulators).

Readings (where the pages say no more):
  * decode: Nq new queries (a few) attend to the Nk keys and values held in
    a cache; O = softmax(scale q K^T) V per (batch, head), L = logsumexp;
  * causal decode: the new queries are the last Nq positions of the
    sequence, so query i (0-based among them) sees keys j <= Nk - Nq + i
    (bottom-right aligned; with Nq = Nk this is the usual causal mask);
  * the kernels split the keys into chunks and merge the per-chunk
    statistics with the pages' rule; the oracle computes the unsplit result
    directly, and `merge_partials` is the rule itself, for its own pin.
"""
from __future__ import annotations

import numpy as np

from .attention import NEG_INF, _f64, _safe_softmax


def decode_allowed(n_q: int, n_k: int, causal: bool) -> np.ndarray:
    """Boolean [n_q, n_k]: query i may see key j (bottom-right aligned when causal)."""
    if not causal:
        return np.ones((n_q, n_k), dtype=bool)
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= n_k - n_q + i


def decode_head(q, k, v, scale: float, causal: bool):
    """O [n_q, d], L [n_q] for n_q queries against n_k cached keys and values."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = scale * (q @ k.T)
    s = np.where(decode_allowed(q.shape[0], k.shape[0], causal), s, NEG_INF)
    p, m, l = _safe_softmax(s)
    with np.errstate(divide="ignore"):
        lse = np.where(np.isfinite(m), m + np.log(l), NEG_INF)
    return p @ v, lse


def attention_decode(q, k, v, scale: float, causal: bool):
    """Over all (batch, head) pairs: q [B,H,Nq,d], k and v [B,H,Nk,d]; returns O, L in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n_q, d = q.shape
    o = np.empty((B, H, n_q, v.shape[-1]))
    lse = np.empty((B, H, n_q))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = decode_head(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def chunk_partial(s_chunk, v_chunk):
    """Softmax statistics of one chunk of scores (natural-log units): m, l, unnormalised acc."""
    m = s_chunk.max()
    if m == NEG_INF:
        return NEG_INF, 0.0, np.zeros(v_chunk.shape[1])
    e = np.exp(s_chunk - m)
    return m, float(e.sum()), e @ v_chunk


def merge_partials(parts):
    """Merge (m, l, acc) of disjoint key chunks ([video] 04:46-05:17): with
    m' = max m_c, alpha_c = e^(m_c - m'), l' = sum alpha_c l_c and
    acc' = sum alpha_c acc_c; returns O = acc' / l' and L = m' + ln l'."""
    m_star = max(m for m, _, _ in parts)
    if m_star == NEG_INF:
        return np.zeros(parts[0][2].shape), NEG_INF
    l_star = 0.0
    acc = np.zeros(parts[0][2].shape)
    for m, l, a in parts:
        if m == NEG_INF:
            continue
        alpha = np.exp(m - m_star)
        l_star += alpha * l
        acc += alpha * a
    return acc / l_star, m_star + np.log(l_star)
