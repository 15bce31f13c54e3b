"""Plain, slow, obviously correct CPU fp64 attention (test infrastructure only).

Nothing in the GPU library may import or call this module; only tests, the
smoke check and the benchmark's CPU-baseline leg do.  It shares no code with
the HIP path.  Every function materialises what it needs in float64, one
(batch, head) pair at a time, with NumPy matrix products as its only library
primitive.

Sources (the pages, by title and section):
  [video]  "What is Flash Attention?" (iania.ai video page, English), full
           transcript: 01:04 (S = Q K^T / sqrt(D), row softmax P, O = P V),
           04:15-05:17 (online softmax: running max m, running sum l, factors
           alpha and beta, deferred division by l), 05:49-06:52 (worked
           example on the scores 1, 2, 3, 0), 06:52-07:24 (backward keeps O and
           per-row statistics and recomputes P), 08:26 (same function, same
           gradients).
  [slides] "Atencao exata, acelerada por nunca escrever a grade gigante"
           (mentria.ai), formulas on block scores S_ij = Q_i K_j^T / sqrt(d),
           safe softmax, the online update and o_flash = o_exact.
  [talk]   FlashAttention talk transcript (youtube-distilled.com, FThvfkXWqtE),
           background on standard attention with an optional mask, and the
           method part on splitting softmax over blocks A1, A2.

Readings where the pages are silent (each listed in the design notes):
  * the scale multiplies Q K^T before the mask and the softmax; default
    1/sqrt(d), any finite scale accepted;
  * the causal mask lets query i see keys j <= i (square, top-left aligned);
  * the saved per-row statistic is one number, L_i = m_i + ln(l_i), in natural
    log of the scaled, masked scores;
  * the backward is the exact gradient of O with respect to Q, K and V for an
    upstream gradient dO; its formulas come from differentiating the
    definition (the pages only say the gradients are the same);
  * block-sparse attention ([talk], questions after the method part: the
    tiled method also takes imposed sparsity, skipping the computation it
    removes) keeps the pairs whose 128 x 128 block is switched on in a block
    mask, on top of the causal mask; a query row with no allowed key has
    P = 0, O = 0 and L = -inf, and contributes no gradient.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

NEG_INF = -np.inf
BLOCK = 128  # side of one block of a block-sparse mask


def _f64(x) -> np.ndarray:
    """Upcast exactly to float64 (bf16 and fp32 values are exact in fp64)."""
    if hasattr(x, "detach"):  # a torch tensor
        x = x.detach().to("cpu")
        import torch

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def allowed_pairs(n_q: int, n_k: int, causal: bool, block_mask=None) -> np.ndarray:
    """Boolean [n_q, n_k]: True where query i may attend key j.

    Causal: j <= i.  Block-sparse: the (i // BLOCK, j // BLOCK) entry of the
    block mask is nonzero ([talk], questions after the method part).
    """
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    ok = np.ones((n_q, n_k), dtype=bool)
    if causal:
        ok &= j <= i
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        ok &= bm[i // BLOCK, j // BLOCK]
    return ok


def scores_head(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, block_mask=None) -> np.ndarray:
    """S = scale * Q K^T for one head, with -inf wherever a pair is not allowed.

    [video] 01:04: scores are Q times K transposed over sqrt(D); [slides] block
    scores formula.  [talk] background: the mask sets entries to -inf before
    the softmax.
    """
    s = scale * (q @ k.T)
    if causal or block_mask is not None:
        s = np.where(allowed_pairs(s.shape[0], s.shape[1], causal, block_mask), s, NEG_INF)
    return s


def _safe_softmax(s: np.ndarray):
    """Row softmax with the row max subtracted first ([slides] safe-softmax formula).

    Returns P, the row max m and the row sum l of exp(s - m).  A row with no
    finite score (every key masked) has m = -inf, l = 0 and P = 0.
    """
    m = s.max(axis=1)
    live = np.isfinite(m)
    e = np.exp(s - np.where(live, m, 0.0)[:, None])  # exp(-inf) = 0 at masked entries
    l = e.sum(axis=1)
    p = np.where(live[:, None], e / np.where(live, l, 1.0)[:, None], 0.0)
    return p, m, l


def forward_head(q, k, v, scale: float, causal: bool, block_mask=None):
    """Standard attention for one head: S, P = softmax(S), O = P V, and L = m + ln l.

    [video] 01:04 for S, P, O; 06:52-07:24 for the per-row statistics kept for
    the backward, stored here as the single logsumexp L.  `block_mask`
    ([ceil(N/128), ceil(N/128)], nonzero = on) restricts the allowed pairs.
    Returns (O [N,d], L [N], P [N,N]); a row with no allowed key has O = 0
    and L = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = scores_head(q, k, scale, causal, block_mask)
    p, m, l = _safe_softmax(s)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(np.isfinite(m), m + np.log(l), NEG_INF)
    return o, lse, p


def backward_head(q, k, v, do, scale: float, causal: bool, block_mask=None):
    """Exact gradients of O = softmax(scale Q K^T + mask) V for one head.

    With P from the definition: dV = P^T dO; dP = dO V^T; the softmax Jacobian
    gives dS = P * (dP - rowsum(P * dP)); then dQ = scale dS K and
    dK = scale dS^T Q.  Masked entries have P = 0, hence dS = 0; a row with
    no allowed key contributes nothing.
    Returns (dQ, dK, dV, Delta) where Delta_i = sum_j P_ij dP_ij.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _, _, p = forward_head(q, k, v, scale, causal, block_mask)
    dv = p.T @ do
    dp = do @ v.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, delta


def head_block_mask(block_mask, b: int, h: int, H: int):
    """The [nb, nb] block mask of head (b, h) from a [1 or B*H, nb, nb] array (or None)."""
    if block_mask is None:
        return None
    bm = np.asarray(block_mask)
    return bm[0] if bm.shape[0] == 1 else bm[b * H + h]


def attention_forward(q, k, v, scale: float, causal: bool, block_mask=None):
    """Forward over all (batch, head) pairs of [B, H, N, d] inputs.

    `block_mask`: None, or [1 or B*H, ceil(N/128), ceil(N/128)] (nonzero = on).
    Returns O [B, H, N, d] and L [B, H, N] in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h], _ = forward_head(q[b, h], k[b, h], v[b, h], scale, causal,
                                                 head_block_mask(block_mask, b, h, H))
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool, block_mask=None):
    """Backward over all (batch, head) pairs; returns dQ, dK, dV in float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], _ = backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal,
                                                            head_block_mask(block_mask, b, h, H))
    return dq, dk, dv


def _row_scores(q_row, i: int, k, scale: float, causal: bool, block_mask):
    """Scores of query row i against all keys, -inf where the pair is not allowed."""
    s = scale * (k @ q_row)
    if causal:
        s[i + 1:] = NEG_INF
    if block_mask is not None:
        on = np.asarray(block_mask)[i // BLOCK] != 0
        s = np.where(np.repeat(on, BLOCK)[: s.shape[0]], s, NEG_INF)
    return s


def forward_rows(q_rows, rows: Sequence[int], k, v, scale: float, causal: bool, block_mask=None):
    """O and L for selected query rows of one head, each computed on its own.

    Row i needs only q_i and all of K and V: s = scale * K q_i (masked to
    j <= i when causal, and to the row's blocks under a block mask), then the
    safe softmax and the weighted sum of V.  Costs O(N d) per row, so it
    serves sampled checks at long N.  A row with no allowed key: O = 0, L = -inf.
    """
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    o = np.empty((len(rows), v.shape[1]))
    lse = np.empty(len(rows))
    for r, i in enumerate(rows):
        s = _row_scores(q_rows[r], i, k, scale, causal, block_mask)
        m = s.max()
        if m == NEG_INF:
            o[r], lse[r] = 0.0, NEG_INF
            continue
        e = np.exp(s - m)
        l = e.sum()
        o[r] = (e / l) @ v
        lse[r] = m + math.log(l)
    return o, lse


def dq_rows(q_rows, do_rows, rows: Sequence[int], k, v, scale: float, causal: bool, block_mask=None):
    """dQ for selected query rows of one head, each computed on its own.

    Row i: P_i from the row's softmax, dP_ij = dO_i . V_j,
    Delta_i = sum_j P_ij dP_ij (= dO_i . O_i), dS_ij = P_ij (dP_ij - Delta_i),
    dQ_i = scale * sum_j dS_ij K_j.  A row with no allowed key: dQ_i = 0.
    """
    q_rows, do_rows, k, v = _f64(q_rows), _f64(do_rows), _f64(k), _f64(v)
    out = np.empty((len(rows), k.shape[1]))
    for r, i in enumerate(rows):
        s = _row_scores(q_rows[r], i, k, scale, causal, block_mask)
        if s.max() == NEG_INF:
            out[r] = 0.0
            continue
        e = np.exp(s - s.max())
        p = e / e.sum()
        dp = v @ do_rows[r]
        delta = float(p @ dp)
        ds = p * (dp - delta)
        out[r] = scale * (ds @ k)
    return out


def online_softmax_row(x: Iterable[float], block_sizes: Sequence[int]):
    """Softmax statistics of one row, visiting it block by block.

    Follows the update in [video] 04:46-05:17: keep the running max m and the
    running sum l (scaled to m).  For a block with max m_b:
      m' = max(m, m_b); alpha = e^(m - m'); beta = e^(m_b - m');
      l' = alpha * l + beta * sum over the block of e^(x - m_b).
    A block whose entries are all -inf (fully masked) changes nothing.
    Returns (m, l, steps) where steps records (m, l, alpha, beta, block_sum)
    after each block.
    """
    x = np.asarray(list(x), dtype=np.float64)
    assert sum(block_sizes) == len(x)
    m, l = NEG_INF, 0.0
    steps = []
    start = 0
    for size in block_sizes:
        blk = x[start:start + size]
        start += size
        m_b = blk.max()
        if m_b == NEG_INF:
            steps.append((m, l, 1.0, 0.0, 0.0))
            continue
        block_sum = float(np.exp(blk - m_b).sum())
        m_new = max(m, m_b)
        alpha = 0.0 if m == NEG_INF else math.exp(m - m_new)
        beta = math.exp(m_b - m_new)
        l = alpha * l + beta * block_sum
        m = m_new
        steps.append((m, l, alpha, beta, block_sum))
    return m, l, steps


def online_attention_row(x: Iterable[float], v, block_sizes: Sequence[int]):
    """One output row from its scores x and V, visiting keys block by block.

    Same running statistics as `online_softmax_row`; the unnormalised output
    accumulator is rescaled with the same factors, acc' = alpha * acc +
    beta * (e^(x_block - m_b) V_block), and divided by l once at the end
    ([video] 05:17).  Returns (o, lse).
    """
    x = np.asarray(list(x), dtype=np.float64)
    v = _f64(v)
    assert sum(block_sizes) == len(x) == v.shape[0]
    m, l = NEG_INF, 0.0
    acc = np.zeros(v.shape[1])
    start = 0
    for size in block_sizes:
        blk = x[start:start + size]
        vb = v[start:start + size]
        start += size
        m_b = blk.max()
        if m_b == NEG_INF:
            continue
        e = np.exp(blk - m_b)
        m_new = max(m, m_b)
        alpha = 0.0 if m == NEG_INF else math.exp(m - m_new)
        beta = math.exp(m_b - m_new)
        l = alpha * l + beta * float(e.sum())
        acc = alpha * acc + beta * (e @ vb)
        m = m_new
    return acc / l, m + math.log(l)
