"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the benchmark and the oracle's callers.
It draws random tensors and shapes them; it holds none of the attention
arithmetic, so the oracle and the HIP path stay independent of each other.

The pages measure on transformer training at sequence lengths from about 1K
to 64K with head dimension 64 or 128 (the FlashAttention talk transcript on
youtube-distilled, background and empirical-results parts; the video page
"What is Flash Attention?", transcript 01:04 and 09:29). Their datasets and
trained models are not available, so i.i.d. N(0, 1) tensors of those shapes
stand in for them.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype, mask and how inputs are drawn."""

    name: str
    index: int  # position in the workload list; the RNG seed is 1000 + index
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "bf16" or "f32"
    causal: bool
    backward: bool  # whether the workload includes the backward pass
    hot_row_fraction: float = 0.0  # fraction of query rows multiplied by hot_row_factor
    hot_row_factor: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    def fwd_flops(self) -> float:
        """Algorithmic forward FLOPs: 4*B*H*N^2*d, halved under the causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """Algorithmic backward FLOPs: 2.5x the forward (five N^2*d contractions)."""
        return 2.5 * self.fwd_flops()

    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def fwd_bytes(self) -> float:
        """Algorithmic forward HBM bytes: read Q, K, V; write O and the fp32 row statistic."""
        E = self.B * self.H * self.N * self.d
        return 4.0 * E * self.elem_bytes() + 4.0 * self.B * self.H * self.N


WORKLOADS = [
    Workload("fp32_small", 0, 1, 1, 128, 64, "f32", False, False),
    Workload("bf16_n2048_d64_hotrows", 1, 4, 16, 2048, 64, "bf16", False, True, 0.01, 20.0),
    Workload("bf16_n8192_d128_causal", 2, 2, 32, 8192, 128, "bf16", True, True),
    Workload("bf16_n32768_d128_causal", 3, 1, 16, 32768, 128, "bf16", True, True),
    Workload("bf16_n256_d64_short", 4, 256, 12, 256, 64, "bf16", False, False),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def draw(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
         backward: bool = True, hot_row_fraction: float = 0.0, hot_row_factor: float = 1.0):
    """Draw Q, K, V (and dO) as CPU tensors of shape [B, H, N, d].

    Values are N(0, 1) in fp32 from torch's CPU generator seeded with `seed`,
    drawn in the order Q, K, V, dO.  When `hot_row_fraction` > 0, that fraction
    of the B*H*N query rows (chosen without replacement from the same
    generator, after dO) is multiplied by `hot_row_factor` before the final
    rounding to `dtype` (round-to-nearest-even for bf16).
    Returns a dict with keys q, k, v, do (do is None when backward is False).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32) if backward else None
    if hot_row_fraction > 0:
        rows = B * H * N
        n_hot = int(math.floor(hot_row_fraction * rows))
        idx = torch.randperm(rows, generator=g)[:n_hot]
        q.view(rows, d)[idx] *= hot_row_factor
    td = torch_dtype(dtype)
    out = {"q": q.to(td), "k": k.to(td), "v": v.to(td), "do": do.to(td) if do is not None else None}
    return out


def draw_workload(w: Workload, N: int | None = None, H: int | None = None, B: int | None = None,
                  seed: int | None = None):
    """Draw the inputs of workload `w`, optionally at another B, H or N (same recipe)."""
    return draw(B if B is not None else w.B, H if H is not None else w.H,
                N if N is not None else w.N, w.d, w.dtype,
                seed if seed is not None else w.seed, backward=True,
                hot_row_fraction=w.hot_row_fraction, hot_row_factor=w.hot_row_factor)


def sample_rows(count: int, B: int, H: int, N: int, seed: int):
    """`count` distinct (b, h, i) query rows drawn uniformly from a generator seeded with `seed`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    flat = torch.randperm(B * H * N, generator=g)[:count].tolist()
    out = []
    for f in flat:
        b, rem = divmod(f, H * N)
        h, i = divmod(rem, N)
        out.append((b, h, i))
    return out


def draw_fp8(B: int, H: int, N: int, d: int, seed: int = 0):
    """Q, K, V as OCP e4m3 codes (uint8 CPU tensors [B, H, N, d]) with one
    fp32 scale per tensor.

    The same N(0, 1) fp32 draws as `draw` (order Q, K, V) are divided by
    amax / 448 (so the largest magnitude maps to the top of the e4m3 range)
    and rounded by torch's float8_e4m3fn cast.  The value of code x of Q is
    dq * e4m3(x).  Returns a dict with q8, k8, v8 and dq, dk, dv (floats).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (B, H, N, d)
    out = {}
    for name in ("q", "k", "v"):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        amax = float(x.abs().max()) if x.numel() else 1.0
        descale = float(torch.tensor(max(amax, 1e-30) / 448.0, dtype=torch.float32))
        out[name + "8"] = (x / descale).to(torch.float8_e4m3fn).view(torch.uint8)
        out["d" + name] = descale
    return out
