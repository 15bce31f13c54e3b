"""GPU parity of block-sparse attention: the HIP path through the C ABI against
the fp64 oracle with the same 128 x 128 block mask.

Masks are drawn from a seeded generator; inputs from workloads.py.  Small
shapes compare every element (ragged N, causal, shared and per-head masks,
row blocks with no allowed key); a longer shape compares sampled rows and
the gradient identities.  With every block on, the block-sparse kernels must
reproduce the dense ones.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as orc
from tests.checks import check_bf16

pytestmark = pytest.mark.gpu

BLK = 128


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def attn():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_io_aware_23_amd as A

    A.load_library()
    return A


def draw_mask(heads, N, density, seed, causal, dead_row_block=None):
    """uint8 [heads, nb, nb]: each block on with probability `density`; causal
    masks keep the diagonal block on (except in `dead_row_block`, whose row of
    blocks is switched off entirely)."""
    nb = -(-N // BLK)
    g = torch.Generator().manual_seed(seed)
    m = (torch.rand((heads, nb, nb), generator=g) < density).to(torch.uint8)
    if causal:
        idx = torch.arange(nb)
        m[:, idx, idx] = 1
    if dead_row_block is not None:
        m[:, dead_row_block, :] = 0
    return m


def check_lse(name, got, ref):
    got = got.double().numpy()
    dead = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), dead), f"{name}: -inf rows differ"
    if (~dead).any():
        check_bf16(name, got[~dead], ref[~dead])


def run_sparse(attn, inp, mask, scale, causal, backward=True):
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    m = mask.cuda()
    o, lse = attn.fwd_block_sparse(q, k, v, m, scale=scale, causal=causal)
    out = {"o": o, "lse": lse}
    if backward:
        do = inp["do"].cuda()
        dq, dk, dv = attn.bwd_block_sparse(q, k, v, o, lse, do, m, scale=scale, causal=causal)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k_: t.float().cpu() for k_, t in out.items()}


@pytest.mark.parametrize("B,H,N,d", [(1, 2, 256, 64), (2, 2, 300, 64), (1, 3, 384, 128), (1, 2, 257, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shared", [False, True])
def test_small_block_sparse_matches_oracle(attn, B, H, N, d, causal, shared):
    seed = 3000 + N + d + 7 * causal + 11 * shared
    _say(f"block-sparse B={B} H={H} N={N} d={d} causal={causal} shared={shared} seed={seed}")
    inp = W.draw(B, H, N, d, "bf16", seed=seed)
    mask = draw_mask(1 if shared else B * H, N, 0.5, seed, causal, dead_row_block=1)
    scale = 1 / math.sqrt(d)
    got = run_sparse(attn, inp, mask, scale, causal)
    q, k, v, do = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    for b in range(B):
        for h in range(H):
            hm = orc.head_block_mask(mask.numpy(), b, h, H)
            o, lse, _ = orc.forward_head(q[b, h], k[b, h], v[b, h], scale, causal, hm)
            dq, dk, dv, _ = orc.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, hm)
            tag = f"N={N} d={d} c={causal} [{b},{h}]"
            check_bf16(f"{tag} o", got["o"][b, h], o)
            check_lse(f"{tag} lse", got["lse"][b, h], lse)
            for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
                check_bf16(f"{tag} {name}", got[name][b, h], ref)
            # rows of the dead block row: exactly zero output and dQ
            dead = slice(BLK, min(N, 2 * BLK))
            assert torch.all(got["o"][b, h][dead] == 0) and torch.all(got["dq"][b, h][dead] == 0)
            assert torch.all(torch.isneginf(got["lse"][b, h][dead]))


def _within_one_bf16_ulp(a, b):
    """|a - b| at most one bf16 spacing at max(|a|, |b|) (8 significant bits)."""
    a32, b32 = a.float(), b.float()
    return bool(torch.all((a32 - b32).abs() <= torch.maximum(a32.abs(), b32.abs()) * 2.0**-7 + 1e-6))


@pytest.mark.parametrize("N,d,causal", [(384, 64, False), (300, 128, True), (1000, 128, True)])
def test_all_blocks_on_equals_dense(attn, N, d, causal):
    """Every block on: the block-sparse kernels visit the same tiles in the same
    order as the dense ones, so the results are bit-identical.  One exception:
    the dense dK, dV kernel at d = 64, not causal, may split each key group's
    queries over two waves and add the two partial sums at the end (when the
    launch would otherwise end with a mostly empty round); that changes the fp32
    summation order, so there dK and dV agree within one bf16 unit in the last
    place."""
    _say(f"all-on mask N={N} d={d} causal={causal}")
    inp = W.draw(1, 2, N, d, "bf16", seed=3100 + N)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    nb = -(-N // BLK)
    ones = torch.ones((1, nb, nb), dtype=torch.uint8, device="cuda")
    o_d, l_d = attn.fwd(q, k, v, causal=causal)
    o_s, l_s = attn.fwd_block_sparse(q, k, v, ones, causal=causal)
    g_d = attn.bwd(q, k, v, o_d, l_d, do, causal=causal)
    g_s = attn.bwd_block_sparse(q, k, v, o_s, l_s, do, ones, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_s) and torch.equal(l_d, l_s)
    dq_d, dk_d, dv_d = g_d
    dq_s, dk_s, dv_s = g_s
    assert torch.equal(dq_d, dq_s)
    for a, b in ((dk_d, dk_s), (dv_d, dv_s)):
        if d == 64 and not causal:
            assert _within_one_bf16_ulp(a, b)
        else:
            assert torch.equal(a, b)


def test_all_blocks_off(attn):
    """No block on: O = 0, L = -inf, and every gradient is zero."""
    N, d = 260, 64
    inp = W.draw(1, 2, N, d, "bf16", seed=3200)
    zeros = torch.zeros((1, 3, 3), dtype=torch.uint8)
    got = run_sparse(attn, inp, zeros, 0.125, False)
    assert torch.all(got["o"] == 0) and torch.all(torch.isneginf(got["lse"]))
    for name in ("dq", "dk", "dv"):
        assert torch.all(got[name] == 0), name


def test_long_block_sparse_sampled_rows(attn):
    """N = 4096, d = 128, causal, half the blocks on: sampled rows of O, L and dQ
    against the row-local oracle, and the identities sum_j dV_j = sum of dO over
    rows with an allowed key, sum_j dK_j = 0, per head."""
    B, H, N, d = 1, 4, 4096, 128
    seed = 3300
    _say(f"block-sparse long B={B} H={H} N={N} d={d} causal seed={seed}")
    inp = W.draw(B, H, N, d, "bf16", seed=seed)
    mask = draw_mask(B * H, N, 0.5, seed, True)
    scale = 1 / math.sqrt(d)
    got = run_sparse(attn, inp, mask, scale, True)
    q, k, v, do = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    rows = sorted(set(int(r) for r in np.random.default_rng(seed).integers(0, N, size=24)) | {0, N - 1})
    for h in range(H):
        hm = mask[h].numpy()
        o_r, lse_r = orc.forward_rows(q[0, h, rows], rows, k[0, h], v[0, h], scale, True, hm)
        dq_r = orc.dq_rows(q[0, h, rows], do[0, h, rows], rows, k[0, h], v[0, h], scale, True, hm)
        check_bf16(f"long o h={h}", got["o"][0, h][rows], o_r)
        check_lse(f"long lse h={h}", got["lse"][0, h][rows], lse_r)
        check_bf16(f"long dq h={h}", got["dq"][0, h][rows], dq_r)
        live = torch.isfinite(got["lse"][0, h])
        sum_dv = got["dv"][0, h].double().sum(0)
        sum_do = inp["do"][0, h].double()[live].sum(0)
        check_bf16(f"long sum dV h={h}", sum_dv, sum_do.numpy(), rel_fro=5e-2)
        sum_dk = got["dk"][0, h].double().sum(0).abs().max().item()
        assert sum_dk <= 2e-2 + 1e-2 * got["dk"][0, h].abs().max().item() * math.sqrt(N), sum_dk
