"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Inputs come from the seeded generators in workloads.py; the oracle and the GPU
consume the same bf16 (or fp32) bits.  Small cases compare every output
element; the full-size workloads compare every element of sampled heads,
sampled rows, and properties that hold at any size.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as orc
from tests.checks import check_bf16, check_f32

pytestmark = pytest.mark.gpu


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


def run_gpu(attn, inp, scale, causal, backward):
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o, lse = attn.fwd(q, k, v, scale=scale, causal=causal)
    out = {"o": o, "lse": lse}
    if backward:
        do = inp["do"].cuda()
        dq, dk, dv = attn.bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k_: t.float().cpu() for k_, t in out.items()}


def oracle_full(inp, scale, causal, backward, heads=None):
    q, k, v = (inp[x].float().numpy() for x in ("q", "k", "v"))
    do = inp["do"].float().numpy() if backward else None
    B, H = q.shape[:2]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    res = {}
    for b, h in heads:
        o, lse, _ = orc.forward_head(q[b, h], k[b, h], v[b, h], scale, causal)
        r = {"o": o, "lse": lse}
        if backward:
            dq, dk, dv, _ = orc.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
            r.update(dq=dq, dk=dk, dv=dv)
        res[(b, h)] = r
    return res


def compare_heads(got, ref, tag, fp32=False):
    for (b, h), r in ref.items():
        for name, val in r.items():
            g = got[name][b, h]
            if fp32:
                check_f32(f"{tag} {name}[{b},{h}]", g, val)
            else:
                check_bf16(f"{tag} {name}[{b},{h}]", g, val)


# ---------------------------------------------------------------- fp32 forward
@pytest.mark.parametrize("N,d,causal", [(128, 64, False), (77, 64, True), (300, 128, False), (130, 128, True)])
def test_fp32_forward(attn, N, d, causal):
    w = W.WORKLOADS[0]
    inp = W.draw(1, 2, N, d, "f32", seed=w.seed + N, backward=False)
    scale = 1 / math.sqrt(d)
    _say(f"fp32 fwd N={N} d={d} causal={causal}")
    got = run_gpu(attn, inp, scale, causal, False)
    compare_heads(got, oracle_full(inp, scale, causal, False), f"f32 N={N}", fp32=True)


@pytest.mark.parametrize("H,N,d,causal", [(16, 2048, 64, False), (16, 2048, 128, True)])
def test_fp32_forward_many_heads(attn, H, N, d, causal):
    """B*H*ceil(N/64) = 512 workgroups: the 64-row fp32 kernel (smaller problems
    take the one that splits each row block's keys over eight waves)."""
    w = W.WORKLOADS[0]
    inp = W.draw(1, H, N, d, "f32", seed=w.seed + 5 * N + d, backward=False)
    scale = 1 / math.sqrt(d)
    _say(f"fp32 fwd H={H} N={N} d={d} causal={causal}")
    got = run_gpu(attn, inp, scale, causal, False)
    compare_heads(got, oracle_full(inp, scale, causal, False, heads=[(0, 0), (0, H - 1)]), f"f32 H={H} N={N}",
                  fp32=True)


def test_fp32_small_workload_full(attn):
    w = W.BY_NAME["fp32_small"]
    inp = W.draw_workload(w)
    _say("fp32 workload 1x1x128x64")
    got = run_gpu(attn, inp, w.scale, w.causal, False)
    compare_heads(got, oracle_full(inp, w.scale, w.causal, False), "fp32_small", fp32=True)


# ---------------------------------------------------------------- bf16 small shapes
SMALL = [
    (1, 2, 1, 64, False), (1, 2, 1, 128, True), (1, 2, 17, 64, True), (2, 3, 200, 64, False),
    (1, 2, 333, 128, True), (1, 2, 512, 128, False), (2, 2, 1000, 128, True), (1, 3, 257, 64, True),
    (1, 2, 640, 64, False), (1, 1, 129, 128, False), (1, 2, 1100, 64, True),
    # the last causal length the one-tile-at-a-time d=64 forward takes, and the
    # first past it; non-causal d=64 takes it at every length, lowering wave
    # priority by quarters from 16 tiles on (ragged last tile)
    (1, 2, 512, 64, True), (1, 2, 513, 64, True), (1, 2, 513, 64, False), (1, 2, 1100, 64, False),
    # causal with B*H a multiple of 8 and an even number of 128-row tiles: the
    # forward and the dq kernel run two query tiles per workgroup, dkdv two key
    # blocks (ragged last tile)
    (1, 8, 1000, 128, True), (2, 4, 900, 64, True),
]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL)
def test_bf16_small_fwd_bwd(attn, B, H, N, d, causal):
    inp = W.draw(B, H, N, d, "bf16", seed=7 * N + d + int(causal))
    scale = 1 / math.sqrt(d)
    _say(f"bf16 fwd+bwd B={B} H={H} N={N} d={d} causal={causal}")
    got = run_gpu(attn, inp, scale, causal, True)
    compare_heads(got, oracle_full(inp, scale, causal, True), f"N={N} d={d} c={causal}")


def test_bf16_nondefault_scale(attn):
    inp = W.draw(1, 2, 300, 64, "bf16", seed=5)
    _say("bf16 scale=0.37")
    got = run_gpu(attn, inp, 0.37, True, True)
    compare_heads(got, oracle_full(inp, 0.37, True, True), "scale=0.37")


# ---------------------------------------------------------------- pinned examples on the GPU
def test_worked_example_embedded(attn):
    """Row 3 of a causal d=64 problem has scaled scores exactly [1, 2, 3, 0]
    (video page, transcript 05:49-06:52): L_3 = ln(e + e^2 + e^3 + 1)."""
    N, d = 128, 64
    inp = W.draw(1, 1, N, d, "bf16", seed=11)
    q, k = inp["q"].clone(), inp["k"].clone()
    q[0, 0, 3] = 0
    q[0, 0, 3, 0] = 8.0  # scale 1/8: score_j = k_j[0]
    for j, x in enumerate([1.0, 2.0, 3.0, 0.0]):
        k[0, 0, j] = 0
        k[0, 0, j, 0] = x
    inp.update(q=q, k=k)
    got = run_gpu(attn, inp, 0.125, True, True)
    l3 = math.log(math.exp(1) + math.exp(2) + math.exp(3) + 1)
    assert abs(l3 - 3.440190) < 1e-6
    assert abs(float(got["lse"][0, 0, 3]) - l3) < 2e-3
    p = np.exp(np.array([1.0, 2.0, 3.0, 0.0]) - l3)
    o3 = p @ inp["v"][0, 0, :4].double().numpy()
    check_bf16("worked-example O_3", got["o"][0, 0, 3], o3, rel_fro=1e-2)
    compare_heads(got, oracle_full(inp, 0.125, True, True), "worked example")


def test_causal_row_zero_exact(attn):
    inp = W.draw(1, 2, 256, 128, "bf16", seed=12)
    got = run_gpu(attn, inp, 1 / math.sqrt(128), True, True)
    assert torch.equal(got["o"][:, :, 0], inp["v"][:, :, 0].float())
    # dQ_0 = scale * P_00 (dP_00 - delta_0) K_0 vanishes exactly in the math; on the GPU
    # dP_00 (MFMA) and delta_0 (preprocess) are fp32 dot products summed in different
    # orders, so it is zero only to fp32 rounding of those sums.
    assert got["dq"][:, :, 0].abs().max() < 1e-6
    s0 = (inp["q"][:, :, 0].double() * inp["k"][:, :, 0].double()).sum(-1) / math.sqrt(128)
    assert (got["lse"][:, :, 0].double() - s0).abs().max() < 1e-4


def test_uniform_scores_give_mean(attn):
    """Q = 0: every allowed score is equal, O_i is the prefix mean of V."""
    inp = W.draw(1, 2, 300, 64, "bf16", seed=13)
    inp["q"] = torch.zeros_like(inp["q"])
    got = run_gpu(attn, inp, 0.125, True, False)
    v = inp["v"].double()
    prefix = torch.cumsum(v, dim=2) / torch.arange(1, 301, dtype=torch.float64).view(1, 1, -1, 1)
    check_bf16("uniform O", got["o"], prefix)
    lse_ref = torch.log(torch.arange(1, 301, dtype=torch.float64)).expand(1, 2, 300)
    assert (got["lse"].double() - lse_ref).abs().max() < 1e-4


def test_deterministic(attn):
    inp = W.draw(1, 4, 700, 128, "bf16", seed=14)
    a = run_gpu(attn, inp, 0.1, True, True)
    b = run_gpu(attn, inp, 0.1, True, True)
    for k_ in a:
        assert torch.equal(a[k_], b[k_]), k_


# ---------------------------------------------------------------- the five workloads
def test_workload_n2048_d64_hotrows_full(attn):
    w = W.BY_NAME["bf16_n2048_d64_hotrows"]
    inp = W.draw_workload(w)
    _say("workload 4x16x2048x64 (hot rows): GPU")
    got = run_gpu(attn, inp, w.scale, w.causal, True)
    _say("  oracle, all 64 heads")
    compare_heads(got, oracle_full(inp, w.scale, w.causal, True), w.name)


@pytest.mark.timeout(900)
def test_workload_n8192_d128_causal(attn):
    """Full-size headline problem, checked in full: every element of O, L,
    dQ, dK and dV of all 64 heads against the oracle (one head at a time, S
    and P materialised), then the 64 sampled rows and the gradient sum
    identities of the long-context check."""
    w = W.BY_NAME["bf16_n8192_d128_causal"]
    inp = W.draw_workload(w)
    _say("workload 2x32x8192x128 causal: GPU")
    got = run_gpu(attn, inp, w.scale, w.causal, True)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for i, bh in enumerate(heads):
        if i % 8 == 0:
            _say(f"  oracle, heads {i}..{min(i + 8, len(heads)) - 1} of {len(heads)}")
        compare_heads(got, oracle_full(inp, w.scale, w.causal, True, heads=[bh]), w.name)
    _sampled_rows_and_identities(got, inp, w)


def _sampled_rows_and_identities(got, inp, w, count=64):
    rows = W.sample_rows(count, w.B, w.H, w.N, seed=w.seed + 1)
    q, k, v, do = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    o_ref, l_ref, dq_ref, o_got, l_got, dq_got = [], [], [], [], [], []
    for b, h, i in rows:
        o_r, l_r = orc.forward_rows(q[b, h, [i]], [i], k[b, h], v[b, h], w.scale, w.causal)
        dq_r = orc.dq_rows(q[b, h, [i]], do[b, h, [i]], [i], k[b, h], v[b, h], w.scale, w.causal)
        o_ref.append(o_r[0]); l_ref.append(l_r[0]); dq_ref.append(dq_r[0])
        o_got.append(got["o"][b, h, i].numpy()); l_got.append(float(got["lse"][b, h, i]))
        dq_got.append(got["dq"][b, h, i].numpy())
    check_bf16(f"{w.name} sampled O rows", np.array(o_got), np.array(o_ref))
    check_bf16(f"{w.name} sampled L rows", np.array(l_got), np.array(l_ref))
    check_bf16(f"{w.name} sampled dQ rows", np.array(dq_got), np.array(dq_ref))
    # sum_j dV_j = sum_i dO_i and sum_j dK_j = 0, per head and column
    dv_sum = got["dv"].double().sum(dim=2)
    do_sum = inp["do"].double().sum(dim=2)
    dk_sum = got["dk"].double().sum(dim=2)
    dv_scale = got["dv"].double().abs().sum(dim=2)
    dk_scale = got["dk"].double().abs().sum(dim=2)
    assert ((dv_sum - do_sum).abs() <= 2e-2 * dv_scale + 1e-2).all(), (dv_sum - do_sum).abs().max()
    assert (dk_sum.abs() <= 2e-2 * dk_scale + 1e-2).all(), dk_sum.abs().max()


def test_workload_n32768_d128_causal(attn):
    w = W.BY_NAME["bf16_n32768_d128_causal"]
    inp = W.draw_workload(w)
    _say("workload 1x16x32768x128 causal: GPU")
    got = run_gpu(attn, inp, w.scale, w.causal, True)
    _say("  oracle, 64 sampled rows + identities")
    _sampled_rows_and_identities(got, inp, w)
    del got, inp
    _say("  full check at N=2048 with the same seed")
    small = W.draw_workload(w, N=2048)
    got_s = run_gpu(attn, small, w.scale, w.causal, True)
    compare_heads(got_s, oracle_full(small, w.scale, w.causal, True), f"{w.name}@2048")


def test_workload_n256_d64_short_full(attn):
    w = W.BY_NAME["bf16_n256_d64_short"]
    inp = W.draw_workload(w)
    _say("workload 256x12x256x64: GPU")
    got = run_gpu(attn, inp, w.scale, w.causal, False)
    _say("  oracle, all 3072 heads (batched)")
    q, k, v = (inp[x].double() for x in ("q", "k", "v"))
    # the oracle's forward, head by head, in chunks to bound memory
    o_ref = np.empty(tuple(q.shape))
    l_ref = np.empty(tuple(q.shape[:3]))
    qn, kn, vn = q.numpy(), k.numpy(), v.numpy()
    for b in range(w.B):
        o_b, l_b = orc.attention_forward(qn[b:b + 1], kn[b:b + 1], vn[b:b + 1], w.scale, False)
        o_ref[b], l_ref[b] = o_b[0], l_b[0]
    check_bf16(f"{w.name} O", got["o"], o_ref)
    check_bf16(f"{w.name} L", got["lse"], l_ref)


@pytest.mark.parametrize("d", [64, 128])
def test_stage_entry_points_match_attn_bwd(attn, d):
    """preprocess -> dq -> dkdv called one by one equals attn_bwd, and the exact
    delta written by the dq stage equals the oracle's sum_j P_ij dP_ij."""
    inp = W.draw(2, 2, 777, d, "bf16", seed=21)
    scale = 0.125
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o, lse = attn.fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = attn.bwd(q, k, v, o, lse, do, scale=scale, causal=True)
    delta = attn.bwd_preprocess(o, do)
    dq2, delta_exact = attn.bwd_dq(q, k, v, lse, do, delta, scale=scale, causal=True)
    dk2, dv2 = attn.bwd_dkdv(q, k, v, lse, do, delta_exact, scale=scale, causal=True)
    # the fused dq stage (what attn_bwd runs) forms delta~ itself, bit for bit
    dq3, delta_exact3 = attn.bwd_dq_fused(q, k, v, o, lse, do, scale=scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    assert torch.equal(dq3, dq2) and torch.equal(delta_exact3, delta_exact)
    qn, kn, vn, don = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    for b in range(2):
        for h in range(2):
            _, _, _, d_ref = orc.backward_head(qn[b, h], kn[b, h], vn[b, h], don[b, h], scale, True)
            err = np.abs(delta_exact[b, h].cpu().numpy() - d_ref).max()
            assert err < 1e-4 * max(1.0, np.abs(d_ref).max()), err
            o_ref, _, _ = orc.forward_head(qn[b, h], kn[b, h], vn[b, h], scale, True)
            d_from_o = (don[b, h] * o_ref).sum(1)
            np.testing.assert_allclose(d_ref, d_from_o, rtol=1e-9, atol=1e-9)
