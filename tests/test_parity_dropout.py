"""GPU parity of attention with dropout: the HIP path through the C ABI against
the fp64 oracle with the same Philox4x32-10 decisions (same seed, same rate).

The kernels regenerate the keep decisions in the forward, dq and dkdv passes;
any difference in the generator, the counter mapping or the byte selection
shows up as a large error in O or in the gradients.  At rate 0 the dropout
kernels must reproduce the plain ones bit for bit.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dropout as drp
from tests.checks import check_bf16

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


def run(attn, inp, p, seed, scale, causal):
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o, lse = attn.fwd_dropout(q, k, v, p, seed, scale=scale, causal=causal)
    dq, dk, dv = attn.bwd_dropout(q, k, v, o, lse, do, p, seed, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return {n: t.float().cpu() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}


@pytest.mark.parametrize("N,d", [(128, 64), (200, 64), (333, 128), (256, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_small_dropout_matches_oracle(attn, N, d, causal, p):
    seed = 0x5EED0000 + N * 7 + d + (1 << 40)
    _say(f"dropout N={N} d={d} causal={causal} p={p} seed={seed:#x}")
    B, H = 1, 2
    inp = W.draw(B, H, N, d, "bf16", seed=4000 + N + d)
    scale = 1 / math.sqrt(d)
    got = run(attn, inp, p, seed, scale, causal)
    t = drp.threshold(p)
    q, k, v, do = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    for h in range(H):
        o, lse, _, _ = drp.forward_head_dropout(q[0, h], k[0, h], v[0, h], scale, causal, seed, t, h)
        dq, dk, dv, _ = drp.backward_head_dropout(q[0, h], k[0, h], v[0, h], do[0, h], scale, causal, seed, t, h)
        tag = f"N={N} d={d} c={causal} p={p} h={h}"
        for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            check_bf16(f"{tag} {name}", got[name][0, h], ref)


@pytest.mark.parametrize("N,d,causal", [(300, 64, True), (512, 128, False)])
def test_rate_zero_equals_plain_kernels(attn, N, d, causal):
    inp = W.draw(1, 2, N, d, "bf16", seed=4100 + N)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o_p, l_p = attn.fwd(q, k, v, causal=causal)
    o_d, l_d = attn.fwd_dropout(q, k, v, 0.0, 12345, causal=causal)
    g_p = attn.bwd(q, k, v, o_p, l_p, do, causal=causal)
    g_d = attn.bwd_dropout(q, k, v, o_d, l_d, do, 0.0, 12345, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_d) and torch.equal(l_p, l_d)
    for a, b in zip(g_p, g_d):
        assert torch.equal(a, b)


def test_seed_changes_output_and_same_seed_repeats(attn):
    inp = W.draw(1, 1, 256, 64, "bf16", seed=4200)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o1, _ = attn.fwd_dropout(q, k, v, 0.3, 1)
    o2, _ = attn.fwd_dropout(q, k, v, 0.3, 1)
    o3, _ = attn.fwd_dropout(q, k, v, 0.3, 2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert not torch.equal(o1, o3)


def test_longer_causal_dropout_matches_oracle(attn):
    """N = 2048, d = 128, causal, rate 0.1: every element of two heads."""
    B, H, N, d, p = 1, 2, 2048, 128, 0.1
    seed = 0xC0FFEE1234
    _say(f"dropout long N={N} d={d} p={p}")
    inp = W.draw(B, H, N, d, "bf16", seed=4300)
    scale = 1 / math.sqrt(d)
    got = run(attn, inp, p, seed, scale, True)
    t = drp.threshold(p)
    q, k, v, do = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    for h in range(H):
        o, lse, _, _ = drp.forward_head_dropout(q[0, h], k[0, h], v[0, h], scale, True, seed, t, h)
        dq, dk, dv, _ = drp.backward_head_dropout(q[0, h], k[0, h], v[0, h], do[0, h], scale, True, seed, t, h)
        for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            check_bf16(f"long h={h} {name}", got[name][0, h], ref)
