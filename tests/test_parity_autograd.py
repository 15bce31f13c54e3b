"""The autograd wrapper (exact_io_aware_23_amd.attention): its forward is
attn_fwd and its gradients are attn_bwd's, bit for bit, and both match the
fp64 oracle within the bf16 gate."""
import math

import pytest
import torch

import workloads as W
from oracle import attention as orc
from tests.checks import check_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_io_aware_23_amd as A

    A.load_library()
    return A


@pytest.mark.parametrize("N,d,causal", [(200, 64, True), (333, 128, False)])
def test_autograd_matches_entry_points_and_oracle(attn, N, d, causal):
    inp = W.draw(1, 2, N, d, "bf16", seed=9000 + N)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = attn.attention(qg, kg, vg, causal=causal)
    o.backward(do)
    o_ref, lse = attn.fwd(q, k, v, causal=causal)
    dq, dk, dv = attn.bwd(q, k, v, o_ref, lse, do, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(qg.grad, dq) and torch.equal(kg.grad, dk) and torch.equal(vg.grad, dv)
    scale = 1 / math.sqrt(d)
    a = [inp[x].float().numpy() for x in ("q", "k", "v", "do")]
    for h in range(2):
        o_h, _, _ = orc.forward_head(a[0][0, h], a[1][0, h], a[2][0, h], scale, causal)
        g = orc.backward_head(a[0][0, h], a[1][0, h], a[2][0, h], a[3][0, h], scale, causal)
        check_bf16(f"autograd O h={h}", o[0, h].float().cpu(), o_h)
        for name, got, ref in (("dQ", qg.grad, g[0]), ("dK", kg.grad, g[1]), ("dV", vg.grad, g[2])):
            check_bf16(f"autograd {name} h={h}", got[0, h].float().cpu(), ref)
