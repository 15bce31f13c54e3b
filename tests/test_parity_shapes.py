"""GPU parity across the shapes at which the launchers choose between kernels.

Every case runs the forward and backward through the C ABI and compares the
first and last head element by element with the fp64 oracle (the same
tolerances as tests/test_parity.py).  The comment on each shape names the
kernels the launchers pick for it; the choices depend on B*H, on the number of
128-row tiles n = ceil(N / 128), on d and on causality:
  * forward: d = 64 non-causal, or causal with N <= 512: one tile at a time;
    causal with B*H a multiple of 8 and n even, n <= 64: two query tiles per
    workgroup (pair); otherwise the pipelined one-tile-per-workgroup kernel;
  * dq: pair when causal, B*H a multiple of 8, n even and n <= 64;
  * dkdv: pair when causal, B*H a multiple of 8, n even and n <= 32; at d = 64
    non-causal the query split when the unsplit launch would take fewer than
    four rounds of resident workgroups and leave the last at most half full
    (on a 256-CU GPU with three such workgroups per CU: 768 per round).
"""
import math
import sys

import pytest
import torch

import workloads as W
from oracle import attention as orc
from tests.checks import check_bf16

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 3, 127, 64, False),     # one-tile forward; dkdv query split (9 workgroups), ragged
    (2, 4, 129, 128, True),     # B*H = 8, n = 2: pair forward, dq and dkdv, ragged
    (1, 8, 255, 64, True),      # d = 64 causal N <= 512: one-tile forward; dq and dkdv pairs
    (1, 8, 513, 64, True),      # d = 64 causal N > 512, n = 5 (odd): pipelined forward, no pairs
    (2, 4, 1025, 64, False),    # query split with an odd number (33) of 32-query blocks
    (1, 3, 1100, 64, False),    # query split, 35 query blocks, B*H = 3
    (4, 125, 128, 64, False),   # B*H = 500: 500 workgroups, last round more than half full: no split
    (2, 8, 1536, 128, True),    # B*H = 16, n = 12: pairs everywhere
    (1, 8, 4352, 128, True),    # n = 34: pair forward and dq, dkdv one block per workgroup (n > 32)
    (1, 5, 2047, 128, False),   # non-causal d = 128, ragged, B*H = 5
    (3, 1, 511, 128, True),     # B*H = 3: no pairs at d = 128
    (1, 16, 1023, 64, True),    # d = 64 causal pairs past N = 512, ragged
]


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


@pytest.mark.parametrize("B,H,N,d,causal", SHAPES)
def test_dispatch_shapes(attn, B, H, N, d, causal):
    _say(f"shape B={B} H={H} N={N} d={d} causal={causal}")
    inp = W.draw(B, H, N, d, "bf16", seed=9100 + 13 * N + d + int(causal) + 7 * B * H)
    scale = 1 / math.sqrt(d)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o, lse = attn.fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = attn.bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    got = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    qn, kn, vn, don = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    for b, h in sorted({(0, 0), (B - 1, H - 1)}):
        ro, rl, _ = orc.forward_head(qn[b, h], kn[b, h], vn[b, h], scale, causal)
        rdq, rdk, rdv, _ = orc.backward_head(qn[b, h], kn[b, h], vn[b, h], don[b, h], scale, causal)
        tag = f"B={B} H={H} N={N} d={d} c={causal} [{b},{h}]"
        for name, ref in (("o", ro), ("lse", rl), ("dq", rdq), ("dk", rdk), ("dv", rdv)):
            check_bf16(f"{tag} {name}", got[name][b, h].float().cpu(), ref)
