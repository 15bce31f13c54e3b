"""attn_bwd_noalloc (the backward with its scratch in a static device array)
through the C ABI against attn_bwd with a caller workspace: bit for bit, on two
calls in a row, the first at the largest size the array takes and the second
smaller, so stale contents of the first call would show in the second."""
import math
import sys

import pytest
import torch

import workloads as W
from oracle import attention as orc
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


def _both(attn, B, H, N, d, causal, seed):
    inp = W.draw(B, H, N, d, "bf16", seed=seed)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    scale = 1 / math.sqrt(d)
    o, lse = attn.fwd(q, k, v, scale=scale, causal=causal)
    ref = attn.bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
    got = attn.bwd_noalloc(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return inp, ref, got


def test_noalloc_matches_attn_bwd_twice(attn):
    rows = attn.bwd_noalloc_max_rows()
    assert rows == 4 * 1024 * 1024
    # call 1: B*H*N = the whole scratch array
    _say("noalloc call 1: B=64 H=64 N=1024 d=64 (every row of the scratch array)")
    _, ref, got = _both(attn, 64, 64, 1024, 64, False, seed=4101)
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), f"call 1 {name} differs from attn_bwd"
    del ref, got
    torch.cuda.empty_cache()
    # call 2: smaller, causal, the other head dimension
    _say("noalloc call 2: B=1 H=2 N=300 d=128 causal")
    inp, ref, got = _both(attn, 1, 2, 300, 128, True, seed=4102)
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), f"call 2 {name} differs from attn_bwd"
    q, k, v, do = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    for h in range(2):
        dq_ref, dk_ref, dv_ref, _ = orc.backward_head(q[0, h], k[0, h], v[0, h], do[0, h], 1 / math.sqrt(128), True)
        for name, t, r in (("dq", got[0], dq_ref), ("dk", got[1], dk_ref), ("dv", got[2], dv_ref)):
            check_bf16(f"noalloc call 2 {name}[{h}]", t[0, h], r)


def test_noalloc_rejects_oversize(attn):
    """One row past the array: ATTN_ERR_SCRATCH, nothing launched, outputs untouched."""
    B, H, N, d = 1, 1, 8, 64
    t = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    outs = [torch.full_like(t, 3.0) for _ in range(3)]
    lse = torch.zeros(B, H, N, dtype=torch.float32, device="cuda")
    lib = attn.load_library()
    import ctypes

    P = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731
    rows = attn.bwd_noalloc_max_rows()
    # B = 2, H = 1, N = rows / 2 + 1: two rows too many, N itself within the 2^22 limit; the
    # call is rejected on its sizes alone, so the small buffers are never read
    st = lib.attn_bwd_noalloc(P(t), P(t), P(t), P(t), P(lse), P(t), *(P(x) for x in outs), 2, 1, rows // 2 + 1, d,
                              1, 0.125, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 4  # ATTN_ERR_SCRATCH
    for x in outs:
        assert (x == 3.0).all()
