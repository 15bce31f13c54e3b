"""GPU parity of decode attention against a KV cache (split-KV partial kernel +
merge kernel, through the C ABI) against the fp64 oracle.

Shapes cover one and several queries, caches shorter than one 512-key chunk,
exactly one chunk, several chunks with a ragged last one, causal (bottom-right
aligned) and not, d 64 and 128, and a 32768-key cache.
"""
import math
import sys

import pytest
import torch

import workloads as W
from oracle import decode as dec
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


def draw(B, H, Nq, Nk, d, seed):
    """q [B,H,Nq,d] and the cache k, v [B,H,Nk,d], bf16 N(0,1), from the seeded generators."""
    cache = W.draw(B, H, Nk, d, "bf16", seed=seed, backward=False)
    q = W.draw(B, H, Nq, d, "bf16", seed=seed + 1, backward=False)["q"]
    return q, cache["k"], cache["v"]


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 100), (2, 700), (4, 512), (8, 513), (3, 1500), (1, 2049), (6, 2500), (7, 33), (8, 8)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_oracle(attn, Nq, Nk, d, causal):
    seed = 5000 + Nq * 31 + Nk + d
    _say(f"decode Nq={Nq} Nk={Nk} d={d} causal={causal} seed={seed}")
    B, H = 2, 3
    q, k, v = draw(B, H, Nq, Nk, d, seed)
    scale = 1 / math.sqrt(d)
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = dec.attention_decode(q.float().numpy(), k.float().numpy(), v.float().numpy(), scale, causal)
    check_bf16(f"decode o Nq={Nq} Nk={Nk} d={d} c={causal}", o.float().cpu(), o_ref)
    check_bf16(f"decode lse Nq={Nq} Nk={Nk} d={d} c={causal}", lse.cpu(), lse_ref)


def test_long_cache(attn):
    B, H, Nq, Nk, d = 1, 8, 2, 32768, 128
    _say(f"decode long B={B} H={H} Nq={Nq} Nk={Nk}")
    q, k, v = draw(B, H, Nq, Nk, d, 5900)
    scale = 1 / math.sqrt(d)
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = dec.attention_decode(q.float().numpy(), k.float().numpy(), v.float().numpy(), scale, True)
    check_bf16("decode long o", o.float().cpu(), o_ref)
    check_bf16("decode long lse", lse.cpu(), lse_ref)


def test_decode_is_deterministic(attn):
    q, k, v = draw(1, 2, 4, 3000, 64, 5950)
    a = attn.decode(q.cuda(), k.cuda(), v.cuda(), causal=True)
    b = attn.decode(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("B,H,Nq,Nk,d", [(1, 8, 4, 3000, 128), (2, 3, 2, 100, 64), (1, 4, 1, 5000, 128)])
def test_decode_replays_in_a_graph(attn, B, H, Nq, Nk, d):
    """attn_decode enqueues kernels only (no allocation, no memset, no host sync), so it can be captured in a
    HIP graph; every replay, with new queries copied in between, matches an eager call bit for bit.  The
    shapes take the merged path (several chunks) and the single-chunk path."""
    _say(f"decode graph B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    q, k, v = draw(B, H, Nq, Nk, d, 5970 + Nk)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=qd.device)
    ws = torch.empty(max(attn.decode_workspace_bytes(B, H, Nq, Nk, d), 1), dtype=torch.uint8, device=qd.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        attn.decode(qd, kd, vd, causal=True, out=o, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn.decode(qd, kd, vd, causal=True, out=o, lse=lse, workspace=ws)
    for r in range(4):
        qn = draw(B, H, Nq, 1, d, 6100 + 17 * r)[0]
        qd.copy_(qn.cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo, el = attn.decode(qd, kd, vd, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el), f"replay {r}"
