"""GPU parity at the largest sizes the entry points accept.

One (batch, head) slab is addressed with 32-bit byte offsets, so the entry
points take N <= 2^22 (attention) and Nk <= 2^23 (decode).  These tests run
exactly those sizes with B = H = 1, so a slab spans 1 GiB (bf16, d = 128) or
2 GiB (decode K and V): any offset that overflowed would read the wrong rows.

Checks, against the fp64 oracle on the same bits:
  * bf16 forward + backward at N = 2^22, d = 128, causal: O, L and dQ on
    sampled rows (first, last and random ones); dK and dV through the
    identities sum_j dV_j = sum_i dO_i and sum_j dK_j = 0 (a dK or dV row
    needs the statistics of every query row, out of reach on the CPU here);
  * the FP8 forward at N = 2^22: O and L on sampled rows, with the FP8
    tolerance of its own parity tests;
  * decode with 1 and 8 queries against 2^23 cached keys: every output.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as orc
from oracle import decode as dec
from oracle import fp8 as orc8
from tests.checks import check_bf16
from tests.test_parity_fp8 import S_REL, check_fp8

pytestmark = pytest.mark.gpu

N_MAX = 1 << 22
NK_MAX = 1 << 23


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


def _rows(n, count, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    pick = torch.randint(1, n - 1, (count,), generator=g).tolist()
    return sorted(set([0, 1, 127, 128, n - 129, n - 1] + pick))


def test_bf16_fwd_bwd_at_max_n(attn):
    N, d = N_MAX, 128
    scale = 1 / math.sqrt(d)
    _say(f"max-size bf16 fwd+bwd N={N} d={d} causal: drawing inputs")
    inp = W.draw(1, 1, N, d, "bf16", seed=8100)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    _say("  GPU forward + backward")
    o, lse = attn.fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = attn.bwd(q, k, v, o, lse, do, scale=scale, causal=True)
    torch.cuda.synchronize()
    o, lse, dq = o[0, 0].float().cpu().numpy(), lse[0, 0].cpu().numpy(), dq[0, 0].float().cpu().numpy()
    dv_sum = dv[0, 0].double().sum(dim=0).cpu()
    dv_scale = dv[0, 0].double().abs().sum(dim=0).cpu()
    dk_sum = dk[0, 0].double().sum(dim=0).cpu()
    dk_scale = dk[0, 0].double().abs().sum(dim=0).cpu()
    del q, k, v, do, dk, dv
    rows = _rows(N, 6, 8101)
    _say(f"  oracle on rows {rows}")
    q64 = inp["q"][0, 0, rows].double().numpy()
    do64 = inp["do"][0, 0, rows].double().numpy()
    k64 = inp["k"][0, 0].double().numpy()
    v64 = inp["v"][0, 0].double().numpy()
    o_r, l_r = orc.forward_rows(q64, rows, k64, v64, scale, True)
    dq_r = orc.dq_rows(q64, do64, rows, k64, v64, scale, True)
    check_bf16("max N O rows", o[rows], o_r)
    check_bf16("max N L rows", lse[rows], l_r)
    check_bf16("max N dQ rows", dq[rows], dq_r)
    do_sum = inp["do"][0, 0].double().sum(dim=0)
    assert ((dv_sum - do_sum).abs() <= 2e-2 * dv_scale + 1e-2).all(), (dv_sum - do_sum).abs().max()
    assert (dk_sum.abs() <= 2e-2 * dk_scale + 1e-2).all(), dk_sum.abs().max()


def test_fp8_fwd_at_max_n(attn):
    N, d = N_MAX, 128
    scale = 1 / math.sqrt(d)
    _say(f"max-size fp8 fwd N={N} d={d} causal: drawing inputs")
    inp = W.draw_fp8(1, 1, N, d, seed=8200)
    q8, k8, v8 = (inp[x].cuda() for x in ("q8", "k8", "v8"))
    o, lse = attn.fwd_fp8(q8, k8, v8, inp["dq"], inp["dk"], inp["dv"], scale=scale, causal=True)
    torch.cuda.synchronize()
    o, lse = o[0, 0].float().cpu().numpy(), lse[0, 0].cpu().numpy()
    del q8, k8, v8
    rows = _rows(N, 6, 8201)
    _say(f"  oracle on rows {rows}")
    ref = orc8.forward_rows_fp8(inp["q8"][0, 0, rows].numpy(), rows, inp["k8"][0, 0].numpy(),
                                inp["v8"][0, 0].numpy(), inp["dq"], inp["dk"], inp["dv"], scale, True, s_rel=S_REL)
    check_fp8("fp8 max N", o[rows], lse[rows], *ref)


@pytest.mark.parametrize("Nq", [1, 8])
def test_decode_at_max_nk(attn, Nq):
    Nk, d = NK_MAX, 128
    scale = 1 / math.sqrt(d)
    _say(f"max-size decode Nq={Nq} Nk={Nk} d={d} causal: drawing inputs")
    cache = W.draw(1, 1, Nk, d, "bf16", seed=8300, backward=False)
    qd = W.draw(1, 1, Nq, d, "bf16", seed=8301 + Nq, backward=False)["q"]
    o, lse = attn.decode(qd.cuda(), cache["k"].cuda(), cache["v"].cuda(), scale=scale, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = dec.decode_head(qd[0, 0].double().numpy(), cache["k"][0, 0].double().numpy(),
                                     cache["v"][0, 0].double().numpy(), scale, True)
    check_bf16(f"decode max Nk o Nq={Nq}", o[0, 0].float().cpu(), o_ref)
    check_bf16(f"decode max Nk lse Nq={Nq}", lse[0, 0].cpu(), lse_ref)
