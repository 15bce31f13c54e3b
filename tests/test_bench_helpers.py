"""CPU checks of bench.py's host arithmetic."""
import importlib.util
import os

import pytest
import torch

from oracle import attention as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("N", [128, 300, 513])
@pytest.mark.parametrize("causal", [False, True])
def test_allowed_pair_count_matches_the_element_mask(N, causal):
    """The FLOP count of the block-sparse bench counts the pairs the oracle allows."""
    nb = -(-N // 128)
    mask = (torch.rand((3, nb, nb), generator=torch.Generator().manual_seed(N)) < 0.5).to(torch.uint8)
    got = _bench().allowed_pairs_per_head(mask, N, causal)
    ref = [int(orc.allowed_pairs(N, N, causal, mask[h].numpy()).sum()) for h in range(3)]
    assert got.tolist() == ref


def test_dense_pair_count_matches_flop_formula():
    """With every block on, 4 d * pairs is the dense forward FLOP count (halved plus the diagonal when causal)."""
    N = 1000
    nb = -(-N // 128)
    ones = torch.ones((1, nb, nb), dtype=torch.uint8)
    b = _bench()
    assert int(b.allowed_pairs_per_head(ones, N, False)) == N * N
    assert int(b.allowed_pairs_per_head(ones, N, True)) == N * (N + 1) // 2
