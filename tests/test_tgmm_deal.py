"""The tgmm GEMM's work-item deal (host model in tests/tgmm_deal.py): every
item reaches exactly one block, and the deal evens out the blocks' modelled
loads where the round-robin deal leaves the heavy experts' remainders on a
few blocks."""
import numpy as np
import pytest

import workloads as W
from tests import tgmm_deal as D

SHAPES = [(3, 7168, 2048), (3, 7168, 4096), (3, 2048, 7168), (3, 384, 2048), (2, 2048, 768), (0, 128, 256)]


def _sizes(cfg):
    gs = np.asarray(W.group_sizes(cfg))
    return gs, int(W.SHAPES[cfg]["M"]) if "M" in W.SHAPES[cfg] else int(gs.sum())


@pytest.mark.parametrize("cfg,K,N", SHAPES)
def test_every_item_dealt_once(cfg, K, N):
    gs, M = _sizes(cfg)
    G = len(gs)
    _, _, per_g, nb = D.geometry(G, K, N, 256)
    offs = D.deal(gs, M, K, N, 256)
    assert offs is not None and all(0 <= o < nb for o in offs)
    # the GEMM block's walk: first item (b - offset) mod nb, then every nb-th
    seen = np.zeros((G, per_g), int)
    for b in range(nb):
        for g in range(G):
            j = (b - offs[g]) % nb
            while j < per_g:
                seen[g, j] += 1
                j += nb
    assert (seen == 1).all()


@pytest.mark.parametrize("cfg,K,N", [(3, 7168, 2048), (3, 7168, 4096), (3, 2048, 7168)])
def test_deal_balances_the_bench_routing(cfg, K, N):
    gs, M = _sizes(cfg)
    G = len(gs)
    _, _, per_g, nb = D.geometry(G, K, N, 256)
    dealt = D.block_loads(gs, M, K, N, 256, D.deal(gs, M, K, N, 256))
    rr = D.block_loads(gs, M, K, N, 256, D.round_robin(G, per_g, nb))
    assert dealt.sum() == rr.sum()
    assert dealt.max() / dealt.mean() < 1.01
    assert dealt.max() <= rr.max()


def test_deal_on_random_zipf_routings():
    rng = np.random.default_rng(7)
    for _ in range(5):
        p = 1.0 / np.arange(1, 33) ** 1.1
        rng.shuffle(p)
        gs = rng.multinomial(19661, p / p.sum())
        M = 32768
        dealt = D.block_loads(gs, M, 7168, 2048, 256, D.deal(gs, M, 7168, 2048, 256))
        rr = D.block_loads(gs, M, 7168, 2048, 256, D.round_robin(32, 448, 256))
        assert dealt.max() / dealt.mean() < 1.02
        assert dealt.max() <= rr.max()


def test_ties_and_limits():
    # equal experts (one 64-row pair each): the windows fill from offset 0 in expert order
    gs = np.full(8, 64)
    offs = D.deal(gs, 512, 256, 256, 256)        # per_g = 2, nb = 16: windows of 2 blocks
    assert offs == [0, 2, 4, 6, 8, 10, 12, 14]
    # too many experts: the library keeps the round-robin deal
    assert D.deal(np.ones(257, int), 257, 256, 128, 256) is None
