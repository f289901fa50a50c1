"""GPU test of the allocation-free forward gmm_fp8_fwd_noalloc: through the C
ABI it must give gmm_fp8_fwd's result bit for bit (same kernels; the
quantized activations live in the library's fixed scratch instead of the
caller's workspace), on two calls in a row, the second with a smaller input,
leaving rows past the valid prefix untouched; an input larger than the
scratch is refused."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FA1


def _inputs(seed, M, K, N, G):
    r = np.random.default_rng(seed)
    lhs = W.to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    codes = np.empty((G, K, N), np.uint8)
    scale = np.empty((G, N), np.float32)
    for g in range(G):
        codes[g], scale[g] = W.weight_codes(r.standard_normal((K, N)).astype(np.float32) * 0.02)
    cuts = np.sort(r.integers(0, M - 17, G - 1))
    gs = np.diff(np.concatenate([[0], cuts, [M - 17]])).astype(np.int32)   # 17 stale rows at the end
    W.fill_garbage(lhs, int(gs.sum()))
    dev = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16
                     else torch.from_numpy(a)).cuda()
    return dev(lhs), dev(codes), dev(scale), dev(gs), int(gs.sum())


def _sentinel(M, N):
    return torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


@pytest.mark.parametrize("shapes", [((11, 4096, 7168, 2048, 8), (12, 300, 1024, 512, 5))])
def test_noalloc_equals_workspace_forward(shapes):
    import fp8_moe_grouped_amd as G
    for seed, M, K, N, Gn in shapes:          # two calls in a row, the second smaller
        print(f"noalloc forward: seed {seed}, M {M}, K {K}, N {N}, G {Gn}", flush=True)
        lhs, codes, scale, gs, mv = _inputs(seed, M, K, N, Gn)
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        got = G.gmm_fp8_fwd_noalloc(lhs, codes, scale, gs, out=_sentinel(M, N), dev_status=st)
        ref = G.gmm_fp8_fwd(lhs, codes, scale, gs, out=_sentinel(M, N))
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "differs from gmm_fp8_fwd"
        assert torch.all(got[mv:].view(torch.int16) == SENTINEL), "rows past the valid prefix were written"


def test_noalloc_rejects_too_large():
    import fp8_moe_grouped_amd as G
    lhs = torch.zeros((4682, 7168), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((1, 7168, 128), dtype=torch.uint8, device="cuda")
    scale = torch.ones((1, 128), dtype=torch.float32, device="cuda")
    gs = torch.tensor([4682], dtype=torch.int32, device="cuda")
    with pytest.raises(G.Fp8GmmError) as e:
        G.gmm_fp8_fwd_noalloc(lhs, codes, scale, gs)
    assert e.value.status == G.ERR_SCRATCH
