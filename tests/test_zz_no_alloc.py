"""moe_layer_forward_noalloc (the decode layer on the library's static
scratch, for callers that cannot allocate) against moe_layer_forward on the
same inputs, through the C ABI: two calls in a row, the second smaller."""
import sys

import numpy as np
import pytest
import torch

import synthetic as syn
from gpu_support import DecodeRunner, compare_decode, oracle_layer, problem_to

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_routed_expert_bf16_amd as m
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _x(seed, nb, H):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(nb, H, generator=g)
    return (x / torch.sqrt((x * x).mean(dim=1, keepdim=True))).cuda().contiguous()


def _both(moe, run, x, layer=0):
    """(moe_layer_forward result, moe_layer_forward_noalloc result)."""
    nb = x.shape[0]
    ref = run.forward(x, layer)
    bufs = moe.DecodeBuffers(run.dims)
    out = torch.full_like(run.out, float("nan"))
    moe.layer_forward_noalloc(x, nb, run.routers[layer], moe.slots_without_workspace(bufs.slots),
                              run.pool, run.shared[layer], out)
    torch.cuda.synchronize()
    got = {"out": out[:nb].cpu().numpy().copy(),
           "tab": bufs.tab.cpu().numpy().view(np.uint64).copy(),
           "wmap": bufs.wmap.cpu().numpy().copy(),
           "ids": bufs.ids.cpu().numpy().view(np.uint32).copy(),
           "topk_idx": bufs.topk_idx[:nb].cpu().numpy().copy(),
           "topk_w": bufs.topk_w[:nb].cpu().numpy().copy(),
           "logits": bufs.logits[:nb].cpu().numpy().copy(),
           "gamma": bufs.gamma[:nb].cpu().numpy().copy()}
    return ref, got


def test_noalloc_matches_layer_forward(moe):
    # call 1: full shape, four rows (the MFMA kernel); call 2: the tiny
    # configuration with one row (VALU kernel, other dims) on the same scratch
    big = syn.CONFIGS["verify_nb4"]
    p1 = syn.make_problem(big, seed=31, device="cuda", n_layers=1)
    run1 = DecodeRunner(moe, p1)
    x1 = syn.make_x(big, seed=32, steps=1, device="cuda", problem=p1)[0, 0]
    tiny = syn.CONFIGS["tiny"]
    p2 = problem_to(syn.make_problem(tiny, seed=33, device="cpu"), "cuda")
    run2 = DecodeRunner(moe, p2)
    x2 = _x(34, 1, tiny.hidden)
    for what, run, p, x, cfg in (("full shape nb 4", run1, p1, x1, big),
                                 ("tiny nb 1", run2, p2, x2, tiny),
                                 ("full shape nb 4 again", run1, p1, x1, big)):
        _say(f"[noalloc] {what}")
        ref, got = _both(moe, run, x)
        for key in ref:
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{what}: {key}")
        compare_decode(got, oracle_layer(p, x.cpu().numpy(), 0), cfg.top_k, f"noalloc {what}")
        assert moe.static_scratch_status() == 0
        assert moe.workspace_status(run.bufs.ws) == 0
