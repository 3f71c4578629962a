"""GPU parity of the prefill chunk path (moe_prefill_forward) against the CPU
oracle, through the C ABI, on seeded synthetic inputs."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle.moe_oracle as mo
import synthetic as syn
from gpu_support import (OUT_TOL, WEIGHT_RTOL, PoolView, assert_no_near_ties, dyadic_x,
                         exact_logits, problem_to, u16)
from test_gpu_decode import TIE_CASES, _tie_problem, tie_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_routed_expert_bf16_amd as m
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


class PrefillRunner:
    def __init__(self, moe, p):
        c = p.cfg
        self.moe, self.p = moe, p
        self.dims = moe.make_dims(c.hidden, c.inter, c.n_experts, c.top_k)
        self.bufs = moe.PrefillBuffers(self.dims)
        self.pool = moe.make_pool(p.pool)
        L = p.rec.shape[0]
        self.routers = [moe.make_router(self.dims, p.router[l], p.rec[l]) for l in range(L)]
        self.shared = [moe.make_shared(p.shared_gate[l], int(p.shared_rec[l])) for l in range(L)]
        self.out = torch.zeros(moe.MAX_PREFILL_ROWS, c.hidden, dtype=torch.float32,
                               device=p.pool.device)

    def forward(self, x, layer):
        t = x.shape[0]
        self.moe.prefill_forward(x, t, self.routers[layer], self.bufs.plan, self.pool,
                                 self.shared[layer], self.out)
        torch.cuda.synchronize()
        b = self.bufs
        k = self.p.cfg.top_k
        return {"out": self.out[:t].cpu().numpy().copy(),
                "logits": b.logits[:t].cpu().numpy().copy(),
                "topk_idx": b.topk_idx[:t].cpu().numpy().copy(),
                "topk_w": b.topk_w[:t].cpu().numpy().copy(),
                "gamma": b.gamma[:t].cpu().numpy().copy(),
                "ptr": b.expert_ptr.cpu().numpy().copy(),
                "rows": b.entry_row[: t * k].cpu().numpy().copy(),
                "ranks": b.entry_rank[: t * k].cpu().numpy().copy()}


def _oracle(p, x, layer):
    c = p.cfg
    return mo.prefill_forward(x, u16(p.router[layer]), p.rec[layer].cpu().numpy(), PoolView(p.pool),
                              u16(p.shared_gate[layer]), int(p.shared_rec[layer]), c.top_k,
                              c.hidden, c.inter)


def _compare(g, r, k, what):
    t = g["out"].shape[0]
    np.testing.assert_allclose(g["logits"], r["logits"], rtol=0, atol=1e-12, err_msg=what)
    for b in range(t):
        idx, _ = mo.topk_softmax(g["logits"][b], k)
        np.testing.assert_array_equal(g["topk_idx"][b], idx, err_msg=what)
    assert_no_near_ties(r["logits"], k, what)
    np.testing.assert_array_equal(g["topk_idx"], r["topk_idx"], err_msg=what)
    np.testing.assert_allclose(g["topk_w"], r["topk_w"], rtol=WEIGHT_RTOL, atol=0, err_msg=what)
    np.testing.assert_allclose(g["gamma"], r["gamma"], rtol=1e-6, err_msg=what)
    # rows grouped by expert: bit-exact CSR
    np.testing.assert_array_equal(g["ptr"], r["ptr"], err_msg=what)
    np.testing.assert_array_equal(g["rows"], r["rows"], err_msg=what)
    np.testing.assert_array_equal(g["ranks"], r["ranks"], err_msg=what)
    ref = r["out_f64"]
    scale = float(np.abs(ref).max())
    err = float(np.abs(g["out"].astype(np.float64) - ref).max())
    assert np.all(np.isfinite(g["out"])), what
    assert err <= OUT_TOL * scale, f"{what}: max err {err:.3e} > {OUT_TOL} * {scale:.3e}"
    return err / scale


def _rms_x(seed, t, H, skew=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(t, H, generator=g)
    if skew is not None:
        x = x + skew
    return (x / torch.sqrt((x * x).mean(dim=1, keepdim=True))).contiguous()


@pytest.mark.parametrize("t", [1, 2, 5, 16, 17, 32])
def test_tiny_prefill(moe, t):
    cfg = syn.CONFIGS["tiny"]
    _say(f"[prefill tiny] t={t}")
    p = problem_to(syn.make_problem(cfg, seed=3, device="cpu"), "cuda")
    run = PrefillRunner(moe, p)
    x = _rms_x(100 + t, t, cfg.hidden).cuda()
    rel = _compare(run.forward(x, 0), _oracle(p, x.cpu().numpy(), 0), cfg.top_k, f"tiny t={t}")
    _say(f"   rel err {rel:.2e}")
    assert moe.workspace_status(run.bufs.ws) == 0


@pytest.mark.parametrize("shape", [
    dict(hidden=256, inter=64, n_experts=4, top_k=1),
    dict(hidden=512, inter=2048, n_experts=3, top_k=3),
    dict(hidden=4096, inter=256, n_experts=16, top_k=4),
    dict(hidden=768, inter=128, n_experts=1, top_k=1),
    dict(hidden=256, inter=128, n_experts=256, top_k=15),
])
@pytest.mark.parametrize("bits", ["q4", "q3", "q2", "mixed"])
def test_prefill_shapes_and_bits(moe, shape, bits):
    cfg = dataclasses.replace(syn.CONFIGS["tiny"], name="custom", bits=bits, **shape)
    _say(f"[prefill shape] {shape} {bits}")
    p = problem_to(syn.make_problem(cfg, seed=6, device="cpu"), "cuda")
    run = PrefillRunner(moe, p)
    for t in (3, 32):
        x = _rms_x(7 + t, t, cfg.hidden).cuda()
        _compare(run.forward(x, 0), _oracle(p, x.cpu().numpy(), 0), cfg.top_k, f"{shape} {bits} t={t}")
    assert moe.workspace_status(run.bufs.ws) == 0


@pytest.mark.parametrize("bits", ["q4", "q3", "q2", "mixed"])
def test_prefill_full_shape_zipf(moe, bits):
    """H 2048, I 512, 128 experts, top-8, 32-row chunks with Zipf-skewed routing."""
    cfg = dataclasses.replace(syn.CONFIGS["prefill_t32"], bits=bits)
    _say(f"[prefill full] {bits}")
    p = syn.make_problem(cfg, seed=2, device="cuda", n_layers=2)
    run = PrefillRunner(moe, p)
    xs = syn.make_x(cfg, seed=5, steps=2, device="cuda", problem=p)
    for chunk in range(2):
        for layer in range(2):
            x = xs[chunk, layer]
            g = run.forward(x, layer)
            r = _oracle(p, x.cpu().numpy(), layer)
            rel = _compare(g, r, cfg.top_k, f"{bits} chunk {chunk} layer {layer}")
            used = int((np.diff(g["ptr"]) > 0).sum())
            _say(f"   chunk {chunk} layer {layer}: experts used {used}, rel err {rel:.2e}")
    assert moe.workspace_status(run.bufs.ws) == 0


def test_prefill_deterministic(moe):
    cfg = syn.CONFIGS["prefill_t32"]
    p = syn.make_problem(cfg, seed=8, device="cuda", n_layers=1)
    run = PrefillRunner(moe, p)
    x = syn.make_x(cfg, seed=8, steps=1, device="cuda", problem=p)[0, 0]
    a = run.forward(x, 0)
    for _ in range(3):
        b = run.forward(x, 0)
        for key in a:
            np.testing.assert_array_equal(a[key], b[key], err_msg=key)


@pytest.mark.parametrize("shape", [None, dict(hidden=256, inter=128, n_experts=256, top_k=15)])
@pytest.mark.parametrize("t", [5, 32])
@pytest.mark.parametrize("case", TIE_CASES)
def test_prefill_exact_ties(moe, shape, t, case):
    """Exact logit ties in a prefill chunk: the top-k of every row, the CSR
    grouping and the outputs match the oracle bit for bit (ids) under the
    lower-id rule."""
    cfg, p = _tie_problem(shape)
    _say(f"[prefill ties] {case} shape={shape} t={t}")
    g0 = torch.Generator().manual_seed(60 + t)
    x = torch.randn(t, cfg.hidden, generator=g0)
    x = dyadic_x(x / torch.sqrt((x * x).mean(dim=1, keepdim=True)), positive=case == "signed_zeros")
    R, expect = tie_case(case, cfg, p, x)
    router = p.router.clone()
    router[0] = R
    p = dataclasses.replace(p, router=router)
    run = PrefillRunner(moe, p)
    g = run.forward(x.cuda(), 0)
    r = _oracle(p, x.numpy(), 0)
    np.testing.assert_array_equal(g["logits"], exact_logits(x, R))
    _compare(g, r, cfg.top_k, f"prefill ties {case} {shape} t={t}")
    if expect is not None:
        assert expect[0] in g["topk_idx"][0] and expect[1] not in g["topk_idx"][0]
    if case == "all_equal":
        np.testing.assert_array_equal(g["topk_idx"], np.tile(np.arange(cfg.top_k), (t, 1)))
    assert moe.workspace_status(run.bufs.ws) == 0
