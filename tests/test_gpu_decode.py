"""GPU parity of the decode path (moe_route / moe_layer_forward) against the
CPU oracle, through the C ABI, on seeded synthetic inputs."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle.moe_oracle as mo
import synthetic as syn
from gpu_support import (DecodeRunner, PoolView, compare_decode, dyadic_router, dyadic_x,
                         exact_logits, oracle_layer, problem_to, u16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_routed_expert_bf16_amd as m
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _x(cfg, seed, nb, H, device):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(nb, H, generator=g)
    if cfg.x_mode == "correlated":
        x = x[:1] + 0.3 * torch.cat([torch.zeros(1, H), x[1:]])
    x = x / torch.sqrt((x * x).mean(dim=1, keepdim=True))
    return x.to(device).contiguous()


def _small_cfg(**kw):
    base = syn.CONFIGS["tiny"]
    return dataclasses.replace(base, name="custom", **kw)


@pytest.mark.parametrize("nb", [1, 2, 3, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_layer(moe, nb, seed):
    cfg = syn.CONFIGS["tiny"]
    _say(f"[tiny] seed={seed} nb={nb}")
    p = problem_to(syn.make_problem(cfg, seed=seed, device="cpu"), "cuda")
    run = DecodeRunner(moe, p)
    x = _x(cfg, seed, nb, cfg.hidden, "cuda")
    g = run.forward(x, 0)
    r = oracle_layer(p, x.cpu().numpy(), 0)
    compare_decode(g, r, cfg.top_k, f"tiny seed {seed} nb {nb}")
    assert moe.workspace_status(run.bufs.ws) == 0


@pytest.mark.parametrize("shape", [
    dict(hidden=256, inter=64, n_experts=4, top_k=1),        # smallest width
    dict(hidden=512, inter=2048, n_experts=3, top_k=3),      # widest expert, k = E
    dict(hidden=4096, inter=256, n_experts=16, top_k=4),     # two chunks per lane
    dict(hidden=768, inter=128, n_experts=1, top_k=1),       # single expert
    dict(hidden=256, inter=128, n_experts=256, top_k=15),    # max experts and k
])
@pytest.mark.parametrize("bits", ["q4", "q3", "q2", "mixed"])
def test_shapes_and_bits(moe, shape, bits):
    cfg = _small_cfg(bits=bits, x_mode="correlated", **shape)
    _say(f"[shape] {shape} {bits}")
    p = problem_to(syn.make_problem(cfg, seed=5, device="cpu"), "cuda")
    run = DecodeRunner(moe, p)
    for nb in (1, 4):
        x = _x(cfg, 11 + nb, nb, cfg.hidden, "cuda")
        g = run.forward(x, 0)
        r = oracle_layer(p, x.cpu().numpy(), 0)
        compare_decode(g, r, cfg.top_k, f"{shape} {bits} nb {nb}")
    assert moe.workspace_status(run.bufs.ws) == 0


@pytest.mark.parametrize("name,nb", [("decode_nb1", 1), ("verify_nb4", 4), ("lowbit_q3", 4),
                                     ("lowbit_q2", 4), ("mixed_q4q2", 4)])
def test_full_shape_layers(moe, name, nb):
    """H 2048, I 512, 128 experts, top-8, two layers generated on the device."""
    cfg = syn.CONFIGS[name]
    _say(f"[full-shape] {name}")
    p = syn.make_problem(cfg, seed=1, device="cuda", n_layers=2)
    run = DecodeRunner(moe, p)
    xs = syn.make_x(cfg, seed=3, steps=2, device="cuda", problem=p)
    for step in range(2):
        for layer in range(2):
            x = xs[step, layer]
            g = run.forward(x, layer)
            r = oracle_layer(p, x.cpu().numpy(), layer)
            st = compare_decode(g, r, cfg.top_k, f"{name} step {step} layer {layer}")
            _say(f"   step {step} layer {layer}: |U|={st['union']} rel err {st['rel']:.2e}")
    assert moe.workspace_status(run.bufs.ws) == 0


@pytest.mark.parametrize("name", ["verify_nb4", "lowbit_q3", "lowbit_q2", "mixed_q4q2"])
@pytest.mark.parametrize("nb", [2, 3, 4])
def test_full_shape_independent_rows(moe, name, nb):
    """Full-shape layers (H 2048, I 512: the MFMA gate/up units and down
    tiles) with 2..4 independent rows, so that at four rows the union passes
    16 slots and the down tiles run more than one batch of slots."""
    cfg = dataclasses.replace(syn.CONFIGS[name], x_mode="iid")
    _say(f"[full-shape independent] {name} nb={nb}")
    p = syn.make_problem(cfg, seed=5, device="cuda", n_layers=1)
    run = DecodeRunner(moe, p)
    x = _x(cfg, 21 + nb, nb, cfg.hidden, "cuda")
    g = run.forward(x, 0)
    r = oracle_layer(p, x.cpu().numpy(), 0)
    st = compare_decode(g, r, cfg.top_k, f"{name} nb {nb}")
    _say(f"   |U|={st['union']} rel err {st['rel']:.2e}")
    if nb == 4:
        assert st["union"] > 16
    assert moe.workspace_status(run.bufs.ws) == 0


def test_full_shape_bad_descriptor(moe):
    """A routed descriptor past the pool in a full-shape four-row layer (MFMA
    kernel): the record is skipped in every row that routed to it, the status
    word is flagged, and the rest matches the oracle without it."""
    cfg = dataclasses.replace(syn.CONFIGS["verify_nb4"], x_mode="iid")
    p = syn.make_problem(cfg, seed=6, device="cuda", n_layers=1)
    x = _x(cfg, 33, 4, cfg.hidden, "cuda")
    r = oracle_layer(p, x.cpu().numpy(), 0)
    bad_e = int(r["topk_idx"][1, 0])
    rec = p.rec.clone()
    rec[0, bad_e] = (p.pool.numel() + 4096) & ~0xFF
    run = DecodeRunner(moe, dataclasses.replace(p, rec=rec))
    g = run.forward(x, 0)
    assert moe.workspace_status(run.bufs.ws) & 1
    Wg, Wu, Wd = mo.read_expert(PoolView(p.pool), int(p.rec[0, bad_e]), cfg.hidden, cfg.inter)
    expect = r["out_f64"].copy()
    xn = x.cpu().numpy().astype(np.float64)
    for b in range(4):
        hit = np.nonzero(r["topk_idx"][b] == bad_e)[0]
        if hit.size:
            y, _ = mo.expert_mlp(Wg, Wu, Wd, xn[b])
            expect[b] -= r["topk_w"][b, hit[0]] * y
    err = np.abs(g["out"] - expect).max()
    assert err <= 1e-3 * np.abs(expect).max()
    assert moe.workspace_status(run.bufs.ws) == 0     # read-and-clear


@pytest.mark.parametrize("shape", [
    None,                                                    # full shape (H 2048, 128 experts, k 8)
    dict(hidden=256, inter=128, n_experts=256, top_k=15),    # max experts and k
    dict(hidden=4096, inter=256, n_experts=16, top_k=4),     # two chunks per lane
    dict(hidden=768, inter=128, n_experts=1, top_k=1),       # single expert
])
@pytest.mark.parametrize("nb", [1, 2, 3, 4])
def test_route_only_rows_and_shapes(moe, shape, nb):
    """moe_route (the route-only kernel) writes the same routing tables as
    moe_layer_forward, bit for bit, and they match the oracle's."""
    if shape is None:
        cfg = dataclasses.replace(syn.CONFIGS["verify_nb4"], x_mode="iid")
        p = syn.make_problem(cfg, seed=7, device="cuda", n_layers=1)
    else:
        cfg = _small_cfg(**shape)
        p = problem_to(syn.make_problem(cfg, seed=7, device="cpu"), "cuda")
    run = DecodeRunner(moe, p)
    x = _x(cfg, 40 + nb, nb, cfg.hidden, "cuda")
    a = run.route(x, 0)
    b = run.forward(x, 0)
    for key in ("tab", "wmap", "ids", "topk_idx", "topk_w", "logits", "gamma"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    r = oracle_layer(p, x.cpu().numpy(), 0)
    compare_decode(b, r, cfg.top_k, f"route {shape} nb {nb}")
    assert moe.workspace_status(run.bufs.ws) == 0


def test_route_only_matches_forward(moe):
    cfg = syn.CONFIGS["verify_nb4"]
    p = syn.make_problem(cfg, seed=2, device="cuda", n_layers=1)
    run = DecodeRunner(moe, p)
    x = syn.make_x(cfg, seed=9, steps=1, device="cuda", problem=p)[0, 0]
    a = run.route(x, 0)
    b = run.forward(x, 0)
    for key in ("tab", "wmap", "ids", "topk_idx", "topk_w", "logits", "gamma"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_deterministic_repeat(moe):
    cfg = syn.CONFIGS["verify_nb4"]
    p = syn.make_problem(cfg, seed=4, device="cuda", n_layers=1)
    run = DecodeRunner(moe, p)
    x = syn.make_x(cfg, seed=4, steps=1, device="cuda", problem=p)[0, 0]
    first = run.forward(x, 0)
    for _ in range(5):
        again = run.forward(x, 0)
        for key in first:
            np.testing.assert_array_equal(first[key], again[key], err_msg=key)


def test_bad_descriptor_is_skipped_and_flagged(moe):
    """A routed record descriptor that points past the pool: the kernels skip
    that expert (in-bounds check), flag the workspace status word, and the
    other experts still match the oracle with that expert's weight dropped."""
    cfg = syn.CONFIGS["tiny"]
    p = problem_to(syn.make_problem(cfg, seed=0, device="cpu"), "cuda")
    x = _x(cfg, 0, 1, cfg.hidden, "cuda")
    r = oracle_layer(p, x.cpu().numpy(), 0)
    bad_e = int(r["topk_idx"][0, 0])
    rec = p.rec.clone()
    rec[0, bad_e] = (p.pool.numel() + 4096) & ~0xFF
    p2 = dataclasses.replace(p, rec=rec)
    run = DecodeRunner(moe, p2)
    g = run.forward(x, 0)
    assert moe.workspace_status(run.bufs.ws) & 1
    # expected: the oracle's output minus the skipped expert's weighted output
    Wg, Wu, Wd = mo.read_expert(PoolView(p.pool), int(p.rec[0, bad_e]), cfg.hidden, cfg.inter)
    y, _ = mo.expert_mlp(Wg, Wu, Wd, x.cpu().numpy()[0].astype(np.float64))
    expect = r["out_f64"][0] - r["topk_w"][0, 0] * y
    err = np.abs(g["out"][0] - expect).max()
    assert err <= 1e-3 * np.abs(expect).max()
    assert moe.workspace_status(run.bufs.ws) == 0     # read-and-clear


# ---------------------------------------------------------------- exact ties
# Router inputs rounded so that every logit is exact on both sides (see
# gpu_support.dyadic_x): equal router rows give bit-equal logits, so the
# top-k, the union and the slot table are decided by the tie rule (logit
# descending, lower expert id first) and must match the oracle bit for bit.

def _tie_problem(shape):
    if shape is None:
        cfg = dataclasses.replace(syn.CONFIGS["verify_nb4"], x_mode="iid")
        p = syn.make_problem(cfg, seed=12, device="cuda", n_layers=1)
    else:
        cfg = _small_cfg(**shape)
        p = problem_to(syn.make_problem(cfg, seed=12, device="cpu"), "cuda")
    router = p.router.clone()
    router[0] = dyadic_router(router[0])
    return cfg, dataclasses.replace(p, router=router)


def tie_case(case, cfg, p, x):
    """Router of layer 0 rewritten for one tie case; returns (router, expect),
    expect = (lower id that must be selected, higher id that must not) or None."""
    E, k = cfg.n_experts, cfg.top_k
    R = p.router[0].clone()
    expect = None
    if case in ("straddle_lower", "straddle_higher"):
        # a copy of the k-th expert's row (row 0 of x) at another id: the two
        # tie across the k boundary and the lower id takes the place
        lg = exact_logits(x[:1], R)[0]
        order = np.lexsort((np.arange(E), -lg))
        ek = int(order[k - 1])
        if case == "straddle_lower":
            cands = [int(e) for e in order[k:] if e < ek]
        else:
            cands = [int(e) for e in order[k:] if e > ek]
        if not cands:
            pytest.skip(f"no expert id on that side of {ek}")
        other = cands[0]
        R[other] = R[ek]
        expect = (min(ek, other), max(ek, other))
    elif case == "signed_zeros":
        # x > 0 (dyadic_x(positive=True)); zero rows, alternately +0 and -0
        # bit patterns, give logits of +-0 that tie with each other; every
        # other row is a distinct negative constant, below them
        zero_ids = list(range(1, E, max(1, E // (k + 3))))[: k + 2]
        for e in range(E):
            R[e] = -float((1 + e % 200)) / 2048.0
        for i, e in enumerate(zero_ids):
            R[e] = -0.0 if i % 2 else 0.0
    elif case == "all_equal":
        R[:] = R[0]
    else:
        raise ValueError(case)
    return R.contiguous(), expect


TIE_CASES = ["straddle_lower", "straddle_higher", "signed_zeros", "all_equal"]


@pytest.mark.parametrize("shape", [None, dict(hidden=256, inter=128, n_experts=256, top_k=15)])
@pytest.mark.parametrize("nb", [1, 4])
@pytest.mark.parametrize("case", TIE_CASES)
def test_exact_ties(moe, shape, nb, case):
    cfg, p = _tie_problem(shape)
    _say(f"[ties] {case} shape={shape} nb={nb}")
    x = dyadic_x(_x(cfg, 50 + nb, nb, cfg.hidden, "cpu"), positive=case == "signed_zeros").cuda()
    R, expect = tie_case(case, cfg, p, x.cpu())
    router = p.router.clone()
    router[0] = R
    p = dataclasses.replace(p, router=router)
    lg = exact_logits(x.cpu(), R)
    assert any(len(set(lg[b])) < cfg.n_experts for b in range(nb))   # ties are there
    run = DecodeRunner(moe, p)
    g = run.forward(x, 0)
    r = oracle_layer(p, x.cpu().numpy(), 0)
    np.testing.assert_array_equal(g["logits"], lg)   # exact on the device too
    compare_decode(g, r, cfg.top_k, f"ties {case} {shape} nb {nb}")
    a = run.route(x, 0)
    for key in ("tab", "wmap", "ids", "topk_idx", "topk_w"):
        np.testing.assert_array_equal(a[key], g[key], err_msg=key)
    if expect is not None:
        assert expect[0] in g["topk_idx"][0] and expect[1] not in g["topk_idx"][0]
    if case == "all_equal":
        for b in range(nb):
            np.testing.assert_array_equal(g["topk_idx"][b], np.arange(cfg.top_k))
        np.testing.assert_array_equal(g["ids"][: cfg.top_k], np.arange(cfg.top_k))
        np.testing.assert_allclose(g["topk_w"], 1.0 / cfg.top_k, rtol=1e-6)
    assert moe.workspace_status(run.bufs.ws) == 0


@pytest.mark.parametrize("inter", [64, 128])
def test_epoch_advances_once_per_call(moe, inter):
    """With I < 256 some slices of the decode grid have no columns; every
    block still reads the call's epoch, so the workspace epoch word goes up
    by exactly one per call whichever block leaves last."""
    cfg = _small_cfg(hidden=256, inter=inter, n_experts=8, top_k=2)
    p = problem_to(syn.make_problem(cfg, seed=9, device="cpu"), "cuda")
    run = DecodeRunner(moe, p)
    x = _x(cfg, 9, 2, cfg.hidden, "cuda")
    ep_word = run.bufs.ws.view(torch.int32)
    first = run.forward(x, 0)
    prev = int(ep_word[608].item())
    for i in range(60):
        g = run.forward(x, 0)
        now = int(ep_word[608].item())
        assert now == prev + 1, f"call {i}: epoch {prev} -> {now}"
        prev = now
        np.testing.assert_array_equal(g["out"], first["out"])
    compare_decode(first, oracle_layer(p, x.cpu().numpy(), 0), cfg.top_k, f"epoch I={inter}")
    assert moe.workspace_status(run.bufs.ws) == 0
