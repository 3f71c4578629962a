"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
the oracle on the same seeded inputs, then compare."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle.moe_oracle as mo
import synthetic as syn

OUT_TOL = 1e-3          # max-abs error <= OUT_TOL * max|out_oracle| per layer and step
WEIGHT_RTOL = 2e-6      # f32 routing weights against float64 softmax
GAP_AMBIGUOUS = 1e-9    # oracle top-k gaps below this are ties in all but name


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class PoolView:
    """Byte slices of a device pool, copied to the host on demand."""

    def __init__(self, pool: torch.Tensor):
        self.pool = pool

    def __getitem__(self, sl):
        return self.pool[sl].cpu().numpy()


def problem_to(p: syn.Problem, device) -> syn.Problem:
    return dataclasses.replace(
        p, pool=p.pool.to(device), rec=p.rec.to(device), router=p.router.to(device),
        shared_gate=p.shared_gate.to(device), shared_rec=p.shared_rec.to(device),
        zipf_dir=None if p.zipf_dir is None else p.zipf_dir.to(device))


class DecodeRunner:
    """One set of C-ABI structs and device buffers for a problem."""

    def __init__(self, moe, p: syn.Problem):
        c = p.cfg
        self.moe, self.p = moe, p
        self.dims = moe.make_dims(c.hidden, c.inter, c.n_experts, c.top_k)
        self.bufs = moe.DecodeBuffers(self.dims)
        self.pool = moe.make_pool(p.pool)
        self.routers = [moe.make_router(self.dims, p.router[l], p.rec[l]) for l in range(p.rec.shape[0])]
        self.shared = [moe.make_shared(p.shared_gate[l], int(p.shared_rec[l]))
                       for l in range(p.rec.shape[0])]
        self.out = torch.zeros(moe.MAX_NB, c.hidden, dtype=torch.float32, device=p.pool.device)

    def forward(self, x: torch.Tensor, layer: int) -> dict:
        nb = x.shape[0]
        self.moe.layer_forward(x, nb, self.routers[layer], self.bufs.slots, self.pool,
                               self.shared[layer], self.out)
        torch.cuda.synchronize()
        return self.snapshot(nb)

    def route(self, x: torch.Tensor, layer: int) -> dict:
        nb = x.shape[0]
        self.moe.route(x, nb, self.routers[layer], self.shared[layer], self.bufs.slots)
        torch.cuda.synchronize()
        return self.snapshot(nb)

    def snapshot(self, nb: int) -> dict:
        b = self.bufs
        return {"out": self.out[:nb].cpu().numpy().copy(),
                "tab": b.tab.cpu().numpy().view(np.uint64).copy(),
                "wmap": b.wmap.cpu().numpy().copy(),
                "ids": b.ids.cpu().numpy().view(np.uint32).copy(),
                "topk_idx": b.topk_idx[:nb].cpu().numpy().copy(),
                "topk_w": b.topk_w[:nb].cpu().numpy().copy(),
                "logits": b.logits[:nb].cpu().numpy().copy(),
                "gamma": b.gamma[:nb].cpu().numpy().copy()}


def oracle_layer(p: syn.Problem, x: np.ndarray, layer: int, pool=None) -> dict:
    c = p.cfg
    return mo.layer_forward(x, u16(p.router[layer]), p.rec[layer].cpu().numpy(),
                            PoolView(p.pool) if pool is None else pool,
                            u16(p.shared_gate[layer]), int(p.shared_rec[layer]),
                            c.top_k, c.hidden, c.inter)


def topk_gap(logits_row: np.ndarray, k: int) -> float:
    s = np.sort(logits_row)[::-1]
    return float("inf") if k >= len(s) else float(s[k - 1] - s[k])


def near_ties(logits_row: np.ndarray, k: int) -> list:
    """Gaps 0 < gap < GAP_AMBIGUOUS between consecutive logits among the
    k + 1 largest: orderings that two correct float64 sums in different
    orders could resolve differently.  Exact ties (gap 0) are not among
    them: the tie rule (lower id first) decides those on both sides."""
    s = np.sort(np.asarray(logits_row, dtype=np.float64))[::-1][: k + 1]
    gaps = s[:-1] - s[1:]
    return [float(v) for v in gaps if 0.0 < v < GAP_AMBIGUOUS]


def assert_no_near_ties(logits: np.ndarray, k: int, what: str) -> None:
    for b in range(logits.shape[0]):
        near = near_ties(logits[b], k)
        assert not near, (f"{what}: row {b} has top-k gaps {near} below {GAP_AMBIGUOUS}; "
                          "the inputs are too close to a tie to compare expert ids")


def compare_decode(g: dict, r: dict, k: int, what: str = "") -> dict:
    """Asserts the decode parity bar (every check, always); returns error
    statistics."""
    nb = g["out"].shape[0]
    assert_no_near_ties(r["logits"], k, what)
    # logits: f64 sums of exact products, only the order of summation differs
    np.testing.assert_allclose(g["logits"], r["logits"], rtol=0, atol=1e-12, err_msg=what)
    # the GPU's own top-k on its exported logits is the brute-force top-k, bit for bit
    for b in range(nb):
        idx, _ = mo.topk_softmax(g["logits"][b], k)
        np.testing.assert_array_equal(g["topk_idx"][b], idx, err_msg=what)
    np.testing.assert_array_equal(g["topk_idx"], r["topk_idx"], err_msg=what)
    np.testing.assert_array_equal(g["ids"], r["ids"], err_msg=what)
    np.testing.assert_array_equal(g["tab"], r["tab"], err_msg=what)
    np.testing.assert_array_equal(g["wmap"] == 0, r["wmap"] == 0, err_msg=what)
    np.testing.assert_allclose(g["wmap"], r["wmap"], rtol=WEIGHT_RTOL, atol=0, err_msg=what)
    np.testing.assert_allclose(g["topk_w"], r["topk_w"], rtol=WEIGHT_RTOL, atol=0, err_msg=what)
    np.testing.assert_allclose(g["gamma"], r["gamma"], rtol=1e-6, atol=0, err_msg=what)
    ref = r["out_f64"]
    scale = float(np.abs(ref).max())
    err = float(np.abs(g["out"].astype(np.float64) - ref).max())
    assert np.all(np.isfinite(g["out"])), what
    assert err <= OUT_TOL * scale, f"{what}: max err {err:.3e} > {OUT_TOL} * {scale:.3e}"
    return {"err": err, "scale": scale, "rel": err / scale if scale else 0.0,
            "union": int(g["tab"][63])}


# ------------------------------------------------------- exact-tie inputs --
# x rounded to multiples of 2^-6 (|x| <= 8) and router weights to multiples
# of 2^-11 (|w| <= 255 * 2^-11, exact in bf16): every product x * w is a
# multiple of 2^-17 of magnitude <= 1, so every partial sum over H <= 4096
# inputs is exact in float64 on both sides, whatever the order.  Router rows
# that are equal (or zero) then give bit-equal logits, and the tie rule alone
# decides the top-k.

def dyadic_x(x: torch.Tensor, positive: bool = False) -> torch.Tensor:
    x = x.float().abs() if positive else x.float()
    return (torch.round(x * 64.0).clamp(-512, 512) / 64.0).contiguous()


def dyadic_router(r: torch.Tensor) -> torch.Tensor:
    """bf16 router [E][H] rounded to multiples of 2^-11 (values stay exact in bf16)."""
    v = torch.round(r.float() * 2048.0).clamp(-255, 255) / 2048.0
    out = v.to(torch.bfloat16)
    assert torch.equal(out.float(), v)
    return out.contiguous()


def exact_logits(x: torch.Tensor, router: torch.Tensor) -> np.ndarray:
    """Router logits of dyadic inputs (exact in float64)."""
    return x.double().cpu().numpy() @ router.double().cpu().numpy().T
