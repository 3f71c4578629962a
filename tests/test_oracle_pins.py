"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a hand-derived fixture
(tests/golden/), a closed form, a library routine (numpy, scipy, torch) or
brute force, chosen so that a plausible slip (a dropped bias, a swapped
gate/up, a wrong nibble order, a transposed matrix, a lost tie rule) fails at
least one of them; ``test_planted_mistakes_are_caught`` plants such slips in
the oracle and checks that they are caught.
"""
import inspect
import math
import os
import textwrap

import numpy as np
import pytest
import scipy.special
import torch

import oracle.moe_oracle as mo
import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers --

def _bf16(v):
    return syn.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _random_record(rng, H, I, bits, noise=1e-3):
    """Raw codes and bf16 (s, b) of one record plus the packed pool bytes."""
    hi = 1 << bits
    gu_q = rng.integers(0, hi, size=(2 * I, H))
    d_q = rng.integers(0, hi, size=(H, I))
    gu_s = _bf16(rng.uniform(0.002, 0.02, size=(2 * I, H // 64)))
    d_s = _bf16(rng.uniform(0.002, 0.02, size=(H, I // 64)))
    off = 2 ** (bits - 1)
    gu_b = _bf16(-off * mo.bf16_to_f64(gu_s) + noise * rng.standard_normal((2 * I, H // 64)))
    d_b = _bf16(-off * mo.bf16_to_f64(d_s) + noise * rng.standard_normal((H, I // 64)))
    return dict(gu_q=gu_q, d_q=d_q, gu_s=gu_s, gu_b=gu_b, d_s=d_s, d_b=d_b)


def _write(pool, off, H, I, bits, r):
    return syn.write_record(pool, off, H, I, bits, r["gu_q"], r["gu_s"], r["gu_b"],
                            r["d_q"], r["d_s"], r["d_b"])


def _torch_dequant(q, s16, b16):
    """Dequantise from raw codes with torch (independent of the oracle)."""
    s = torch.tensor(s16.astype(np.int32) << 16, dtype=torch.int32).view(torch.float32).double()
    b = torch.tensor(b16.astype(np.int32) << 16, dtype=torch.int32).view(torch.float32).double()
    s = s.repeat_interleave(64, dim=1)
    b = b.repeat_interleave(64, dim=1)
    return torch.tensor(q, dtype=torch.float64) * s + b


def _torch_mlp(r, x64):
    """Dense float64 MLP (torch matmul + torch silu) from raw codes."""
    gu = _torch_dequant(r["gu_q"], r["gu_s"], r["gu_b"])
    Wg, Wu = gu[0::2], gu[1::2]
    Wd = _torch_dequant(r["d_q"], r["d_s"], r["d_b"])
    xt = torch.tensor(x64)
    a = torch.nn.functional.silu(xt @ Wg.T) * (xt @ Wu.T)
    return (a @ Wd.T).numpy()


def _rms_rows(rng, nb, H):
    x = rng.standard_normal((nb, H))
    return (x / np.sqrt((x * x).mean(axis=1, keepdims=True))).astype(np.float32)


# ------------------------------------------------------------- unpacking --

def test_unpack_matches_golden_words():
    n_cases = 0
    with open(os.path.join(GOLDEN, "packing.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            bits_s, words_s, codes_s = line.split("|")
            bits = int(bits_s)
            words = np.array([int(w, 16) for w in words_s.split()], dtype="<u4")
            codes = np.array([int(c) for c in codes_s.split()])
            got = mo.unpack_codes(words.view(np.uint8)[None, :], 64, bits)[0]
            np.testing.assert_array_equal(got, codes)
            # and the generator's packer writes exactly these words
            np.testing.assert_array_equal(syn.pack_codes(codes[None, :], bits)[0],
                                          words.view(np.uint8))
            n_cases += 1
    assert n_cases == 9


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_pack_unpack_exhaustive(bits):
    # every code value at every position of a 64-code group
    rng = np.random.default_rng(bits)
    n = 256
    rows = []
    for v in range(1 << bits):
        rows.append(np.full(n, v))
    rows.append(np.arange(n) % (1 << bits))
    rows.append(rng.integers(0, 1 << bits, n))
    codes = np.array(rows)
    packed = syn.pack_codes(codes, bits)
    assert packed.shape == (codes.shape[0], n * bits // 8)
    np.testing.assert_array_equal(mo.unpack_codes(packed, n, bits), codes)


def test_bf16_decode_matches_torch():
    pats = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3C23, 0x7F7F, 0x0001, 0x4049],
                    dtype=np.uint16)
    ref = torch.tensor(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(mo.bf16_to_f64(pats), ref)
    assert mo.bf16_to_f64(np.uint16(0x3F80)) == 1.0


def test_dequant_closed_form_constant_codes():
    # all codes c with constant s, b give W == c*s + b exactly
    for bits in (4, 3, 2):
        for c in (0, 1, (1 << bits) - 1):
            q = np.full((3, 128), c)
            s16 = _bf16(np.full((3, 2), 0.0123))
            b16 = _bf16(np.full((3, 2), -0.0456))
            W = mo.dequant(q, syn.sb_words(s16, b16))
            s, b = mo.bf16_to_f64(s16)[0, 0], mo.bf16_to_f64(b16)[0, 0]
            assert np.all(W == c * s + b)


def test_dequant_group_boundaries():
    # scale/bias change exactly at multiples of 64 along the input dimension
    q = np.ones((1, 256), dtype=np.int64)
    s16 = _bf16([[1.0, 2.0, 4.0, 8.0]])
    b16 = _bf16([[0.0, 0.5, 0.25, 0.125]])
    W = mo.dequant(q, syn.sb_words(s16, b16))[0]
    np.testing.assert_array_equal(W[:64], 1.0)
    np.testing.assert_array_equal(W[64:128], 2.5)
    np.testing.assert_array_equal(W[128:192], 4.25)
    np.testing.assert_array_equal(W[192:], 8.125)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_read_expert_matches_raw_codes(bits):
    rng = np.random.default_rng(10 + bits)
    H, I = 256, 128
    r = _random_record(rng, H, I, bits)
    pool = np.zeros(syn.record_bytes(H, I, bits) + 512, dtype=np.uint8)
    desc = _write(pool, 256, H, I, bits, r)
    Wg, Wu, Wd = mo.read_expert(pool, desc, H, I)
    gu = _torch_dequant(r["gu_q"], r["gu_s"], r["gu_b"]).numpy()
    np.testing.assert_array_equal(Wg, gu[0::2])
    np.testing.assert_array_equal(Wu, gu[1::2])
    np.testing.assert_array_equal(Wd, _torch_dequant(r["d_q"], r["d_s"], r["d_b"]).numpy())


def test_record_layout_sizes():
    # sizes of the 2048/512 records: 4-bit 1,769,472 B, 3-bit 1,376,256, 2-bit 983,040
    assert mo.record_layout(2048, 512, 4)["total"] == 1769472
    assert mo.record_layout(2048, 512, 3)["total"] == 1376256
    assert mo.record_layout(2048, 512, 2)["total"] == 983040
    assert mo.record_layout(256, 128, 4)["total"] == 55296
    for bits in (4, 3, 2):
        assert mo.record_layout(2048, 512, bits) == {
            k: v for k, v in syn.record_sections(2048, 512, bits).items()}


# --------------------------------------------------------------- routing --

def test_router_logits_exact():
    # products bf16 x f32 are exact in f64: compare with a correctly rounded sum
    rng = np.random.default_rng(3)
    x = _rms_rows(rng, 2, 256)
    R = _bf16(0.02 * rng.standard_normal((8, 256)))
    L = mo.router_logits(x, R)
    Rf = mo.bf16_to_f64(R)
    for b in range(2):
        for e in range(8):
            exact = math.fsum(float(Rf[e, i]) * float(x[b, i]) for i in range(256))
            assert abs(L[b, e] - exact) <= 1e-15 * sum(abs(Rf[e] * x[b]))


def test_topk_matches_lexsort_and_ties():
    rng = np.random.default_rng(4)
    for trial in range(200):
        E, k = int(rng.integers(2, 40)), 0
        k = int(rng.integers(1, E + 1))
        # coarse values so that ties are frequent
        logits = rng.integers(-3, 4, size=E).astype(np.float64)
        idx, w = mo.topk_softmax(logits, k)
        ref = np.lexsort((np.arange(E), -logits))[:k]
        np.testing.assert_array_equal(idx, ref)
    idx, _ = mo.topk_softmax(np.array([1.0, 5.0, 5.0, 0.0, 5.0]), 2)
    np.testing.assert_array_equal(idx, [1, 2])


def test_topk_weights_softmax():
    rng = np.random.default_rng(5)
    for _ in range(50):
        logits = rng.standard_normal(32) * 3
        idx, w = mo.topk_softmax(logits, 8)
        assert abs(w.sum() - 1.0) < 1e-12
        np.testing.assert_allclose(w, scipy.special.softmax(logits[idx]), rtol=1e-13)
        assert np.all(np.diff(w) <= 0)
    # k = 1 gives weight 1; two experts: w0 = 1/(1+exp(l1-l0))
    assert mo.topk_softmax(np.array([0.3, -2.0, 1.5]), 1)[1][0] == 1.0
    _, w = mo.topk_softmax(np.array([0.7, -0.4]), 2)
    assert abs(w[0] - 1.0 / (1.0 + math.exp(-0.4 - 0.7))) < 1e-15


def test_union_slots_first_seen():
    rng = np.random.default_rng(6)
    for _ in range(100):
        nb, k, E = int(rng.integers(1, 5)), int(rng.integers(1, 9)), 16
        idx = np.array([rng.choice(E, size=k, replace=False) for _ in range(nb)])
        w = rng.uniform(0.01, 1, size=(nb, k))
        rec = (np.arange(E, dtype=np.uint64) * 256 + 3)
        s = mo.union_slots(idx, w, rec)
        ref = list(dict.fromkeys(idx.reshape(-1).tolist()))
        u = len(ref)
        assert s["n_union"] == u
        np.testing.assert_array_equal(s["ids"][:u], ref)
        assert np.all(s["ids"][u:] == 0) and np.all(s["tab"][u:62] == 0)
        assert s["tab"][62] == u and s["tab"][63] == u
        np.testing.assert_array_equal(s["tab"][:u], rec[np.array(ref)])
        for b in range(nb):
            row = {int(e): ww for e, ww in zip(idx[b], w[b])}
            for j, e in enumerate(ref):
                assert s["wmap"][b, j] == row.get(e, 0.0)
        assert np.all(s["wmap"][nb:] == 0) and np.all(s["wmap"][:, u:] == 0)


# ---------------------------------------------------------------- layers --

def _golden_values(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=")
                vals[k.strip()] = float(v)
    return vals


def test_golden_tiny_layer():
    vals = _golden_values("tiny_layer.txt")
    H = I = 64
    pool = np.zeros(4 * syn.record_bytes(H, I, 4), dtype=np.uint8)
    s = _bf16(np.full((2 * I, 1), 2.0 ** -6))
    sd = _bf16(np.full((H, 1), 2.0 ** -6))
    z = _bf16(np.zeros((2 * I, 1)))
    zd = _bf16(np.zeros((H, 1)))
    gu0 = np.zeros((2 * I, H), dtype=np.int64)
    gu0[0::2] = 1
    gu0[1::2] = 2
    rb = syn.record_bytes(H, I, 4)
    d0 = syn.write_record(pool, 0, H, I, 4, gu0, s, z, np.ones((H, I), np.int64), sd, zd)
    d1 = syn.write_record(pool, rb, H, I, 4, np.full((2 * I, H), 15), s, z,
                          np.full((H, I), 15), sd, zd)
    ds = syn.write_record(pool, 2 * rb, H, I, 4, np.zeros((2 * I, H), np.int64), s, s,
                          np.zeros((H, I), np.int64), sd, sd)
    router = _bf16(np.stack([np.full(H, 2.0 ** -6), np.full(H, -2.0 ** -6)]))
    x = np.ones((1, H), dtype=np.float32)
    r = mo.layer_forward(x, router, [d0, d1], pool, _bf16(np.zeros(H)), ds, 1, H, I)
    assert r["logits"][0, 0] == vals["logit0"] and r["logits"][0, 1] == vals["logit1"]
    assert r["topk_idx"][0, 0] == vals["expert"] and r["topk_w"][0, 0] == vals["weight"]
    assert r["gamma"][0] == vals["gamma"]
    np.testing.assert_allclose(r["out_f64"][0], vals["out"], rtol=1e-15)
    assert abs(vals["out"] - 2.5 / (1 + math.exp(-1))) < 1e-15


def _sig(v):
    return 1.0 / (1.0 + math.exp(-v))


def test_golden_tiny_layer_k2():
    """Two routed experts per row and a non-zero shared gate vector
    (tests/golden/tiny_layer_k2.txt): pins the routing-weighted combine at
    k = 2 and the sign of the shared gate, through layer_forward and, for two
    identical rows, prefill_forward."""
    vals = _golden_values("tiny_layer_k2.txt")
    # the stored numbers are the closed forms stated in the file
    assert vals["out"] == pytest.approx(3 * _sig(1) ** 2 + 6 * _sig(-1) * _sig(2), rel=1e-15)
    assert vals["weight0"] == pytest.approx(_sig(1), rel=1e-15)
    assert vals["weight1"] == pytest.approx(_sig(-1), rel=1e-15)
    assert vals["gamma"] == pytest.approx(_sig(1), rel=1e-15)
    H = I = 64
    rb = syn.record_bytes(H, I, 4)
    pool = np.zeros(4 * rb, dtype=np.uint8)
    s = _bf16(np.full((2 * I, 1), 2.0 ** -6))
    sd = _bf16(np.full((H, 1), 2.0 ** -6))
    z = _bf16(np.zeros((2 * I, 1)))
    zd = _bf16(np.zeros((H, 1)))

    def gu(gc, uc):
        q = np.zeros((2 * I, H), dtype=np.int64)
        q[0::2] = gc
        q[1::2] = uc
        return q

    d0 = syn.write_record(pool, 0, H, I, 4, gu(1, 2), s, z, np.full((H, I), 1), sd, zd)
    d1 = syn.write_record(pool, rb, H, I, 4, gu(2, 1), s, z, np.full((H, I), 3), sd, zd)
    d2 = syn.write_record(pool, 2 * rb, H, I, 4, np.full((2 * I, H), 15), s, z,
                          np.full((H, I), 15), sd, zd)
    ds = syn.write_record(pool, 3 * rb, H, I, 4, gu(1, 1), s, z, np.full((H, I), 1), sd, zd)
    router = _bf16(np.stack([np.full(H, 2.0 ** -6), np.zeros(H), np.full(H, -2.0 ** -6)]))
    gvec = _bf16(np.full(H, 2.0 ** -6))
    r = mo.layer_forward(np.ones((1, H), dtype=np.float32), router, [d0, d1, d2], pool, gvec,
                         ds, 2, H, I)
    np.testing.assert_array_equal(r["logits"][0], [vals["logit0"], vals["logit1"], vals["logit2"]])
    np.testing.assert_array_equal(r["topk_idx"][0], [vals["expert0"], vals["expert1"]])
    np.testing.assert_allclose(r["topk_w"][0], [vals["weight0"], vals["weight1"]], rtol=1e-15)
    np.testing.assert_allclose(r["gamma"], [vals["gamma"]], rtol=1e-15)
    np.testing.assert_allclose(r["out_f64"][0], vals["out"], rtol=1e-14)
    p = mo.prefill_forward(np.ones((2, H), dtype=np.float32), router, [d0, d1, d2], pool, gvec,
                           ds, 2, H, I)
    np.testing.assert_allclose(p["topk_w"], [[vals["weight0"], vals["weight1"]]] * 2, rtol=1e-15)
    np.testing.assert_allclose(p["out_f64"], vals["out"], rtol=1e-14)


def _bf16_torch(v16):
    """bf16 bit patterns -> float64 through torch (independent of the oracle)."""
    t = torch.tensor(np.asarray(v16).astype(np.int32) << 16, dtype=torch.int32)
    return t.view(torch.float32).double().numpy()


def test_zero_scales_layer_closed_form():
    """Every scale 0 in every record, so each weight row is its group biases
    and an expert is a closed form in group sums: g = B_g xs, u = B_u xs,
    y = B_d (group sums of silu(g) u).  The layer output over 4 rows with
    k = 3 of 6 experts is then sum_r w_r y_{e_r} + gamma y_shared, with the
    logits from a numpy product, top-k from lexsort, weights from
    scipy.special.softmax and gamma from scipy.special.expit; it pins the
    k >= 2 combine of layer_forward and prefill_forward."""
    rng = np.random.default_rng(8)
    H, I, E, k, nb = 256, 128, 6, 3, 4
    rb = syn.record_bytes(H, I, 4)
    pool = np.zeros((E + 1) * rb, dtype=np.uint8)
    recs, descs = [], []
    for e in range(E + 1):
        r = _random_record(rng, H, I, 4, noise=0.05)
        r["gu_s"] = _bf16(np.zeros(r["gu_s"].shape))
        r["d_s"] = _bf16(np.zeros(r["d_s"].shape))
        descs.append(_write(pool, e * rb, H, I, 4, r))
        recs.append(r)
    router = _bf16(0.3 * rng.standard_normal((E, H)))
    gvec = _bf16(0.05 * rng.standard_normal(H))
    x = _rms_rows(rng, nb, H)
    xd = x.astype(np.float64)
    logits = xd @ _bf16_torch(router).T
    gam = scipy.special.expit(xd @ _bf16_torch(gvec))

    def expert_out(r, xb):
        xs = xb.reshape(-1, 64).sum(axis=1)
        gb = _bf16_torch(r["gu_b"])
        g, u = gb[0::2] @ xs, gb[1::2] @ xs
        a = g * scipy.special.expit(g) * u
        return _bf16_torch(r["d_b"]) @ a.reshape(-1, 64).sum(axis=1)

    expect = np.zeros((nb, H))
    for b in range(nb):
        top = np.lexsort((np.arange(E), -logits[b]))[:k]
        w = scipy.special.softmax(logits[b, top])
        assert w.min() < 0.9 * w.max()      # weights that matter
        for wr, e in zip(w, top):
            expect[b] += wr * expert_out(recs[e], xd[b])
        expect[b] += gam[b] * expert_out(recs[E], xd[b])
    atol = 1e-12 * np.abs(expect).max()
    res = mo.layer_forward(x, router, descs[:E], pool, gvec, descs[E], k, H, I)
    np.testing.assert_allclose(res["out_f64"], expect, rtol=1e-11, atol=atol)
    pre = mo.prefill_forward(x, router, descs[:E], pool, gvec, descs[E], k, H, I)
    np.testing.assert_allclose(pre["out_f64"], expect, rtol=1e-11, atol=atol)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_single_expert_equals_dense_mlp(bits):
    # E = k = 1 and a zero shared gate vector (gamma = 1/2):
    # out = expert(x) + shared(x)/2 against a torch float64 dense MLP
    rng = np.random.default_rng(20 + bits)
    H, I = 256, 128
    r0 = _random_record(rng, H, I, bits)
    rs = _random_record(rng, H, I, 4)
    rb = syn.record_bytes(H, I, 4)
    pool = np.zeros(2 * rb, dtype=np.uint8)
    d0 = _write(pool, 0, H, I, bits, r0)
    ds = _write(pool, rb, H, I, 4, rs)
    x = _rms_rows(rng, 3, H)
    router = _bf16(0.02 * rng.standard_normal((1, H)))
    res = mo.layer_forward(x, router, [d0], pool, _bf16(np.zeros(H)), ds, 1, H, I)
    assert np.all(res["gamma"] == 0.5) and np.all(res["topk_w"] == 1.0)
    ref = _torch_mlp(r0, x.astype(np.float64)) + 0.5 * _torch_mlp(rs, x.astype(np.float64))
    np.testing.assert_allclose(res["out_f64"], ref, rtol=1e-12, atol=1e-12)


def _tiny_problem(seed=0, nb=4):
    cfg = syn.CONFIGS["tiny"]
    p = syn.make_problem(cfg, seed=seed, device="cpu")
    pool = p.pool.numpy()
    rec = p.rec[0].numpy()
    router = p.router[0].view(torch.int16).numpy().view(np.uint16)
    gvec = p.shared_gate[0].view(torch.int16).numpy().view(np.uint16)
    rng = np.random.default_rng(seed)
    x = _rms_rows(rng, nb, cfg.hidden)
    return cfg, pool, rec, router, gvec, int(p.shared_rec[0]), x


def test_batch_equals_independent_rows():
    cfg, pool, rec, router, gvec, sd, x = _tiny_problem()
    batch = mo.layer_forward(x, router, rec, pool, gvec, sd, cfg.top_k, cfg.hidden, cfg.inter)
    for b in range(x.shape[0]):
        one = mo.layer_forward(x[b:b + 1], router, rec, pool, gvec, sd, cfg.top_k,
                               cfg.hidden, cfg.inter)
        np.testing.assert_array_equal(one["topk_idx"][0], batch["topk_idx"][b])
        np.testing.assert_allclose(one["out_f64"][0], batch["out_f64"][b], rtol=1e-13, atol=1e-13)


def test_expert_permutation_equivariance():
    cfg, pool, rec, router, gvec, sd, x = _tiny_problem(seed=1)
    base = mo.layer_forward(x, router, rec, pool, gvec, sd, cfg.top_k, cfg.hidden, cfg.inter)
    perm = np.random.default_rng(2).permutation(cfg.n_experts)   # new id p <- old id perm[p]
    res = mo.layer_forward(x, router[perm], rec[perm], pool, gvec, sd, cfg.top_k,
                           cfg.hidden, cfg.inter)
    np.testing.assert_array_equal(perm[res["topk_idx"]], base["topk_idx"])
    np.testing.assert_allclose(res["out_f64"], base["out_f64"], rtol=1e-13, atol=1e-13)


def test_zero_scales_closed_form():
    # every scale 0: each row of W is its bias per group, so W x = sum_g b_g * sum(x in g)
    rng = np.random.default_rng(7)
    H, I = 256, 128
    r = _random_record(rng, H, I, 4)
    r["gu_s"] = _bf16(np.zeros_like(r["gu_s"], dtype=np.float64))
    r["d_s"] = _bf16(np.zeros_like(r["d_s"], dtype=np.float64))
    pool = np.zeros(syn.record_bytes(H, I, 4), dtype=np.uint8)
    desc = _write(pool, 0, H, I, 4, r)
    Wg, Wu, Wd = mo.read_expert(pool, desc, H, I)
    x = _rms_rows(rng, 1, H)[0].astype(np.float64)
    xs = np.add.reduceat(x, np.arange(0, H, 64))
    gb = mo.bf16_to_f64(r["gu_b"])
    g = gb[0::2] @ xs
    u = gb[1::2] @ xs
    y, a = mo.expert_mlp(Wg, Wu, Wd, x)
    np.testing.assert_allclose(a, scipy.special.expit(g) * g * u, rtol=1e-12)
    np.testing.assert_allclose(y, mo.bf16_to_f64(r["d_b"]) @ np.add.reduceat(a, np.arange(0, I, 64)),
                               rtol=1e-12, atol=1e-14)


def test_silu_sigmoid_values():
    v = np.array([-30.0, -1.0, 0.0, 0.5, 3.0, 40.0])
    np.testing.assert_allclose(mo.sigmoid(v), scipy.special.expit(v), rtol=1e-15)
    np.testing.assert_allclose(mo.silu(v), v * scipy.special.expit(v), rtol=1e-15)
    assert mo.silu(np.array(0.0)) == 0.0 and mo.sigmoid(0.0) == 0.5


def test_prefill_csr_and_rows():
    cfg, pool, rec, router, gvec, sd, _ = _tiny_problem(seed=3)
    rng = np.random.default_rng(11)
    x = _rms_rows(rng, 9, cfg.hidden)
    res = mo.prefill_forward(x, router, rec, pool, gvec, sd, cfg.top_k, cfg.hidden, cfg.inter)
    flat = res["topk_idx"].reshape(-1)
    order = np.argsort(flat, kind="stable")        # expert ascending, then row-major
    np.testing.assert_array_equal(res["rows"], order // cfg.top_k)
    np.testing.assert_array_equal(res["ranks"], order % cfg.top_k)
    np.testing.assert_array_equal(np.diff(res["ptr"]), np.bincount(flat, minlength=cfg.n_experts))
    for r_ in range(x.shape[0]):
        one = mo.layer_forward(x[r_:r_ + 1], router, rec, pool, gvec, sd, cfg.top_k,
                               cfg.hidden, cfg.inter)
        np.testing.assert_allclose(res["out_f64"][r_], one["out_f64"][0], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------ planted mistakes --

def _planted(monkeypatch, name, fn):
    monkeypatch.setattr(mo, name, fn)


def _edited(fn, old, new):
    """fn recompiled from its own source with one expression replaced (a
    mistake planted inside the function body)."""
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) == 1, f"{old!r} not found once in {fn.__name__}"
    ns = {}
    exec(compile(src.replace(old, new), inspect.getsourcefile(fn), "exec"), fn.__globals__, ns)
    return ns[fn.__name__]


LAYER_COMBINE = 'acc[b] += slots["wmap"][b, j] * y'
PREFILL_COMBINE = 'acc[r_] += csr["wts"][p] * y'


@pytest.mark.parametrize("mistake", ["nibble_order", "swap_gate_up", "drop_bias",
                                     "tie_to_higher_id", "no_renormalise", "transpose_down",
                                     "gamma_without_sigmoid", "union_sorted",
                                     "combine_drops_weight", "layer_combine_drops_weight",
                                     "prefill_combine_drops_weight", "gate_sign"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    orig = {n: getattr(mo, n) for n in ("unpack_codes", "read_expert", "dequant",
                                        "topk_softmax", "union_slots", "shared_gate",
                                        "layer_forward", "prefill_forward")}
    if mistake == "nibble_order":
        def bad(packed, n, bits):
            c = orig["unpack_codes"](packed, n, bits)
            return c.reshape(c.shape[0], -1, 2)[:, :, ::-1].reshape(c.shape) if bits == 4 else c
        _planted(monkeypatch, "unpack_codes", bad)
        checks = [test_unpack_matches_golden_words]
    elif mistake == "swap_gate_up":
        def bad(pool, desc, H, I):
            g, u, d = orig["read_expert"](pool, desc, H, I)
            return u, g, d
        _planted(monkeypatch, "read_expert", bad)
        checks = [lambda: test_single_expert_equals_dense_mlp(4)]
    elif mistake == "drop_bias":
        def bad(codes, sb):
            sb = np.asarray(sb).astype(np.uint32) & 0xFFFF
            return orig["dequant"](codes, sb)
        _planted(monkeypatch, "dequant", bad)
        checks = [test_dequant_closed_form_constant_codes]
    elif mistake == "tie_to_higher_id":
        def bad(l, k):
            order = sorted(range(len(l)), key=lambda e: (-l[e], -e))[:k]
            sel = np.array([l[e] for e in order])
            ex = np.exp(sel - sel[0])
            return np.array(order), ex / ex.sum()
        _planted(monkeypatch, "topk_softmax", bad)
        checks = [test_topk_matches_lexsort_and_ties]
    elif mistake == "no_renormalise":
        def bad(l, k):
            idx, _ = orig["topk_softmax"](l, k)
            full = np.exp(l - l.max())
            return idx, full[idx] / full.sum()
        _planted(monkeypatch, "topk_softmax", bad)
        checks = [test_topk_weights_softmax]
    elif mistake == "transpose_down":
        def bad(pool, desc, H, I):
            g, u, d = orig["read_expert"](pool, desc, H, I)
            # same shape, wrong element order inside each row
            return g, u, d[:, ::-1]
        _planted(monkeypatch, "read_expert", bad)
        checks = [lambda: test_single_expert_equals_dense_mlp(3)]
    elif mistake == "gamma_without_sigmoid":
        def bad(x, gvec):
            return np.asarray(x, dtype=np.float64) @ mo.bf16_to_f64(gvec)
        _planted(monkeypatch, "shared_gate", bad)
        checks = [test_golden_tiny_layer]
    elif mistake == "union_sorted":
        def bad(idx, w, rec):
            s = orig["union_slots"](np.sort(idx, axis=1), w, rec)
            return s
        _planted(monkeypatch, "union_slots", bad)
        checks = [test_union_slots_first_seen]
    elif mistake in ("combine_drops_weight", "layer_combine_drops_weight",
                     "prefill_combine_drops_weight"):
        # the routing weight left out of the combine, in one function or both
        if mistake != "prefill_combine_drops_weight":
            _planted(monkeypatch, "layer_forward",
                     _edited(orig["layer_forward"], LAYER_COMBINE, "acc[b] += y"))
        if mistake != "layer_combine_drops_weight":
            _planted(monkeypatch, "prefill_forward",
                     _edited(orig["prefill_forward"], PREFILL_COMBINE, "acc[r_] += y"))
        checks = [test_golden_tiny_layer_k2, test_zero_scales_layer_closed_form]
    elif mistake == "gate_sign":
        def bad(x, gvec):
            return mo.sigmoid(-(np.asarray(x, dtype=np.float64) @ mo.bf16_to_f64(gvec)))
        _planted(monkeypatch, "shared_gate", bad)
        checks = [test_golden_tiny_layer_k2, test_zero_scales_layer_closed_form]
    for check in checks:
        with pytest.raises(AssertionError):
            check()
