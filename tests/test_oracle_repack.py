"""Pins of the oracle's low-bit store builder (Q4 record -> Q3/Q2 record)
against exact rational arithmetic, closed forms and torch's bf16 rounding.

The rule (min/max affine requantization of each 64-code group, exact in the
code domain) is this project's reading: the pages describe building the
3/2-bit store from the 4-bit source but print no rule.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.moe_oracle as mo
import synthetic as syn


def _bf16_torch(v32: float) -> int:
    """float -> bf16 bit pattern through torch (round to nearest even)."""
    t = torch.tensor([v32], dtype=torch.float32).to(torch.bfloat16)
    return int(t.view(torch.int16).item()) & 0xFFFF


def _f32(v) -> float:
    return float(np.float32(v))


def _bf16_value(bits16: int) -> Fraction:
    return Fraction(float(mo.bf16_to_f64(np.uint16(bits16))))


def _expected_group(q, s16, b16, bits):
    """Codes by exact rationals (nearest level of the new grid, ties up);
    scale and bias by float32 operations rounded to bf16 through torch."""
    s, b = _bf16_value(s16), _bf16_value(b16)
    levels = (1 << bits) - 1
    w = [qi * s + b for qi in q]
    lo, hi = min(w), max(w)
    q_lo = int(min(q)) if s >= 0 else int(max(q))
    q_hi = int(max(q)) if s >= 0 else int(min(q))
    d = abs(q_hi - q_lo)
    if d == 0 or s == 0:
        codes = [0] * len(q)
        step16 = _bf16_torch(0.0)
    else:
        step = (hi - lo) / levels
        codes = []
        for wi in w:
            x = (wi - lo) / step                   # exact position on the new grid
            codes.append(int(x + Fraction(1, 2)) if x >= 0 else 0)   # floor(x + 1/2): ties up
        # |s| d is exact in float32; the division rounds once
        step16 = _bf16_torch(_f32(float(abs(s) * d) / levels))
    bias16 = _bf16_torch(_f32(float(b) + float(s * q_lo)))   # s q_lo exact; one rounding
    return codes, step16, bias16


def _random_groups(rng, n, neg=False):
    q = rng.integers(0, 16, size=(n, 64))
    q[0] = 7                                        # a constant group
    q[1] = np.where(np.arange(64) % 2, 3, 9)        # a narrow range
    s = rng.uniform(0.002, 0.02, size=n) * (np.where(rng.random(n) < 0.5, -1, 1) if neg else 1)
    s16 = syn.f32_to_bf16_bits(s.astype(np.float32))
    b16 = syn.f32_to_bf16_bits((-8 * mo.bf16_to_f64(s16) + 1e-3 * rng.standard_normal(n)).astype(np.float32))
    return q, s16, b16


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("neg", [False, True])
def test_requantize_matches_exact_rationals(bits, neg):
    rng = np.random.default_rng(40 + bits + 10 * neg)
    q, s16, b16 = _random_groups(rng, 24, neg)
    codes, st, bi = mo.requantize_group_codes(q, s16, b16, bits)
    assert codes.min() >= 0 and codes.max() <= (1 << bits) - 1
    for g in range(q.shape[0]):
        ec, es, eb = _expected_group(q[g], int(s16[g]), int(b16[g]), bits)
        np.testing.assert_array_equal(codes[g], ec, err_msg=f"group {g}")
        assert int(st[g]) == es and int(bi[g]) == eb, f"group {g}"


def test_grid_aligned_codes_are_exact():
    # 2-bit: 4-bit codes on the levels {0, 5, 10, 15} of a group spanning
    # 0..15 become q / 5 with scale 5 s and the same bias: the dequantised
    # weights are unchanged (scales chosen so that 5 s is exact in bf16)
    rng = np.random.default_rng(3)
    q = rng.choice([0, 5, 10, 15], size=(8, 64))
    q[:, 0], q[:, 1] = 0, 15
    s16 = syn.f32_to_bf16_bits(np.float32(2.0 ** -6) * np.ones(8, np.float32))
    b16 = syn.f32_to_bf16_bits(np.float32(-0.125) * np.ones(8, np.float32))
    codes, st, bi = mo.requantize_group_codes(q, s16, b16, 2)
    np.testing.assert_array_equal(codes, q // 5)
    np.testing.assert_array_equal(mo.bf16_to_f64(st), 5 * 2.0 ** -6)
    np.testing.assert_array_equal(bi, b16)
    w_old = q * 2.0 ** -6 - 0.125
    w_new = codes * mo.bf16_to_f64(st)[:, None] + mo.bf16_to_f64(bi)[:, None]
    np.testing.assert_array_equal(w_new, w_old)


@pytest.mark.parametrize("bits", [3, 2])
def test_repack_record_roundtrip_and_error(bits):
    """A whole record: the repacked record written with the generator's
    writer reads back (oracle reader) to the requantized weights, every
    weight moves by at most half a new step, and the dense MLP output of the
    repacked expert stays close to the 4-bit one."""
    rng = np.random.default_rng(50 + bits)
    H, I = 256, 128
    r = {"gu_q": rng.integers(0, 16, (2 * I, H)), "d_q": rng.integers(0, 16, (H, I))}
    r["gu_s"] = syn.f32_to_bf16_bits(rng.uniform(0.002, 0.02, (2 * I, H // 64)).astype(np.float32))
    r["d_s"] = syn.f32_to_bf16_bits(rng.uniform(0.002, 0.02, (H, I // 64)).astype(np.float32))
    r["gu_b"] = syn.f32_to_bf16_bits((-8 * mo.bf16_to_f64(r["gu_s"])).astype(np.float32))
    r["d_b"] = syn.f32_to_bf16_bits((-8 * mo.bf16_to_f64(r["d_s"])).astype(np.float32))
    pool = np.zeros(syn.record_bytes(H, I, 4) + syn.record_bytes(H, I, bits), dtype=np.uint8)
    d4 = syn.write_record(pool, 0, H, I, 4, r["gu_q"], r["gu_s"], r["gu_b"], r["d_q"], r["d_s"], r["d_b"])
    rp = mo.repack_record(pool, d4, bits, H, I)
    off = syn.record_bytes(H, I, 4)
    dl = syn.write_record(pool, off, H, I, bits, rp["gu_q"], rp["gu_s"], rp["gu_b"], rp["d_q"], rp["d_s"], rp["d_b"])
    Wg4, Wu4, Wd4 = mo.read_expert(pool, d4, H, I)
    Wgl, Wul, Wdl = mo.read_expert(pool, dl, H, I)
    for old, new, s_new in ((Wg4, Wgl, mo.bf16_to_f64(rp["gu_s"][0::2])),
                            (Wd4, Wdl, mo.bf16_to_f64(rp["d_s"]))):
        half_step = np.repeat(s_new, 64, axis=1) / 2
        # half a new step plus the bf16 rounding of scale and bias
        assert np.all(np.abs(new - old) <= half_step * 1.02 + 1e-3)
    # a sanity bound on the layer-level change (random zero-mean weights:
    # the requantization noise passes through gate/up and down); the exact
    # checks are the rational ones above
    x = rng.standard_normal(H)
    y4, _ = mo.expert_mlp(Wg4, Wu4, Wd4, x)
    yl, _ = mo.expert_mlp(Wgl, Wul, Wdl, x)
    rel = np.linalg.norm(yl - y4) / np.linalg.norm(y4)
    assert rel < (0.8 if bits == 2 else 0.4), rel


@pytest.mark.parametrize("mistake", ["round_down", "wrong_levels", "bias_from_max"])
def test_repack_planted_mistakes_are_caught(monkeypatch, mistake):
    orig = mo.requantize_group_codes

    def bad(q, s16, b16, bits):
        c, st, bi = orig(q, s16, b16, bits)
        if mistake == "round_down":
            q = np.asarray(q)
            t = np.abs(q - q.min(axis=1, keepdims=True)) * ((1 << bits) - 1)
            d = np.maximum(q.max(axis=1, keepdims=True) - q.min(axis=1, keepdims=True), 1)
            c = t // d
        elif mistake == "wrong_levels":
            c = np.minimum(c, (1 << bits) - 2)
        else:
            _, _, bi = orig(q, s16, b16, bits)
            s = mo.bf16_to_f64(s16)
            bi = mo._f32_to_bf16_rne((mo.bf16_to_f64(b16) + s * np.asarray(q).max(axis=1)).astype(np.float32))
        return c, st, bi

    monkeypatch.setattr(mo, "requantize_group_codes", bad)
    with pytest.raises(AssertionError):
        test_requantize_matches_exact_rationals(3, False)
