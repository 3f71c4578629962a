"""CPU oracle of the routed-expert MoE layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library:
it has its own record reader, its own unpacker and its own arithmetic, all in
float64, written as the plain definition of what the layer computes.

What is computed (sources are the three pages on the qwen4_exp GPU engine:
the rustdoc page "Struct Gpu", and the source pages gpu.rs and gpu/load.rs):

* Dequantisation (gpu.rs, struct ``Q``, the affine 4-bit projection; load.rs, the
  ``q`` closure that reads ``.weight``/``.scales``/``.biases``; the
  expert-width check naming the 64-code quantisation group):
  W[o][i] = q[o][i] * s[o][i // 64] + b[o][i // 64].
* Router (Struct Gpu, ``router_b``: softmax over the router logits, then top-k; the router
  weight is the bf16 tensor ``mlp.gate.weight`` of load.rs):
  logits[b][e] = sum_i R[e][i] * x[b][i].
* Top-k: the k largest logits, ties to the lower expert id, ordered by
  descending logit; weights are the softmax over the k selected logits, i.e.
  the full softmax renormalised over the top-k (reading chosen because the
  pages leave renormalisation open).
* Union and slot table (gpu.rs, ``union_of``: the union keeps each expert
  once, in the order it is first met walking the (row, rank) list row by row;
  the ``slot_tab``/``wmap`` field docs: 64 entries per layer, entry 62 =
  resident count, 63 = union size; per-row routing weight per slot).
* Experts (Struct Gpu, ``experts_b``: routed experts of the union plus the
  shared expert, summed per row): a = silu(Wg x) * (Wu x), y = Wd a, with
  silu(g) = g / (1 + exp(-g)).
* Shared expert (load.rs, ``Moe``: ``shared_expert_gate.weight`` bf16 plus the
  shared gate/up/down projections; the check that the shared width equals the
  routed width): gamma_b = sigmoid(sum_i gvec[i] x[b][i]), weight gamma_b.
* Output (Struct Gpu, ``encode_block``: the MoE output is left for the next
  fused norm, so no residual is added):
  out[b] = sum_j w[b][j] y_j[b] + gamma_b y_shared[b], rounded to f32 once.
* Prefill (Struct Gpu, ``prepare_expert_jobs`` and ``pf_experts``): the same
  per-row result for t rows, with rows grouped by expert (expert ids
  ascending, rows ascending inside an expert).

Parity pins: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` against closed forms, library routines, brute
force or hand-computed fixtures under ``tests/golden/``.
"""
from __future__ import annotations

import numpy as np

GROUP = 64          # codes per quantisation group along the input dimension
SLOT_STRIDE = 64    # slot table entries per layer
RESIDENT_ENTRY = 62
UNION_ENTRY = 63
MAX_NB = 4
BITS_OF_TAG = {0: 4, 1: 3, 2: 2}


# ---------------------------------------------------------------- records --

def _round_up(n: int, a: int) -> int:
    return -(-n // a) * a


def record_layout(hidden: int, inter: int, bits: int) -> dict:
    """Section offsets of one record, read from the record format: gate/up
    codes (2I rows of H codes), their (s,b) words, down codes (I/64 column
    groups of H rows of 64 codes), their (s,b) words (group-major too); each
    section 256-byte aligned."""
    sizes = [
        ("gu_codes", 2 * inter * hidden * bits // 8),
        ("gu_sb", 2 * inter * (hidden // GROUP) * 4),
        ("d_codes", hidden * inter * bits // 8),
        ("d_sb", hidden * (inter // GROUP) * 4),
    ]
    out = {}
    pos = 0
    for name, size in sizes:
        out[name] = (pos, size)
        pos = _round_up(pos + size, 256)
    out["total"] = pos
    return out


def unpack_codes(packed: np.ndarray, n: int, bits: int) -> np.ndarray:
    """Codes [rows][n] of packed rows [rows][n*bits/8] (uint8)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    i = np.arange(n)
    if bits == 4:
        words = packed.view("<u4").reshape(rows, n // 8).astype(np.int64)
        return (words[:, i // 8] >> (4 * (i % 8))) & 0xF
    if bits == 2:
        words = packed.view("<u4").reshape(rows, n // 16).astype(np.int64)
        return (words[:, i // 16] >> (2 * (i % 16))) & 0x3
    if bits == 3:
        low_bytes = n // 4
        low = unpack_codes(packed[:, :low_bytes], n, 2)
        hw = np.ascontiguousarray(packed[:, low_bytes:]).view("<u4")
        hw = hw.reshape(rows, n // 32).astype(np.int64)
        j = i % 32                      # position inside the 32-code block
        bit = 8 * ((j // 4) % 4) + 4 * (j // 16) + j % 4
        high = (hw[:, i // 32] >> bit) & 0x1
        return low + 4 * high
    raise ValueError(f"unsupported bit width {bits}")


def bf16_to_f64(bits16) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits16).astype(np.uint32) & 0xFFFF
    return (b << 16).view(np.float32).astype(np.float64)


def dequant(codes: np.ndarray, sb_words: np.ndarray) -> np.ndarray:
    """W[o][i] = q[o][i] * s[o][i//64] + b[o][i//64] in float64."""
    sb = np.asarray(sb_words).astype(np.uint32)
    s = bf16_to_f64(sb & 0xFFFF)
    b = bf16_to_f64(sb >> 16)
    g = np.arange(codes.shape[1]) // GROUP
    return codes.astype(np.float64) * s[:, g] + b[:, g]


def read_expert(pool, desc: int, hidden: int, inter: int):
    """Dequantised (Wg [I][H], Wu [I][H], Wd [H][I]) of the record at desc.

    ``pool`` is any object whose slice ``pool[a:b]`` gives the bytes a..b-1.
    """
    desc = int(desc)
    bits = BITS_OF_TAG[desc & 0x3]
    base = desc & ~0xFF
    lay = record_layout(hidden, inter, bits)

    def sect(name):
        o, size = lay[name]
        return np.asarray(pool[base + o: base + o + size], dtype=np.uint8)

    gu_q = unpack_codes(sect("gu_codes").reshape(2 * inter, -1), hidden, bits)
    gu_sb = sect("gu_sb").view("<u4").reshape(2 * inter, hidden // GROUP)
    n_groups = inter // GROUP
    # down codes are stored group-major: [group][row][64 codes]
    d_grouped = unpack_codes(sect("d_codes").reshape(n_groups * hidden, -1), GROUP, bits)
    d_q = d_grouped.reshape(n_groups, hidden, GROUP).transpose(1, 0, 2).reshape(hidden, inter)
    d_sb = sect("d_sb").view("<u4").reshape(n_groups, hidden).T
    gu = dequant(gu_q, gu_sb)
    return gu[0::2], gu[1::2], dequant(d_q, d_sb)


# ---------------------------------------------------------------- routing --

def router_logits(x: np.ndarray, router_bf16: np.ndarray) -> np.ndarray:
    """logits[b][e] = sum_i R[e][i] x[b][i] (float64)."""
    R = bf16_to_f64(router_bf16)
    return np.asarray(x, dtype=np.float64) @ R.T


def topk_softmax(logits_row: np.ndarray, k: int):
    """Brute force: sort experts by (-logit, id), keep k, softmax over them."""
    order = sorted(range(len(logits_row)), key=lambda e: (-logits_row[e], e))[:k]
    sel = np.array([logits_row[e] for e in order], dtype=np.float64)
    ex = np.exp(sel - sel[0])
    return np.array(order, dtype=np.int64), ex / ex.sum()


def route(x: np.ndarray, router_bf16: np.ndarray, k: int):
    """Per row: logits, top-k ids and renormalised weights."""
    logits = router_logits(x, router_bf16)
    idx = np.zeros((logits.shape[0], k), dtype=np.int64)
    w = np.zeros((logits.shape[0], k), dtype=np.float64)
    for b in range(logits.shape[0]):
        idx[b], w[b] = topk_softmax(logits[b], k)
    return logits, idx, w


def union_slots(idx: np.ndarray, w: np.ndarray, rec) -> dict:
    """First-seen union of the rows' ids and the 64-entry slot table."""
    nb, k = idx.shape
    ids = []
    for b in range(nb):
        for r in range(k):
            e = int(idx[b, r])
            if e not in ids:
                ids.append(e)
    u = len(ids)
    assert u <= RESIDENT_ENTRY
    tab = np.zeros(SLOT_STRIDE, dtype=np.uint64)
    ids_arr = np.zeros(SLOT_STRIDE, dtype=np.uint32)
    wmap = np.zeros((MAX_NB, SLOT_STRIDE), dtype=np.float64)
    for j, e in enumerate(ids):
        ids_arr[j] = e
        tab[j] = np.uint64(int(rec[e]))
        for b in range(nb):
            for r in range(k):
                if idx[b, r] == e:
                    wmap[b, j] = w[b, r]
    tab[RESIDENT_ENTRY] = u   # every record is resident in device memory
    tab[UNION_ENTRY] = u
    return {"ids": ids_arr, "tab": tab, "wmap": wmap, "n_union": u}


# ---------------------------------------------------------------- experts --

def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def expert_mlp(Wg, Wu, Wd, xb: np.ndarray):
    """Returns (y [H], act [I]) of one expert on one row (float64)."""
    act = silu(Wg @ xb) * (Wu @ xb)
    return Wd @ act, act


def shared_gate(x: np.ndarray, gvec_bf16: np.ndarray) -> np.ndarray:
    """gamma_b = sigmoid(sum_i gvec[i] x[b][i])."""
    return sigmoid(np.asarray(x, dtype=np.float64) @ bf16_to_f64(gvec_bf16))


def layer_forward(x, router_bf16, rec, pool, gvec_bf16, shared_desc, k,
                  hidden, inter) -> dict:
    """One MoE layer over nb rows: routing, union/slots, experts, combine."""
    x = np.asarray(x, dtype=np.float32)
    nb = x.shape[0]
    xd = x.astype(np.float64)
    logits, idx, w = route(x, router_bf16, k)
    slots = union_slots(idx, w, rec)
    gamma = shared_gate(x, gvec_bf16)
    acc = np.zeros((nb, hidden), dtype=np.float64)
    act = {}
    for j in range(slots["n_union"]):
        Wg, Wu, Wd = read_expert(pool, int(slots["tab"][j]), hidden, inter)
        for b in range(nb):
            if slots["wmap"][b, j] != 0.0:
                y, a = expert_mlp(Wg, Wu, Wd, xd[b])
                acc[b] += slots["wmap"][b, j] * y
                act[(j, b)] = a
    Wg, Wu, Wd = read_expert(pool, int(shared_desc), hidden, inter)
    for b in range(nb):
        y, a = expert_mlp(Wg, Wu, Wd, xd[b])
        acc[b] += gamma[b] * y
        act[("shared", b)] = a
    return {"out": acc.astype(np.float32), "out_f64": acc, "logits": logits,
            "topk_idx": idx, "topk_w": w, "gamma": gamma, "act": act, **slots}


def expert_csr(idx: np.ndarray, w: np.ndarray, n_experts: int) -> dict:
    """Rows grouped by expert: experts ascending, rows ascending inside one."""
    t, k = idx.shape
    ptr = np.zeros(n_experts + 1, dtype=np.int64)
    rows, wts, ranks = [], [], []
    for e in range(n_experts):
        for r_ in range(t):
            for c in range(k):
                if idx[r_, c] == e:
                    rows.append(r_)
                    wts.append(w[r_, c])
                    ranks.append(c)
        ptr[e + 1] = len(rows)
    return {"ptr": ptr, "rows": np.array(rows, dtype=np.int64),
            "wts": np.array(wts), "ranks": np.array(ranks, dtype=np.int64)}


def prefill_forward(x, router_bf16, rec, pool, gvec_bf16, shared_desc, k,
                    hidden, inter) -> dict:
    """t rows of a prefill chunk, each routed independently (float64)."""
    x = np.asarray(x, dtype=np.float32)
    t = x.shape[0]
    xd = x.astype(np.float64)
    n_experts = len(rec)
    logits, idx, w = route(x, router_bf16, k)
    csr = expert_csr(idx, w, n_experts)
    gamma = shared_gate(x, gvec_bf16)
    acc = np.zeros((t, hidden), dtype=np.float64)
    for e in range(n_experts):
        lo, hi = csr["ptr"][e], csr["ptr"][e + 1]
        if lo == hi:
            continue
        Wg, Wu, Wd = read_expert(pool, int(rec[e]), hidden, inter)
        for p in range(lo, hi):
            r_ = csr["rows"][p]
            y, _ = expert_mlp(Wg, Wu, Wd, xd[r_])
            acc[r_] += csr["wts"][p] * y
    Wg, Wu, Wd = read_expert(pool, int(shared_desc), hidden, inter)
    for r_ in range(t):
        y, _ = expert_mlp(Wg, Wu, Wd, xd[r_])
        acc[r_] += gamma[r_] * y
    return {"out": acc.astype(np.float32), "out_f64": acc, "logits": logits,
            "topk_idx": idx, "topk_w": w, "gamma": gamma, **csr}


# ------------------------------------------------------------- low-bit store --
# The pages build a 3- or 2-bit copy of every expert record from the 4-bit
# source once (gpu/load.rs source page, load_bounded: the low-bit store set
# up by lowbit::ensure_with_policy, a record stride below the 4-bit one) and
# give no rule for the requantization.  The reading taken here is plain
# min/max affine requantization of each 64-code group of dequantised
# weights, w = q s + b: the group's weights span [lo, hi] with lo and hi at
# its extreme codes, and the new grid of 2^bits - 1 steps spans the same
# interval.  Because w is affine in q, the new code of every weight is an
# exact rational of the old codes, rounded half up, so it is computed in
# integers; the new scale and bias are float32 operations rounded to bf16.

def _f32_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns, round to nearest even (finite v)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (rounded & 0xFFFF).astype(np.uint16)


def requantize_group_codes(q: np.ndarray, s16: np.ndarray, b16: np.ndarray, bits: int):
    """Requantize groups of 64 4-bit codes (q [n][64], with bf16 scale and
    bias bit patterns [n]) to `bits` bits.  Returns (codes [n][64], scale
    bf16 [n], bias bf16 [n])."""
    q = np.asarray(q, dtype=np.int64)
    s = bf16_to_f64(s16).astype(np.float32)
    b = bf16_to_f64(b16).astype(np.float32)
    levels = (1 << bits) - 1
    qmin, qmax = q.min(axis=1), q.max(axis=1)
    neg = s < 0
    q_lo = np.where(neg, qmax, qmin)          # code of the smallest weight
    q_hi = np.where(neg, qmin, qmax)          # code of the largest weight
    d = np.abs(q_hi - q_lo)                    # steps between them, 0..15
    t = np.abs(q - q_lo[:, None]) * levels     # (w - lo) / s_old in new-step units times d
    safe_d = np.maximum(d, 1)[:, None]
    codes = np.where(d[:, None] > 0, (2 * t + safe_d) // (2 * safe_d), 0)
    # scale: |s| d / levels (|s| d is exact in float32), bias: b + s q_lo
    step = (np.abs(s) * d.astype(np.float32)) / np.float32(levels)
    bias = b + s * q_lo.astype(np.float32)
    step = np.where(d > 0, step, np.float32(0.0)).astype(np.float32)
    return codes, _f32_to_bf16_rne(step), _f32_to_bf16_rne(bias.astype(np.float32))


def repack_record(pool, desc: int, bits: int, hidden: int, inter: int) -> dict:
    """A 4-bit record requantized to `bits` bits: raw codes and bf16 (s, b)
    in the layout the record writer takes (gate/up [2I][H], [2I][H/64];
    down [H][I], [H][I/64])."""
    desc = int(desc)
    assert BITS_OF_TAG[desc & 0x3] == 4, "the source record must be 4-bit"
    base = desc & ~0xFF
    lay = record_layout(hidden, inter, 4)

    def sect(name):
        o, size = lay[name]
        return np.asarray(pool[base + o: base + o + size], dtype=np.uint8)

    gu_q = unpack_codes(sect("gu_codes").reshape(2 * inter, -1), hidden, 4)
    gu_sb = sect("gu_sb").view("<u4").reshape(2 * inter, hidden // GROUP)
    n_groups = inter // GROUP
    d_grouped = unpack_codes(sect("d_codes").reshape(n_groups * hidden, -1), GROUP, 4)
    d_sb = sect("d_sb").view("<u4").reshape(n_groups, hidden)     # [group][row]

    def requant(codes_rows, sb_words):
        rows, n = codes_rows.shape
        g = codes_rows.reshape(rows * (n // GROUP), GROUP)
        w = sb_words.reshape(-1)
        c, s16, b16 = requantize_group_codes(g, w & 0xFFFF, w >> 16, bits)
        return c.reshape(rows, n), s16.reshape(sb_words.shape), b16.reshape(sb_words.shape)

    gq, gs, gb = requant(gu_q, gu_sb)
    # down groups are stored group-major: row r of group g holds codes 64g..64g+63 of row r
    dq_g, ds_g, db_g = requant(d_grouped, d_sb.reshape(-1, 1))
    dq = dq_g.reshape(n_groups, hidden, GROUP).transpose(1, 0, 2).reshape(hidden, inter)
    ds = ds_g.reshape(n_groups, hidden).T
    db = db_g.reshape(n_groups, hidden).T
    return {"gu_q": gq, "gu_s": gs, "gu_b": gb, "d_q": dq, "d_s": ds, "d_b": db}
