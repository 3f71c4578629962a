"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only draws random numbers and lays them out in memory: it holds
none of the layer's arithmetic (no dequantisation, no matvec, no routing).
Both the CPU oracle (``oracle/``) and the HIP library's tests and benchmark
take their inputs from here, so the two sides always see the same bits.

Record layout written here (one routed or shared expert = one record in a
byte pool; every section starts on a 256-byte boundary):

  section   layout                                 content
  GU codes  2*I rows x H*bits/8 bytes (gate j at   packed codes, input dim H
            row 2j, up j at row 2j+1)
  GU sb     2*I rows x (H/64) words                (scale, bias) bf16 pairs
  D codes   I/64 column groups, each H rows x      packed codes, input dim I,
            64*bits/8 bytes (group g of row r =    group-major
            codes 64g..64g+63 of row r packed as
            a 64-code row)
  D sb      I/64 column groups, each H words       (scale, bias) bf16 pairs

Code packing inside a row (little-endian u32 words):
  4-bit: code i is bits [4*(i%8), 4*(i%8)+4) of word i//8.
  2-bit: code i is bits [2*(i%16), 2*(i%16)+2) of word i//16.
  3-bit: the row is two planes: first the low two bits of every code packed
         exactly like a 2-bit row (n/4 bytes), then the high bits (n/8 bytes),
         one u32 word per 32-code block; code i of a block (m = i//16,
         k = (i//4)%4, p = i%4) has its high bit at bit 8k + 4m + p.
An (s, b) pair is one u32 word: bf16 bits of s in the low half, of b in the
high half.  A record descriptor is ``byte_offset | tag`` with the offset a
multiple of 256 and tag 0/1/2 for 4/3/2-bit codes.

The affine 4-bit projection with separate scales and biases, 8 codes per u32
word and 64-code groups along the input dimension follow the "Q" projection
type and the expert-width check in the gpu.rs and load.rs source pages; the
3/2-bit records and their kind codes follow the low-bit store described in
load.rs (``load_bounded``).  The exact bit order, the interleaving of gate and
up rows and the section alignment are this project's own choices.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

GROUP = 64
ALIGN = 256
TAG_OF_BITS = {4: 0, 3: 1, 2: 2}


def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def row_bytes(n_codes: int, bits: int) -> int:
    """Bytes taken by one packed row of ``n_codes`` codes."""
    assert n_codes % GROUP == 0
    return n_codes * bits // 8


def record_sections(hidden: int, inter: int, bits: int) -> dict:
    """Byte offsets and sizes of the four sections of one record."""
    gu_codes = 2 * inter * row_bytes(hidden, bits)
    gu_sb = 2 * inter * (hidden // GROUP) * 4
    d_codes = hidden * row_bytes(inter, bits)
    d_sb = hidden * (inter // GROUP) * 4
    off = {}
    pos = 0
    for name, size in (("gu_codes", gu_codes), ("gu_sb", gu_sb),
                       ("d_codes", d_codes), ("d_sb", d_sb)):
        off[name] = (pos, size)
        pos = _align(pos + size)
    off["total"] = pos
    return off


def record_bytes(hidden: int, inter: int, bits: int) -> int:
    return record_sections(hidden, inter, bits)["total"]


# --------------------------------------------------------------------------
# packing (used for structured test records; random records are random bytes)
# --------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes [rows][n] into bytes [rows][n*bits/8]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint64)
    rows, n = codes.shape
    assert n % GROUP == 0 and codes.max(initial=0) < (1 << bits)
    if bits in (4, 2):
        per = 32 // bits
        c = codes.reshape(rows, n // per, per)
        shifts = (np.arange(per, dtype=np.uint64) * bits)
        words = (c << shifts).sum(axis=2).astype(np.uint32)
        return words.view(np.uint8).reshape(rows, -1)
    if bits == 3:
        low = pack_codes(codes & 3, 2)
        hb = (codes >> 2).reshape(rows, n // 32, 32)
        i = np.arange(32, dtype=np.uint64)
        pos = 8 * ((i // 4) % 4) + 4 * (i // 16) + i % 4
        words = (hb << pos).sum(axis=2).astype(np.uint32)
        high = words.view(np.uint8).reshape(rows, -1)
        return np.concatenate([low, high], axis=1)
    raise ValueError(bits)


def sb_words(scale_bf16: np.ndarray, bias_bf16: np.ndarray) -> np.ndarray:
    """Interleave bf16 bit patterns (uint16) of s and b into u32 words."""
    s = np.asarray(scale_bf16, dtype=np.uint16).astype(np.uint32)
    b = np.asarray(bias_bf16, dtype=np.uint16).astype(np.uint32)
    return (s | (b << 16)).astype(np.uint32)


def f32_to_bf16_bits(v) -> np.ndarray:
    """Round-to-nearest-even f32 -> bf16 bit patterns (uint16)."""
    t = torch.as_tensor(np.asarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def write_record(pool: np.ndarray, offset: int, hidden: int, inter: int, bits: int,
                 gu_codes, gu_s, gu_b, d_codes, d_s, d_b) -> int:
    """Write one record with explicit codes and bf16 (s, b) into a host pool.

    gu_codes [2I][H] (gate j at row 2j, up j at row 2j+1), gu_s/gu_b [2I][H/64]
    bf16 bit patterns; d_codes [H][I], d_s/d_b [H][I/64].  Returns the
    descriptor.
    """
    sec = record_sections(hidden, inter, bits)
    assert offset % ALIGN == 0 and offset + sec["total"] <= pool.size

    def put(name, arr):
        o, size = sec[name]
        flat = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert flat.size == size, (name, flat.size, size)
        pool[offset + o: offset + o + size] = flat

    put("gu_codes", pack_codes(gu_codes, bits))
    put("gu_sb", sb_words(gu_s, gu_b))
    d_codes = np.asarray(d_codes)
    n_groups = d_codes.shape[1] // GROUP
    # group-major: [group][row][64 codes packed]
    grouped = d_codes.reshape(d_codes.shape[0], n_groups, GROUP).transpose(1, 0, 2)
    put("d_codes", pack_codes(grouped.reshape(-1, GROUP), bits))
    put("d_sb", np.ascontiguousarray(sb_words(d_s, d_b).T))
    return offset | TAG_OF_BITS[bits]


# --------------------------------------------------------------------------
# workload configurations
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    n_layers: int
    nb: int               # rows per step (decode) or rows per chunk (prefill)
    bits: str             # "q4", "q3", "q2" or "mixed" (routed experts; shared is q4)
    x_mode: str           # "iid", "correlated" or "zipf"
    steps: int            # steps (decode) or chunks (prefill) of the benchmark
    prefill: bool = False
    description: str = ""


CONFIGS = {
    "tiny": MoeConfig("tiny", 256, 128, 8, 2, 1, 1, "q4", "iid", 1,
                      description="hidden 256, expert width 128, 8 experts, top-2, nb=1, 1 layer"),
    "decode_nb1": MoeConfig("decode_nb1", 2048, 512, 128, 8, 40, 1, "q4", "iid", 1000,
                            description="decode nb=1, hidden 2048, width 512, 128 experts, "
                                        "top-8, Q4, 40 layers"),
    "verify_nb4": MoeConfig("verify_nb4", 2048, 512, 128, 8, 40, 4, "q4", "correlated", 1000,
                            description="speculative-verify nb=4, correlated rows"),
    "lowbit_q3": MoeConfig("lowbit_q3", 2048, 512, 128, 8, 40, 4, "q3", "correlated", 1000,
                           description="nb=4, every routed expert 3-bit"),
    "lowbit_q2": MoeConfig("lowbit_q2", 2048, 512, 128, 8, 40, 4, "q2", "correlated", 1000,
                           description="nb=4, every routed expert 2-bit"),
    "mixed_q4q2": MoeConfig("mixed_q4q2", 2048, 512, 128, 8, 40, 4, "mixed", "correlated", 1000,
                            description="nb=4, per layer 32 of 128 experts 2-bit, rest 4-bit"),
    "prefill_t32": MoeConfig("prefill_t32", 2048, 512, 128, 8, 40, 32, "q4", "zipf", 16,
                             prefill=True,
                             description="prefill chunks of 32 rows, Zipf(1.1)-skewed routing"),
}


def expert_bits(cfg: MoeConfig, layer_gen: torch.Generator) -> list[int]:
    """Bit width of each routed expert of one layer."""
    if cfg.bits == "mixed":
        perm = torch.randperm(cfg.n_experts, generator=layer_gen)
        low = set(perm[: cfg.n_experts // 4].tolist())
        return [2 if e in low else 4 for e in range(cfg.n_experts)]
    return [int(cfg.bits[1])] * cfg.n_experts


@dataclasses.dataclass
class Problem:
    cfg: MoeConfig
    pool: torch.Tensor           # uint8 [bytes]
    rec: torch.Tensor            # int64 [L][E] descriptors (offset | tag)
    router: torch.Tensor         # bfloat16 [L][E][H]
    shared_gate: torch.Tensor    # bfloat16 [L][H]
    shared_rec: torch.Tensor     # int64 [L]
    bits: list                   # [L][E] bit widths of routed experts
    zipf_dir: torch.Tensor | None = None   # float32 [L][H] unit vectors (zipf configs)


def _bf16_bits(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16).view(torch.int16).to(torch.int32) & 0xFFFF


def _fill_sb(pool: torch.Tensor, off: int, n_words: int, bits: int, noise: float,
             gen: torch.Generator) -> None:
    dev = pool.device
    s = torch.empty(n_words, device=dev).uniform_(0.002, 0.02, generator=gen)
    s16 = s.to(torch.bfloat16)
    b = -float(1 << (bits - 1)) * s16.float()
    if noise:
        b = b + noise * torch.randn(n_words, device=dev, generator=gen)
    w = _bf16_bits(s16) | (_bf16_bits(b) << 16)
    pool[off: off + 4 * n_words] = w.to(torch.int32).view(torch.uint8)


def make_problem(cfg: MoeConfig, seed: int = 0, device="cpu",
                 n_layers: int | None = None) -> Problem:
    """Build the pool, routers and shared experts of a configuration.

    Codes are uniform over 0..2^bits-1 (uniform random bytes give exactly that
    in every packing above), scales U(0.002, 0.02) rounded to bf16, biases
    -2^(bits-1)*scale (+ N(0, 1e-3) for 4-bit records), router rows and the
    shared gate vector bf16 N(0, 0.02).  For the Zipf prefill workload each
    layer's router rows get a skew along a seeded unit vector u: expert e of
    seeded rank r_e gets + (-1.1 ln r_e) * u / sqrt(H/2).
    """
    L = cfg.n_layers if n_layers is None else n_layers
    H, I, E = cfg.hidden, cfg.inter, cfg.n_experts
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    cpu_gen = torch.Generator()
    cpu_gen.manual_seed(seed + 7919)

    bits = [expert_bits(cfg, cpu_gen) for _ in range(L)]
    # offsets: layer-major routed records, then one shared record per layer
    offs = []
    pos = 0
    for l in range(L):
        row = []
        for e in range(E):
            row.append(pos | TAG_OF_BITS[bits[l][e]])
            pos += record_bytes(H, I, bits[l][e])
        offs.append(row)
    shared = []
    for l in range(L):
        shared.append(pos | TAG_OF_BITS[4])
        pos += record_bytes(H, I, 4)
    pool = torch.randint(0, 256, (pos,), dtype=torch.uint8, device=dev, generator=gen)

    def fill(desc: int, b: int):
        off = desc & ~0xFF
        sec = record_sections(H, I, b)
        noise = 1e-3 if b == 4 else 0.0
        for name in ("gu_sb", "d_sb"):
            o, size = sec[name]
            _fill_sb(pool, off + o, size // 4, b, noise, gen)

    for l in range(L):
        for e in range(E):
            fill(offs[l][e], bits[l][e])
        fill(shared[l], 4)

    router = (0.02 * torch.randn(L, E, H, device=dev, generator=gen))
    zipf_dir = None
    if cfg.x_mode == "zipf":
        u = torch.randn(L, H, device=dev, generator=gen)
        u = u / u.norm(dim=1, keepdim=True)
        ranks = torch.stack([torch.randperm(E, generator=cpu_gen) for _ in range(L)]) + 1
        beta = -1.1 * torch.log(ranks.to(torch.float32)).to(dev)          # [L][E]
        router = router + beta[:, :, None] * u[:, None, :] / math.sqrt(H / 2)
        zipf_dir = u
    router = router.to(torch.bfloat16)
    shared_gate = (0.02 * torch.randn(L, H, device=dev, generator=gen)).to(torch.bfloat16)
    return Problem(cfg=cfg, pool=pool,
                   rec=torch.tensor(offs, dtype=torch.int64, device=dev),
                   router=router, shared_gate=shared_gate,
                   shared_rec=torch.tensor(shared, dtype=torch.int64, device=dev),
                   bits=bits, zipf_dir=zipf_dir)


def _rms(x: torch.Tensor) -> torch.Tensor:
    return x / torch.sqrt((x * x).mean(dim=-1, keepdim=True))


def make_x(cfg: MoeConfig, seed: int, steps: int, device="cpu",
           problem: Problem | None = None, rows: int | None = None) -> torch.Tensor:
    """Activations [steps][L][rows][H] f32, RMS-normalised.

    iid: every row N(0,1).  correlated: row 0 = x0, row b>0 = x0 + 0.3 N(0,1).
    zipf: N(0,1) + sqrt(H) u_l (u_l the layer's skew direction).
    """
    L, H = cfg.n_layers, cfg.hidden
    if problem is not None:
        L = problem.rec.shape[0]
    nb = cfg.nb if rows is None else rows
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 1000003 + 17)
    if cfg.x_mode == "iid":
        x = torch.randn(steps, L, nb, H, device=dev, generator=gen)
    elif cfg.x_mode == "correlated":
        x0 = torch.randn(steps, L, 1, H, device=dev, generator=gen)
        n = torch.randn(steps, L, nb, H, device=dev, generator=gen)
        n[:, :, 0] = 0
        x = x0 + 0.3 * n
    elif cfg.x_mode == "zipf":
        assert problem is not None and problem.zipf_dir is not None
        u = problem.zipf_dir.to(dev)
        x = torch.randn(steps, L, nb, H, device=dev, generator=gen) \
            + math.sqrt(H) * u[None, :, None, :]
    else:
        raise ValueError(cfg.x_mode)
    return _rms(x).contiguous()
