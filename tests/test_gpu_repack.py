"""GPU parity of the low-bit store builder (moe_repack) against the oracle's
repack_record: every output byte of every repacked record, through the C ABI;
then a decode layer running on the repacked store."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle.moe_oracle as mo
import synthetic as syn
from gpu_support import DecodeRunner, PoolView, compare_decode, oracle_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_routed_expert_bf16_amd as m
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _expected_bytes(pool_host, desc4, bits, H, I):
    """The oracle's repacked record, written by the generator's writer into
    a zeroed buffer (section padding stays zero, as on the device)."""
    rp = mo.repack_record(pool_host, int(desc4), bits, H, I)
    buf = np.zeros(syn.record_bytes(H, I, bits), dtype=np.uint8)
    syn.write_record(buf, 0, H, I, bits, rp["gu_q"], rp["gu_s"], rp["gu_b"], rp["d_q"], rp["d_s"], rp["d_b"])
    return buf


def _layout_dst(bits_list, H, I):
    descs, pos = [], 0
    for b in bits_list:
        descs.append(pos | syn.TAG_OF_BITS[b])
        pos += syn.record_bytes(H, I, b)
    return descs, pos


@pytest.mark.parametrize("shape", [dict(hidden=256, inter=128), dict(hidden=512, inter=64),
                                   dict(hidden=1024, inter=256)])
def test_repack_bytes_match_oracle(moe, shape):
    H, I = shape["hidden"], shape["inter"]
    cfg = dataclasses.replace(syn.CONFIGS["tiny"], name="custom", n_experts=6, top_k=2, **shape)
    p = syn.make_problem(cfg, seed=13, device="cpu")
    pool = p.pool.numpy().copy()
    src = [int(d) for d in p.rec[0].tolist()]
    # negative scales in record 5: flip the sign bit of every scale
    off = src[5] & ~0xFF
    lay = mo.record_layout(H, I, 4)
    for name in ("gu_sb", "d_sb"):
        o, size = lay[name]
        w = pool[off + o: off + o + size].view("<u4")
        w ^= 0x8000
    bits = [3, 2, 3, 2, 3, 2]
    dst, nbytes = _layout_dst(bits, H, I)
    src_t = torch.tensor(src, dtype=torch.int64, device="cuda")
    dst_t = torch.tensor(dst, dtype=torch.int64, device="cuda")
    pool_d = torch.from_numpy(pool).cuda()
    out_d = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.repack(pool_d, src_t, out_d, dst_t, len(src), H, I, status=status)
    torch.cuda.synchronize()
    out = out_d.cpu().numpy()
    assert int(status.item()) == 0
    for i, (d4, dl, b) in enumerate(zip(src, dst, bits)):
        exp = _expected_bytes(pool, d4, b, H, I)
        o = dl & ~0xFF
        got = out[o: o + exp.size]
        bad = np.nonzero(got != exp)[0]
        assert bad.size == 0, f"record {i} ({b}-bit): {bad.size} bytes differ, first at {bad[:5]}"


def test_repack_bad_descriptor_is_skipped(moe):
    H, I = 256, 128
    cfg = dataclasses.replace(syn.CONFIGS["tiny"], name="custom", n_experts=3, **dict(hidden=H, inter=I))
    p = syn.make_problem(cfg, seed=14, device="cpu")
    pool = p.pool.numpy()
    src = [int(d) for d in p.rec[0].tolist()]
    dst, nbytes = _layout_dst([3, 3, 3], H, I)
    src_bad = list(src)
    src_bad[1] = (pool.size + 4096) & ~0xFF          # past the source pool
    dst_bad = list(dst)
    dst_bad[2] = dst[2] & ~0xFF | 0                  # tag 0: not a low-bit width
    out_d = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.repack(torch.from_numpy(pool.copy()).cuda(), torch.tensor(src_bad, device="cuda"), out_d,
               torch.tensor(dst_bad, device="cuda"), 3, H, I, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & 1
    out = out_d.cpu().numpy()
    exp = _expected_bytes(pool, src[0], 3, H, I)
    np.testing.assert_array_equal(out[: exp.size], exp)
    assert not out[dst[1] & ~0xFF: (dst[1] & ~0xFF) + exp.size].any() and not out[dst[2] & ~0xFF:].any()


@pytest.mark.parametrize("bits", [3, 2])
def test_repack_full_layer_and_decode(moe, bits):
    """The 128 4-bit records of a full-shape layer repacked in one call:
    sampled records byte-exact against the oracle, then a decode layer on the
    repacked store (routed records low-bit, shared expert 4-bit) against the
    oracle on the same bytes."""
    cfg = syn.CONFIGS["decode_nb1"]
    H, I, E = cfg.hidden, cfg.inter, cfg.n_experts
    p = syn.make_problem(cfg, seed=15, device="cuda", n_layers=1)
    dst, nbytes = _layout_dst([bits] * E, H, I)
    shared_off = nbytes
    nbytes += syn.record_bytes(H, I, 4)
    store = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    s_off = int(p.shared_rec[0]) & ~0xFF
    store[shared_off: shared_off + syn.record_bytes(H, I, 4)] = p.pool[s_off: s_off + syn.record_bytes(H, I, 4)]
    dst_t = torch.tensor(dst, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.repack(p.pool, p.rec[0].contiguous(), store, dst_t, E, H, I, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    pv = PoolView(p.pool)
    for e in (0, 57, 127):
        exp = _expected_bytes(pv, int(p.rec[0, e]), bits, H, I)
        o = dst[e] & ~0xFF
        got = store[o: o + exp.size].cpu().numpy()
        np.testing.assert_array_equal(got, exp, err_msg=f"record {e}")
    q = dataclasses.replace(p, pool=store, rec=dst_t[None, :].clone(),
                            shared_rec=torch.tensor([shared_off], dtype=torch.int64, device="cuda"))
    run = DecodeRunner(moe, q)
    x = syn.make_x(cfg, seed=16, steps=1, device="cuda", problem=q)[0, 0]
    g = run.forward(x, 0)
    st = compare_decode(g, oracle_layer(q, x.cpu().numpy(), 0), cfg.top_k, f"decode on the {bits}-bit store")
    _say(f"   decode on the repacked {bits}-bit store: rel err {st['rel']:.2e}")
    assert moe.workspace_status(run.bufs.ws) == 0
