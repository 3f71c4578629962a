"""Host-only checks of the C ABI: the library loads, exports every function
include/moe.h declares, sizes records and workspaces, and rejects bad
arguments before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
moe = pytest.importorskip("quantized_routed_expert_bf16_amd")


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert "moe_layer_forward" in names and "moe_route" in names and "moe_prefill_forward" in names
    for n in names:
        assert hasattr(moe.lib, n), n


def test_record_bytes():
    assert moe.record_bytes(2048, 512, 4) == 1769472
    assert moe.record_bytes(2048, 512, 3) == 1376256
    assert moe.record_bytes(2048, 512, 2) == 983040
    assert moe.record_bytes(256, 128, 4) == 55296
    assert moe.record_bytes(2048, 512, 5) == 0
    assert moe.record_bytes(300, 512, 4) == 0


def test_record_bytes_match_generator():
    import synthetic as syn
    for H, I in ((256, 128), (2048, 512), (4096, 64), (512, 2048)):
        for bits in (4, 3, 2):
            assert moe.record_bytes(H, I, bits) == syn.record_bytes(H, I, bits)


def test_workspace_bytes():
    d = moe.make_dims(2048, 512, 128, 8)
    n4 = moe.workspace_bytes(d, 4)
    n32 = moe.workspace_bytes(d, 32)
    assert n4 > 0 and n32 >= n4 and n4 % 256 == 0
    assert moe.workspace_bytes(d, 0) == 0 and moe.workspace_bytes(d, 33) == 0
    for bad in (moe.make_dims(300, 512, 128, 8), moe.make_dims(2048, 96, 128, 8),
                moe.make_dims(2048, 512, 0, 1), moe.make_dims(2048, 512, 128, 16),
                moe.make_dims(2048, 512, 4, 8), moe.make_dims(8192, 512, 128, 8)):
        assert moe.workspace_bytes(bad, 4) == 0


# fake device addresses: validation never dereferences them
A = 1 << 20


def _args(H=2048, I=512, E=128, k=8, ws_bytes=None):
    d = moe.make_dims(H, I, E, k)
    router = moe.MoeRouter(d, A, A + 4096)
    pool = moe.MoePool(A * 16, 1 << 34)
    shared = moe.MoeShared(A + 8192, 0)
    nbytes = moe.workspace_bytes(d, 4) if ws_bytes is None else ws_bytes
    slots = moe.MoeSlots(A + 1024 * 1, A + 1024 * 2, A + 1024 * 3, A + 1024 * 4, A + 1024 * 5,
                         A + 1024 * 6, A + 1024 * 7, A * 2, nbytes)
    return d, router, pool, shared, slots


def _call(x=A * 4, nb=1, out=A * 5, **kw):
    d, router, pool, shared, slots = _args(**kw)
    return moe.lib.moe_layer_forward(x, nb, ctypes.byref(router), ctypes.byref(slots),
                                     ctypes.byref(pool), ctypes.byref(shared), out, None)


@pytest.mark.parametrize("nb", [0, 5, -1])
def test_rejects_bad_nb(nb):
    assert _call(nb=nb) == moe.EINVAL
    assert "nb" in moe.last_error()


@pytest.mark.parametrize("kw,word", [
    (dict(H=300), "hidden"), (dict(H=128), "hidden"), (dict(I=96), "inter"),
    (dict(I=4096), "inter"), (dict(E=0), "n_experts"), (dict(E=300), "n_experts"),
    (dict(k=16), "top_k"), (dict(E=4, k=5), "top_k"),
])
def test_rejects_bad_dims(kw, word):
    assert _call(**kw) == moe.EINVAL
    assert word in moe.last_error()


def test_rejects_null_and_misaligned():
    assert _call(x=0) == moe.EINVAL and "x is NULL" in moe.last_error()
    assert _call(x=A * 4 + 4) == moe.EINVAL and "aligned" in moe.last_error()
    assert _call(out=0) == moe.EINVAL and "out" in moe.last_error()


def test_rejects_small_workspace():
    assert _call(ws_bytes=1024) == moe.EWORKSPACE
    assert "workspace" in moe.last_error()


def test_rejects_shared_outside_pool_or_lowbit():
    d, router, pool, shared, slots = _args()
    pool.bytes = 1000
    rc = moe.lib.moe_layer_forward(A * 4, 1, ctypes.byref(router), ctypes.byref(slots),
                                   ctypes.byref(pool), ctypes.byref(shared), A * 5, None)
    assert rc == moe.EINVAL and "outside" in moe.last_error()
    d, router, pool, shared, slots = _args()
    shared.rec = 256 | 2
    rc = moe.lib.moe_layer_forward(A * 4, 1, ctypes.byref(router), ctypes.byref(slots),
                                   ctypes.byref(pool), ctypes.byref(shared), A * 5, None)
    assert rc == moe.EINVAL and "4-bit" in moe.last_error()


def test_prefill_rejects_bad_rows():
    d, router, pool, shared, _ = _args()
    plan = moe.MoePrefillPlan(*([A + 1024 * i for i in range(1, 8)]), A * 2,
                              moe.workspace_bytes(d, 32))
    for t in (0, 33):
        rc = moe.lib.moe_prefill_forward(A * 4, t, ctypes.byref(router), ctypes.byref(plan),
                                         ctypes.byref(pool), ctypes.byref(shared), A * 5, None)
        assert rc == moe.EINVAL and "t " in moe.last_error()


def test_route_and_init_validation():
    d, router, pool, shared, slots = _args()
    rc = moe.lib.moe_route(A * 4, 9, ctypes.byref(router), ctypes.byref(shared),
                           ctypes.byref(slots), None)
    assert rc == moe.EINVAL
    assert moe.lib.moe_workspace_init(None, 256, None) == moe.EWORKSPACE
    assert moe.lib.moe_workspace_init(A + 3, 256, None) == moe.EINVAL


def _noalloc(nb=1, **kw):
    d, router, pool, shared, slots = _args(**kw)
    s0 = moe.slots_without_workspace(slots)
    return moe.lib.moe_layer_forward_noalloc(A * 4, nb, ctypes.byref(router), ctypes.byref(s0),
                                             ctypes.byref(pool), ctypes.byref(shared), A * 5, None), slots


def test_noalloc_rejects_before_any_hip_call():
    # sizes past the 3 MiB static scratch, a caller workspace, and the usual checks
    rc, _ = _noalloc(I=2048)
    assert rc == moe.EWORKSPACE and "static" in moe.last_error()
    rc, _ = _noalloc(H=4096, I=1024)
    assert rc == moe.EWORKSPACE
    d, router, pool, shared, slots = _args()
    rc = moe.lib.moe_layer_forward_noalloc(A * 4, 1, ctypes.byref(router), ctypes.byref(slots),
                                           ctypes.byref(pool), ctypes.byref(shared), A * 5, None)
    assert rc == moe.EINVAL and "ws must be NULL" in moe.last_error()
    rc, _ = _noalloc(nb=5)
    assert rc == moe.EINVAL and "nb" in moe.last_error()
    rc, _ = _noalloc(H=300)
    assert rc == moe.EINVAL and "hidden" in moe.last_error()
