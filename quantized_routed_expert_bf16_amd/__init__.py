"""Python binding of the routed-expert MoE HIP library (libmoe.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch is used for device memory and streams; the C ABI itself takes
plain pointers (see include/moe.h for layouts, ownership and errors).
Importing this module loads ``libmoe.so`` and raises if it is missing: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MAX_NB = 4
SLOT_STRIDE = 64
RESIDENT_ENTRY = 62
UNION_ENTRY = 63
MAX_PREFILL_ROWS = 32
OK, EINVAL, EWORKSPACE, ELAUNCH = 0, -1, -2, -3
STATUS_BAD_RECORD = 1     # a record descriptor outside the pool (or tag 3) was skipped
STATUS_WAIT_RAN_OUT = 4   # a bounded cross-block wait ran out: the output is not valid


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


class MoeDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class MoeRouter(ctypes.Structure):
    _fields_ = [("dims", MoeDims), ("weight", ctypes.c_void_p), ("rec", ctypes.c_void_p)]


class MoePool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("bytes", ctypes.c_uint64)]


class MoeShared(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("rec", ctypes.c_uint64)]


class MoeSlots(ctypes.Structure):
    _fields_ = [("tab", ctypes.c_void_p), ("wmap", ctypes.c_void_p), ("ids", ctypes.c_void_p),
                ("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("logits", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


class MoePrefillPlan(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("logits", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("expert_ptr", ctypes.c_void_p), ("entry_row", ctypes.c_void_p),
                ("entry_rank", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


class MoeTierConfig(ctypes.Structure):
    _fields_ = [("dims", MoeDims), ("n_layers", ctypes.c_int32), ("host_tier", ctypes.c_void_p),
                ("host_bytes", ctypes.c_uint64), ("host_desc", ctypes.c_void_p),
                ("dev_pool", ctypes.c_void_p), ("dev_bytes", ctypes.c_uint64),
                ("slot_offset", ctypes.c_uint64), ("slot_stride", ctypes.c_uint64),
                ("n_slots", ctypes.c_int32)]


class MoeTierPolicy(ctypes.Structure):
    _fields_ = [("cut_w", ctypes.c_float), ("deadline_now", ctypes.c_int32),
                ("lookahead", ctypes.c_int32), ("timing", ctypes.c_int32)]


class MoeTierStats(ctypes.Structure):
    _fields_ = [("n_union", ctypes.c_int32), ("n_resident", ctypes.c_int32),
                ("n_fetched", ctypes.c_int32), ("n_cut", ctypes.c_int32),
                ("n_prefetched", ctypes.c_int32), ("n_predicted", ctypes.c_int32),
                ("n_hit", ctypes.c_int32), ("part0_us", ctypes.c_float), ("fetch_us", ctypes.c_float)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python quantized_routed_expert_bf16_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.moe_record_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.moe_record_bytes.restype = ctypes.c_uint64
    lib.moe_workspace_bytes.argtypes = [P(MoeDims), ctypes.c_int32]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_workspace_init.argtypes = [vp, ctypes.c_size_t, vp]
    lib.moe_route.argtypes = [vp, ctypes.c_int32, P(MoeRouter), P(MoeShared), P(MoeSlots), vp]
    lib.moe_layer_forward.argtypes = [vp, ctypes.c_int32, P(MoeRouter), P(MoeSlots), P(MoePool),
                                      P(MoeShared), vp, vp]
    lib.moe_layer_forward_noalloc.argtypes = lib.moe_layer_forward.argtypes
    lib.moe_experts_part.argtypes = [vp, ctypes.c_int32, P(MoeDims), P(MoeSlots), ctypes.c_int32,
                                     P(MoePool), P(MoeShared), vp, vp]
    lib.moe_prefill_forward.argtypes = [vp, ctypes.c_int32, P(MoeRouter), P(MoePrefillPlan),
                                        P(MoePool), P(MoeShared), vp, vp]
    lib.moe_workspace_status.argtypes = [vp, ctypes.c_size_t, vp]
    lib.moe_repack.argtypes = [vp, ctypes.c_uint64, vp, vp, ctypes.c_uint64, vp, ctypes.c_int32,
                               ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.moe_set_stage_events.argtypes = [P(ctypes.c_void_p), ctypes.c_int32]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_tier_create.argtypes = [P(MoeTierConfig), P(ctypes.c_void_p)]
    lib.moe_tier_destroy.argtypes = [vp]
    lib.moe_tier_destroy.restype = None
    lib.moe_tier_warm.argtypes = [vp, ctypes.c_int32, vp, ctypes.c_int32, vp]
    lib.moe_tier_layer.argtypes = [vp, ctypes.c_int32, vp, ctypes.c_int32, P(MoeRouter), P(MoeSlots),
                                   P(MoeShared), vp, P(MoeTierPolicy), P(MoeRouter), P(MoeSlots),
                                   P(MoeTierStats), vp, vp]
    lib.moe_tier_join.argtypes = [vp, vp]
    lib.moe_tier_last_error.restype = ctypes.c_char_p
    for name in ("moe_set_stage_events", "moe_workspace_init", "moe_route", "moe_layer_forward",
                 "moe_layer_forward_noalloc", "moe_prefill_forward", "moe_workspace_status",
                 "moe_repack", "moe_experts_part", "moe_tier_create", "moe_tier_warm",
                 "moe_tier_layer", "moe_tier_join"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def last_error() -> str:
    return lib.moe_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise MoeError(rc, last_error())
    return rc


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------ plain calls --

def record_bytes(hidden: int, inter: int, bits: int) -> int:
    return int(lib.moe_record_bytes(hidden, inter, bits))


def workspace_bytes(dims: MoeDims, max_rows: int) -> int:
    return int(lib.moe_workspace_bytes(ctypes.byref(dims), max_rows))


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check(lib.moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def _status_checked(ws_ptr: int, ws_bytes: int, stream) -> None:
    """Synchronise the stream, read and clear the workspace status word and
    raise if the call skipped a record or a bounded wait ran out."""
    st = _check(lib.moe_workspace_status(ws_ptr, ws_bytes, _stream(stream)))
    if st & STATUS_WAIT_RAN_OUT:
        raise MoeError(ELAUNCH, f"status {st:#x}: a bounded wait between blocks ran out "
                                "(another workload held the GPU); the output is not valid")
    if st & STATUS_BAD_RECORD:
        raise MoeError(EINVAL, f"status {st:#x}: a record descriptor outside the pool was skipped")


def route(x, nb: int, router: MoeRouter, shared: MoeShared, slots: MoeSlots, stream=None,
          check: bool = False) -> None:
    """moe_route.  check=True synchronises and raises on a non-zero status."""
    _check(lib.moe_route(_ptr(x), nb, ctypes.byref(router), ctypes.byref(shared),
                         ctypes.byref(slots), _stream(stream)))
    if check:
        _status_checked(slots.ws, slots.ws_bytes, stream)


def layer_forward(x, nb: int, router: MoeRouter, slots: MoeSlots, pool: MoePool,
                  shared: MoeShared, out, stream=None, check: bool = False) -> None:
    """moe_layer_forward.  check=True synchronises and raises on a non-zero
    status (the checked mode for callers that may share the GPU)."""
    _check(lib.moe_layer_forward(_ptr(x), nb, ctypes.byref(router), ctypes.byref(slots),
                                 ctypes.byref(pool), ctypes.byref(shared), _ptr(out),
                                 _stream(stream)))
    if check:
        _status_checked(slots.ws, slots.ws_bytes, stream)


def layer_forward_noalloc(x, nb: int, router: MoeRouter, slots: MoeSlots, pool: MoePool,
                          shared: MoeShared, out, stream=None) -> None:
    """moe_layer_forward_noalloc: slots.ws must be None and slots.ws_bytes 0
    (the library's static scratch is used)."""
    _check(lib.moe_layer_forward_noalloc(_ptr(x), nb, ctypes.byref(router), ctypes.byref(slots),
                                         ctypes.byref(pool), ctypes.byref(shared), _ptr(out),
                                         _stream(stream)))


def experts_part(x, nb: int, dims: MoeDims, slots: MoeSlots, part: int, pool: MoePool,
                 shared: MoeShared, out, stream=None) -> None:
    """moe_experts_part: part 0 (resident slots + shared, overwrites out) or
    part 1 (fetched slots, adds to out) of the table in slots.tab / wmap."""
    _check(lib.moe_experts_part(_ptr(x), nb, ctypes.byref(dims), ctypes.byref(slots), part,
                                ctypes.byref(pool), ctypes.byref(shared), _ptr(out), _stream(stream)))


def repack(src_pool, src_desc, dst_pool, dst_desc, n: int, hidden: int, inter: int,
           status=None, stream=None) -> None:
    """moe_repack: 4-bit records at src_desc[:n] requantized into the widths
    and offsets dst_desc[:n] name (device tensors)."""
    _check(lib.moe_repack(_ptr(src_pool), src_pool.numel(), _ptr(src_desc), _ptr(dst_pool),
                          dst_pool.numel(), _ptr(dst_desc), n, hidden, inter, _ptr(status),
                          _stream(stream)))


def static_scratch_status(stream=None) -> int:
    """Read and clear the status word of the static scratch on the current device."""
    return _check(lib.moe_workspace_status(None, 0, _stream(stream)))


def prefill_forward(x, t: int, router: MoeRouter, plan: MoePrefillPlan, pool: MoePool,
                    shared: MoeShared, out, stream=None, check: bool = False) -> None:
    """moe_prefill_forward.  check=True synchronises and raises on a non-zero status."""
    _check(lib.moe_prefill_forward(_ptr(x), t, ctypes.byref(router), ctypes.byref(plan),
                                   ctypes.byref(pool), ctypes.byref(shared), _ptr(out),
                                   _stream(stream)))
    if check:
        _status_checked(plan.ws, plan.ws_bytes, stream)


def set_stage_events(events) -> None:
    """events: list of raw hipEvent_t handles (ints, or None); [] turns the hook off."""
    arr = (ctypes.c_void_p * max(1, len(events)))(*events)
    _check(lib.moe_set_stage_events(arr, len(events)))


def workspace_status(ws: torch.Tensor, stream=None) -> int:
    return _check(lib.moe_workspace_status(_ptr(ws), ws.numel() * ws.element_size(),
                                           _stream(stream)))


# ------------------------------------------- device buffers (torch plumbing) --

def make_dims(hidden: int, inter: int, n_experts: int, top_k: int) -> MoeDims:
    return MoeDims(hidden, inter, n_experts, top_k)


def make_router(dims: MoeDims, weight: torch.Tensor, rec: torch.Tensor) -> MoeRouter:
    """weight: bf16 [E][H] on the device; rec: int64 [E] descriptors on the device."""
    assert weight.dtype == torch.bfloat16 and weight.is_contiguous()
    assert rec.dtype == torch.int64 and rec.is_contiguous()
    return MoeRouter(dims, weight.data_ptr(), rec.data_ptr())


def make_pool(pool: torch.Tensor) -> MoePool:
    return MoePool(pool.data_ptr(), pool.numel())


def make_shared(gate: torch.Tensor, rec: int) -> MoeShared:
    assert gate.dtype == torch.bfloat16 and gate.is_contiguous()
    return MoeShared(gate.data_ptr(), int(rec))


def slots_without_workspace(slots: MoeSlots) -> MoeSlots:
    """The same result buffers with no workspace (for moe_layer_forward_noalloc)."""
    return MoeSlots(slots.tab, slots.wmap, slots.ids, slots.topk_idx, slots.topk_w,
                    slots.logits, slots.gamma, None, 0)


class DecodeBuffers:
    """Device buffers of moe_slots for up to ``max_nb`` rows."""

    def __init__(self, dims: MoeDims, device="cuda", max_nb: int = MAX_NB):
        E, k = dims.n_experts, dims.top_k
        dev = torch.device(device)
        self.tab = torch.zeros(SLOT_STRIDE, dtype=torch.int64, device=dev)
        self.wmap = torch.zeros(MAX_NB, SLOT_STRIDE, dtype=torch.float32, device=dev)
        self.ids = torch.zeros(SLOT_STRIDE, dtype=torch.int32, device=dev)
        self.topk_idx = torch.zeros(max_nb, k, dtype=torch.int32, device=dev)
        self.topk_w = torch.zeros(max_nb, k, dtype=torch.float32, device=dev)
        self.logits = torch.zeros(max_nb, E, dtype=torch.float64, device=dev)
        self.gamma = torch.zeros(max_nb, dtype=torch.float32, device=dev)
        nbytes = workspace_bytes(dims, max_nb)
        if nbytes == 0:
            raise MoeError(EINVAL, "invalid dims")
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.slots = MoeSlots(self.tab.data_ptr(), self.wmap.data_ptr(), self.ids.data_ptr(),
                              self.topk_idx.data_ptr(), self.topk_w.data_ptr(),
                              self.logits.data_ptr(), self.gamma.data_ptr(),
                              self.ws.data_ptr(), nbytes)


class PrefillBuffers:
    """Device buffers of moe_prefill_plan for up to ``max_rows`` rows."""

    def __init__(self, dims: MoeDims, device="cuda", max_rows: int = MAX_PREFILL_ROWS):
        E, k = dims.n_experts, dims.top_k
        dev = torch.device(device)
        self.topk_idx = torch.zeros(max_rows, k, dtype=torch.int32, device=dev)
        self.topk_w = torch.zeros(max_rows, k, dtype=torch.float32, device=dev)
        self.logits = torch.zeros(max_rows, E, dtype=torch.float64, device=dev)
        self.gamma = torch.zeros(max_rows, dtype=torch.float32, device=dev)
        self.expert_ptr = torch.zeros(E + 1, dtype=torch.int32, device=dev)
        self.entry_row = torch.zeros(max_rows * k, dtype=torch.int32, device=dev)
        self.entry_rank = torch.zeros(max_rows * k, dtype=torch.int32, device=dev)
        nbytes = workspace_bytes(dims, max_rows)
        if nbytes == 0:
            raise MoeError(EINVAL, "invalid dims")
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.plan = MoePrefillPlan(self.topk_idx.data_ptr(), self.topk_w.data_ptr(),
                                   self.logits.data_ptr(), self.gamma.data_ptr(),
                                   self.expert_ptr.data_ptr(), self.entry_row.data_ptr(),
                                   self.entry_rank.data_ptr(), self.ws.data_ptr(), nbytes)


class Tier:
    """A moe_tier over a pinned host tier (torch pin_memory tensor, which
    torch allocates with hipHostMalloc) and a device pool; the binding only
    passes pointers and keeps the tensors alive."""

    def __init__(self, dims: MoeDims, n_layers: int, host_tier: torch.Tensor,
                 host_desc, dev_pool: torch.Tensor, slot_offset: int, slot_stride: int,
                 n_slots: int):
        assert host_tier.is_pinned() and host_tier.dtype == torch.uint8
        import numpy as np
        self._desc = np.ascontiguousarray(np.asarray(host_desc, dtype=np.uint64).reshape(-1))
        self._keep = (host_tier, dev_pool)
        self.cfg = MoeTierConfig(dims, n_layers, host_tier.data_ptr(), host_tier.numel(),
                                 self._desc.ctypes.data, dev_pool.data_ptr(), dev_pool.numel(),
                                 slot_offset, slot_stride, n_slots)
        h = ctypes.c_void_p()
        rc = lib.moe_tier_create(ctypes.byref(self.cfg), ctypes.byref(h))
        if rc:
            raise MoeError(rc, lib.moe_tier_last_error().decode())
        self.handle = h.value
        self.copy_stream = torch.cuda.Stream()

    def _chk(self, rc):
        if rc:
            raise MoeError(rc, lib.moe_tier_last_error().decode())

    def warm(self, layer: int, experts) -> None:
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
        self._chk(lib.moe_tier_warm(self.handle, layer, ids.ctypes.data, ids.size,
                                    self.copy_stream.cuda_stream))
        self.copy_stream.synchronize()

    def layer(self, layer: int, x, nb: int, router: MoeRouter, slots: MoeSlots,
              shared: MoeShared, out, policy: MoeTierPolicy | None = None,
              next_router: MoeRouter | None = None, la_slots: MoeSlots | None = None,
              stream=None) -> dict:
        st = MoeTierStats()
        self._chk(lib.moe_tier_layer(self.handle, layer, _ptr(x), nb, ctypes.byref(router),
                                     ctypes.byref(slots), ctypes.byref(shared), _ptr(out),
                                     ctypes.byref(policy) if policy is not None else None,
                                     ctypes.byref(next_router) if next_router is not None else None,
                                     ctypes.byref(la_slots) if la_slots is not None else None,
                                     ctypes.byref(st), _stream(stream), self.copy_stream.cuda_stream))
        return st.as_dict()

    def join(self, stream=None) -> None:
        self._chk(lib.moe_tier_join(self.handle, _stream(stream)))

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib.moe_tier_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()
