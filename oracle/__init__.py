"""CPU oracle of the routed-expert MoE layer (test infrastructure only).

Importable only from tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg; the HIP library never imports or calls it.
"""
from .moe_oracle import (  # noqa: F401
    GROUP, SLOT_STRIDE, RESIDENT_ENTRY, UNION_ENTRY, MAX_NB,
    record_layout, unpack_codes, bf16_to_f64, dequant, read_expert,
    router_logits, topk_softmax, route, union_slots, silu, sigmoid,
    expert_mlp, shared_gate, layer_forward, expert_csr, prefill_forward,
    requantize_group_codes, repack_record,
)
