"""CPU oracle of the fused MoE layer -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The product path never does.
"""

from .moe_oracle import (  # noqa: F401
    align,
    align_capacity,
    decode_bf16,
    decode_e4m3fn,
    decode_weights,
    expert_ffn,
    gate_weights,
    moe_forward,
    mx_dequantize,
    mx_quantize,
    router_logits,
    select_topk,
    silu,
)
