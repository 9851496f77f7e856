"""CPU fp64 oracle -- test infrastructure only (see gguf_oracle's header).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the product path never does.
"""

from .gguf_oracle import *  # noqa: F401,F403
from .gguf_oracle import (  # noqa: F401
    IQ4_GRID,
    IQ4_XS_BLOCK_BYTES,
    IQ4_XS_BLOCK_WEIGHTS,
    Q4_K_BLOCK_BYTES,
    Q4_K_BLOCK_WEIGHTS,
    Q5_K_BLOCK_BYTES,
    Q8_0_BLOCK_BYTES,
    Q8_0_BLOCK_WEIGHTS,
    bf16_bits_to_f64,
    dequant_iq4_xs,
    dequant_q4_k,
    dequant_q4_k_bf16_bits,
    dequant_q4_k_f32,
    dequant_q5_k,
    dequant_q5_k_f32,
    dequant_q8_0,
    dequant_q8_0_f32,
    expert_matrix,
    floored_rel_err,
    fp16_bits_to_f64,
    frobenius_rel_err,
    gather_pairs,
    gemv,
    iq4_xs_fields,
    moe_iq4_xs,
    moe_q4_k,
    prefill_q4_k,
    q4_k_fields,
    q5_k_fields,
    q8_0_fields,
    qmv_iq4_xs,
    qmv_q4_k,
    qmv_q5_k,
    qmv_q8_0,
    round_f32_to_bf16_bits,
    round_to_f32,
    route_top_k,
    silu,
)
