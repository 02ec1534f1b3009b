"""fp64 CPU oracle for the online-softmax attention path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package. The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
never imports the product path: the two share no code. The only module both
sides use is ``workloads`` (seeded input draws, no arithmetic of the method).
"""
from .oracle import (  # noqa: F401
    attention,
    attention_score_mod,
    bf16_bits_to_f64,
    decode_gqa,
    decode_splitkv_partials,
    element_mask,
    layernorm_rows,
    logsumexp_rows,
    moe_route,
    lse_merge,
    online_attention,
    online_softmax_stats,
    round_to_bf16,
    softmax_rows,
    split_ranges,
)
