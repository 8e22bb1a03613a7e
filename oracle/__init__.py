"""Oracle package: the fp64 CPU definition of the H3 per-rank path.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .h3_oracle import (  # noqa: F401
    bf16_to_f64,
    f64_to_bf16_bits,
    rope_tables,
    rms_norm,
    rope_rotate,
    qknorm_rope,
    attention_head,
    attention,
    attention_lse_head,
    merge_partials,
    qkv_project,
    split_heads,
    qkv_proj_qknorm_rope,
    e4m3_to_f64,
    qkv_proj_fp8_qknorm_rope,
)
