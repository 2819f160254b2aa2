"""CPU oracle for 3D-RoPE full spatiotemporal attention and its factorised variant.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's CPU-baseline leg
may import this package.  The library under ``full_spatiotemporal_attention_amd`` never imports,
links or runs anything here, and nothing here imports that library.
"""
from .st_oracle import (  # noqa: F401
    ORACLE_DTYPE,
    attention_dense,
    attention_rows,
    attn_flop_model,
    cross_attention_ref,
    full_attention_ref,
    factorized_ref,
    latent_token_grid,
    merge_partials_ref,
    metric_flops,
    factorized_flops,
    partial_attention_ref,
    qkv_rope_ref,
    window_attention_ref,
    rope_frequencies,
    rope_pair_layout,
    rope3d_ref,
    token_positions,
)
