"""Slow, plain float64 CPU oracle for multi-head differential attention.

Test infrastructure only.  The test suite, the smoke check and the CPU-baseline
leg of the benchmark may call it; the product path (the HIP library and its
Python binding) never imports it, and it imports nothing from the product.
"""
from .diffattn_oracle import (  # noqa: F401
    lambda_init,
    lambda_value,
    diff_weights,
    diff_attn_fwd,
    diff_attn_bwd,
    diff_attn_lambda_grad,
    v2_decode,
    v2_prefill_fwd,
    v2_prefill_bwd,
    v2_prefill_fwd_block_sparse,
    v1_decode,
    fp8_quantize_rows,
    fp8_decode,
    diff_attn_fwd_fp8_logits,
    sigmoid,
)
from .brute import brute_diff_attn_fwd, brute_v2_decode, brute_v2_prefill_fwd  # noqa: F401
