"""fp64 CPU oracle for exact attention (forward, lse, backward) and the streaming row
operators (softmax, LayerNorm) -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP path.
"""
from .attention import (  # noqa: F401
    allowed_mask,
    attention_fp64,
    attention_full_fp64,
    attention_lse_fp64,
    attention_bwd_fp64,
    attention_bwd_rows_fp64,
    attention_bwd_sampled_fp64,
    attention_rows_fp64,
    decode_bf16_bits,
    decode_e4m3_bits,
    attention_fp8_fp64,
    effective_kv_len,
    to_fp64,
)
from .rows import layernorm_rows_fp64, softmax_rows_fp64  # noqa: F401
