"""CPU oracle for the QLoRA hot path (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP library and its binding never do.
"""
from .qlora_oracle import (  # noqa: F401
    BLOCK, GROUP,
    fp32, bf16_round, bf16_bits, bf16_value,
    nf4_levels, nf4_levels_f64, nf4_midpoints, nf4_nearest_code,
    e4m3fn_decode, e4m3fn_encode,
    nf4_quantize, unpack_codes, nf4_double_quant, block_scales, nf4_dequantize,
    dequantize_blocks,
    qlora_forward, qlora_backward, qlora_merge, bits_per_weight,
)
from . import variants  # noqa: F401,E402  (code-book and second-level-scale variants)
from . import block  # noqa: F401,E402  (stacked linears and the adapter-only optimizer step)
