"""MI355X (gfx950) QLoRA hot path: NF4 blockwise encoder, double quantization
and the quantized LoRA linear layer (forward and backward) as hand-written HIP
kernels behind the C ABI in include/qlora.h.  This package is the thin ctypes
binding; torch provides device memory and streams only."""
from ._lib import (  # noqa: F401
    QloraError, lib, EXPORTS,
    nf4_quantize, nf4_quantize_dq, nf4_double_quant, nf4_dequantize,
    qlora_linear_fwd_workspace, qlora_linear_fwd,
    qlora_linear_bwd_workspace, qlora_linear_bwd,
    qlora_nf4_levels, ql_status_string,
    qlora_lora_down, qlora_linear_fwd_t, qlora_lora_grad_in, qlora_linear_dx,
    qlora_merge,
    CODEBOOKS, SCALE_CODES, q4_quantize, q4_double_quant, q4_dequantize, q4_levels,
    qlora_group_fwd, qlora_group_bwd, qlora_adamw_step, qlora_linear_fwd_noalloc, NOALLOC_SCRATCH_BYTES,
    lora_linear_fwd, lora_linear_bwd, lora_linear_fwd_t, lora_linear_dx,
)
