"""MI355X-native QLoRA NF4 linear layer: a C-ABI HIP library (libqlora.so,
include/qlora.h) and its thin Python binding."""

from .qlora import (  # noqa: F401
    QLoRAError, QTYPES, adamw_step, adamw_workspace_bytes, device_status, double_quant, dequantize_nf4, lib, linear_bwd, linear_bwd_workspace_bytes,
    linear_bwd_grouped, linear_fwd, linear_fwd_grouped, linear_fwd_noalloc, linear_fwd_workspace_bytes, load_4bit, load_4bit_info, nf4_codebook, quantize_dq,
    quantize_nf4, save_4bit, table_4bit,
)
