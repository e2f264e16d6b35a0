"""MI355X-native QLoRA NF4 linear layer: a C-ABI HIP library (libqlora.so,
include/qlora.h) and its thin Python binding."""

from .qlora import (  # noqa: F401
    QLoRAError, double_quant, dequantize_nf4, lib, linear_bwd, linear_bwd_workspace_bytes, linear_fwd,
    linear_fwd_workspace_bytes, nf4_codebook, quantize_nf4,
)
