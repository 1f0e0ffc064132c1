"""MI355X (gfx950) QLoRA quantized linear layer.

NF4 quantisation (blocks of 64 or 128) with 8-bit double quantisation of the
block constants, and the layer y = x W^T + (alpha/r) (x A^T) B^T with its
backward (dx, dA, dB) in bf16, fp16 or fp32 compute, all in hand-written HIP
kernels behind the C ABI of include/qlora.h.  This package is the thin
Python binding.
"""
from .binding import (DQ_BLOCK, NF4_BLOCK, QL_OP_BWD, QL_OP_FWD, QL_OP_QUANTIZE, NF4Weight,
                      QLoRAArgumentError, QLoRAError, adamw_step, dropout_mask, lib,
                      nf4_dequantize, nf4_quantize, nf4_quantize_many,
                      nf4_sizes, qlora_linear_bwd, qlora_linear_bwd_dropout, qlora_linear_fwd,
                      qlora_linear_fwd_dropout, qlora_linear_fwd_u, quantize_many_workspace_bytes,
                      workspace, workspace_bytes)

__all__ = ["NF4Weight", "nf4_quantize", "nf4_quantize_many", "nf4_dequantize",
           "qlora_linear_fwd", "qlora_linear_fwd_u", "qlora_linear_bwd",
           "qlora_linear_fwd_dropout", "qlora_linear_bwd_dropout", "dropout_mask", "adamw_step",
           "nf4_sizes", "workspace", "workspace_bytes", "quantize_many_workspace_bytes", "lib",
           "QLoRAError", "QLoRAArgumentError", "NF4_BLOCK", "DQ_BLOCK", "QL_OP_QUANTIZE",
           "QL_OP_FWD", "QL_OP_BWD"]
