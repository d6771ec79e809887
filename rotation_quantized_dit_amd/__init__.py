"""MI355X-native ConvRot int8 quantized linear (MiniMax H3 DiT projections).

A group-wise Hadamard-256 rotation spreads activation outliers, activations are
quantized to int8 per token and weights per row, the product is an int8 x int8
-> int32 contraction on CDNA4 MFMA, and the result is rescaled to bf16 (with
an optional fused SwiGLU).  The work runs in hand-written HIP kernels for
gfx950 behind the C ABI of include/convrot.h; this package is its Python
binding (torch provides device memory and the stream).
"""
from ._lib import (  # noqa: F401
    ATTN_HEAD_DIM,
    GROUP,
    MAX_K,
    ConvRotError,
    attention,
    attention_prep,
    attention_prepared,
    attention_workspace,
    dequantize_weight,
    gemm_dequant,
    gemm_s32,
    gemm_swiglu,
    NOALLOC_SCRATCH_BYTES,
    linear,
    linear_noalloc,
    linear_swiglu,
    lora_add,
    load_library,
    merge_lora,
    mx_gemm,
    mx_linear,
    mx_quantize_act,
    mx_quantize_weight,
    mx_workspace_bytes,
    quantize_weight,
    rotate_quant_act,
    status_string,
    swiglu_rotate_quant_act,
    workspace_bytes,
)
