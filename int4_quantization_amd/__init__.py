"""libdquant for MI355X (gfx950): per-token dynamic quantization
(DynamicQuantV2), its AdaLayerNorm fusion, AntiQuantize, mx block
quantization (e8m0 scales per 32 elements), and the weight-quantized
matmul (int8 / int4 weights dequantized into the matrix cores).

The compute runs in hand-written HIP kernels inside ``libdquant.so``, reached
through the C ABI declared in ``include/dquant.h``.  This package is the thin
ctypes binding over that library (``dquant``) plus the seeded synthetic
input generators (``synth``).  There is no CPU fallback: calling an op
without the built library raises.
"""
from .dquant import (  # noqa: F401
    DquantError,
    ada_layernorm_quant,
    antiquantize,
    dq_ada_layernorm_quant,
    dq_ada_layernorm_quant_get_workspace_size,
    dq_antiquantize,
    dq_antiquantize_get_workspace_size,
    dq_copy_probe,
    dq_dynamic_quant,
    dq_dynamic_quant_get_workspace_size,
    dq_executor_destroy,
    dq_get_last_error,
    dq_mx_quantize,
    dq_mx_quantize_get_workspace_size,
    dq_weight_quant_matmul,
    dq_weight_quant_matmul_get_workspace_size,
    dynamic_quant,
    library,
    library_path,
    mx_quantize,
    mx_scale_shape,
    weight_quant_matmul,
)
