"""GPTQ / AWQ layer quantization on MI355X (gfx950): Python binding of libptq.so.

The compute path is the HIP library behind the C ABI in include/ptq.h; this
package only marshals torch tensors (device memory) and the current stream
into those calls. Importing it loads the library and fails loudly if it has
not been built (``python post_int4_weight_amd/build.py``).
"""
from .api import (PTQError, PTQ_BF16, PTQ_F32, library_path, hessian_workspace_bytes, hessian_accumulate,
                  gptq_factor_workspace_bytes, gptq_inverse_factor, gptq_columns_workspace_bytes,
                  gptq_quantize_columns, gptq_workspace_bytes, gptq_quantize_layer, awq_workspace_bytes,
                  awq_search_alpha, awq_gptq_quantize_layer, gptq_quantize_layer_zp, pack_int4,
                  dequantize_int4, layer_output_error_workspace_bytes, layer_output_error)

__all__ = [
    "PTQError", "PTQ_BF16", "PTQ_F32", "library_path", "hessian_workspace_bytes", "hessian_accumulate",
    "gptq_factor_workspace_bytes", "gptq_inverse_factor", "gptq_columns_workspace_bytes",
    "gptq_quantize_columns", "gptq_workspace_bytes", "gptq_quantize_layer", "awq_workspace_bytes",
    "awq_search_alpha", "awq_gptq_quantize_layer", "gptq_quantize_layer_zp", "pack_int4", "dequantize_int4",
    "layer_output_error_workspace_bytes", "layer_output_error",
]
