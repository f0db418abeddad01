"""fp64 CPU oracle for GPTQ / AWQ layer quantization — TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. The HIP library never does, and the two share no code;
the seeded generators in ``inputs/`` are the only common dependency.
"""
from .gptq import (qmax, hessian_nbytes, proxy_hessian, damped, act_order_permutation,
                   inverse_upper_factor, gptq_columns, rtn, dequantize, gptq_layer,
                   output_error, output_energy, quadratic_error)
from .awq import channel_mean_abs, awq_quantize, awq_search, awq_gptq_layer
from .pack import pack_int4, unpack_int4, dequantize_packed
from .zero_point import (group_params as zp_group_params, gptq_columns as zp_gptq_columns, rtn as zp_rtn,
                         dequantize as zp_dequantize, gptq_layer as zp_gptq_layer)

__all__ = [
    "qmax", "hessian_nbytes", "proxy_hessian", "damped", "act_order_permutation",
    "inverse_upper_factor", "gptq_columns", "rtn", "dequantize", "gptq_layer",
    "output_error", "output_energy", "quadratic_error",
    "channel_mean_abs", "awq_quantize", "awq_search", "awq_gptq_layer",
    "pack_int4", "unpack_int4", "dequantize_packed",
    "zp_group_params", "zp_gptq_columns", "zp_rtn", "zp_dequantize", "zp_gptq_layer",
]
