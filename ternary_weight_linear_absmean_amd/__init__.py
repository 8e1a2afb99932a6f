"""libbitlinear: BitLinear W1.58A8 (BitNet b1.58) on AMD Instinct MI355X.

Python names match the C entry points of include/bitlinear.h; see _native.py.
Importing the package does not load the native library; the first call (or
``load()``) does, and raises if it has not been built.
"""
from ._native import (  # noqa: F401
    BL_BF16, BL_F32, BL_MAX_JOBS, BL_MAX_K, BL_OP_BACKWARD_INPUT, BL_OP_BACKWARD_WEIGHT,
    BL_OP_DECODE_STACK, BL_OP_FFN_RELU2, BL_OP_QUANT_WEIGHT, BL_STACK_AUTO, BL_STACK_LAUNCHES,
    BL_STACK_PERSISTENT, EXPORTS, LAYER_GAMMAS, LAYER_WEIGHTS, LIB_PATH, BitLinearError,
    GemvJob, Layer, StackDims, bitlinear_backward_input, bitlinear_backward_weight,
    bitlinear_a4, bitlinear_decode_stack, bitlinear_decode_stack_status, bitlinear_ffn_relu2, bitlinear_gemm, bitlinear_gemv,
    bitlinear_gemv_fused, bitlinear_gemv_t5, bitlinear_repack_t5, load, quant_act_absmax_i4,
    quant_act_absmax_i8,
    quant_weight_absmean_pack, quant_weight_absmean_pack_noalloc, t5_row_bytes, workspace_bytes,
)
