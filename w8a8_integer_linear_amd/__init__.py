"""INT8 W8A8 linear layer for quantized training on AMD MI355X (gfx950).

The compute path lives in libqlin.so (hand-written HIP kernels behind the C ABI
of include/qlin.h); this package only binds it for torch tensors.
"""
from ._native import (  # noqa: F401
    MAX_CONTRACTION, MFMA_CEILING_FRAG_BYTES, NOALLOC_SCRATCH_BYTES, QLIN_BF16, QLIN_F32,
    QLIN_OP_DW, QLIN_OP_DX, QLIN_OP_FWD, QlinError, SIGNATURES, lib, qlin_adamw_requant,
    qlin_bwd_dw, qlin_bwd_dx, qlin_dequantize_weight, qlin_fwd, qlin_gemm_s32, qlin_hadamard,
    qlin_mfma_ceiling, qlin_product_noalloc, qlin_product_ws, qlin_product_ws_bytes,
    qlin_quantize_cols, qlin_quantize_grad, qlin_quantize_rows, qlin_sgd_requant,
    qlin_stream_copy, qlin_wn_init, qlin_wn_sgd_requant)
from .layer import LinearW8A8Training  # noqa: F401
