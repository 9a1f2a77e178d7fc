"""QuantSparse attention hot path for MI355X (gfx950): int8 per-block Q/K
quantisation, pooled top-k + band block selection, block-sparse flash
attention on MFMA, and the second-order residual cache of sparse steps.

The compute lives in libqsa.so (HIP kernels behind a C ABI, include/qsa.h);
this package only binds it.
"""
from .binding import (QSAError, load_library, qsa_apply_residual, qsa_full_attn_residual,
                      qsa_quantize, qsa_select_blocks, qsa_sparse_attn, default_sm_scale)
from .layer import QSAConfig, QuantSparseAttention

__all__ = ["QSAError", "load_library", "qsa_quantize", "qsa_select_blocks", "qsa_sparse_attn",
           "qsa_full_attn_residual", "qsa_apply_residual", "default_sm_scale", "QSAConfig",
           "QuantSparseAttention"]
