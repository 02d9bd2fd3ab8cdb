"""MI355X-native SageSLA attention, forward and backward (sparse-linear attention on INT8
SageAttention).

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI of
``libsla.so`` (include/sla.h).  Import is cheap; the library is loaded on the
first call and a missing build raises instead of falling back.
"""
from ._lib import (  # noqa: F401
    BLOCK, HEAD_DIM, OP_ATTENTION, OP_ATTENTION_BWD, OP_QUANTIZE, OP_SELECT, PHI, SLAAttention,
    SLAError, attention, attention_bwd, attention_noalloc, attention_train, block_select, debug_qk_i32, fused_norm_i8, load, n_blocks,
    quantize_qk, rowquant_i8, topk_count, train_residual_bytes, w8a8_linear, workspace_bytes,
    workspace_size)

__version__ = "0.1.0"
