"""MI355X-native Kimi Delta Attention (KDA): chunkwise prefill, its training backward and
recurrent decode.

The operator lives in libkda.so (hand-written HIP kernels for gfx950, C ABI in
include/kda.h); this package is its thin Python binding.
"""
from ._binding import (KDA_DTYPE_BF16, KDA_DTYPE_F32, LIB_PATH, OPT_BETA_LOGITS,
                       OPT_GATE_LOGITS, OPT_L2NORM_QK, OPT_SCALAR_GATE, KdaError,
                       bwd_workspace_size, chunk_bwd, chunk_fwd, chunk_fwd_noalloc,
                       chunk_fwd_scan, ckpt_empty, ckpt_interval, decode_step,
                       declared_functions, lib, workspace_size)

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_scan", "chunk_bwd", "decode_step",
           "workspace_size", "bwd_workspace_size", "ckpt_interval", "ckpt_empty", "KdaError", "lib", "LIB_PATH",
           "declared_functions", "KDA_DTYPE_BF16", "KDA_DTYPE_F32", "OPT_SCALAR_GATE",
           "OPT_GATE_LOGITS", "OPT_BETA_LOGITS", "OPT_L2NORM_QK"]
