"""MI355X-native Kimi Delta Attention (KDA): chunked forward/backward, decode step,
packed-document metadata.  The compute runs in libkda.so (hand-written HIP for
gfx950); this package only marshals torch tensors into its C ABI (include/kda.h).
"""
from .binding import (CHUNK, F_BETA_LOGITS, F_GATE_IN_KERNEL, F_QK_L2NORM, KdaError, bwd,
                      check_cu_seqlens, fwd, load_library, max_chunks, plan_varlen, step,
                      timing_collect, timing_enable, workspace_bytes)

__all__ = ["CHUNK", "F_BETA_LOGITS", "F_GATE_IN_KERNEL", "F_QK_L2NORM", "KdaError", "bwd",
           "check_cu_seqlens", "fwd", "load_library", "max_chunks", "plan_varlen", "step",
           "timing_collect", "timing_enable", "workspace_bytes"]
