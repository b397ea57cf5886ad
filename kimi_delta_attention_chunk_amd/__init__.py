"""MI355X-native Kimi Delta Attention (KDA): chunked forward/backward, decode step,
packed-document metadata, and the short convolution and gated output norm next
to it in the layer.  The compute runs in libkda.so (hand-written HIP for
gfx950); this package only marshals torch tensors into its C ABI (include/kda.h).
"""
from .binding import (CHUNK, F_BETA_LOGITS, F_GATE_IN_KERNEL, F_QK_L2NORM, RMS_EPS, KdaError, bwd,
                      check_cu_seqlens, conv_bwd, conv_fwd, fwd, fwd_noalloc, gnorm_bwd, gnorm_fwd, load_library,
                      max_chunks, plan_varlen, segment_maps, state_scan, step, timing_collect, timing_enable,
                      workspace_bytes)

__all__ = ["CHUNK", "F_BETA_LOGITS", "F_GATE_IN_KERNEL", "F_QK_L2NORM", "RMS_EPS", "KdaError", "bwd",
           "check_cu_seqlens", "conv_bwd", "conv_fwd", "fwd", "fwd_noalloc", "gnorm_bwd", "gnorm_fwd", "load_library",
           "max_chunks", "plan_varlen", "segment_maps", "state_scan", "step", "timing_collect", "timing_enable",
           "workspace_bytes"]
