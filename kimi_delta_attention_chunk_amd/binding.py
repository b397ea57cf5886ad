"""Thin ctypes binding of libkda.so (include/kda.h).

Argument marshalling only: every step of the operator runs in the HIP
kernels of libkda.so.  PyTorch provides device memory and the current
stream.  Tensors must already be contiguous, on the GPU and of the right
dtype: the wrappers raise ValueError instead of copying (the Primus guide,
Troubleshooting, warns that silent copies double activation memory).
If the library is missing every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_BF16, KDA_FP32 = 0, 1
F_QK_L2NORM, F_GATE_IN_KERNEL, F_BETA_LOGITS, F_SAVE_FOR_BWD, F_FWD_SAVED, F_DH0_ONLY = 1, 2, 4, 8, 16, 32
CHUNK = 64

EXPORTS = ["kda_max_chunks", "kda_plan_varlen", "kda_check_cu_seqlens", "kda_fwd_workspace",
           "kda_bwd_workspace", "kda_fwd", "kda_bwd", "kda_step", "kda_status_str",
           "kda_last_error", "kda_timing_enable", "kda_timing_collect", "kda_timing_count",
           "kda_timing_get", "kda_conv_fwd", "kda_conv_bwd_workspace", "kda_conv_bwd", "kda_gnorm_fwd",
           "kda_gnorm_bwd_workspace", "kda_gnorm_bwd", "kda_segment_maps", "kda_state_scan",
           "kda_fwd_noalloc", "kda_debug_ws_layout"]
CONV_SILU = 1
RMS_EPS = 1e-6


class KdaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("N", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


class KdaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("kda status %d: %s" % (status, msg))
        self.status = status


_lib = None


def load_library():
    """Load libkda.so (built in-tree by kimi_delta_attention_chunk_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkda.so is not built (%s); run __graft_entry__.build() or "
                           "python -m kimi_delta_attention_chunk_amd.build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, f32, u32 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float,
                             ctypes.c_uint32)
    dp = ctypes.POINTER(KdaDesc)
    lib.kda_max_chunks.argtypes = [i32, i32, i32]
    lib.kda_max_chunks.restype = i32
    lib.kda_plan_varlen.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.kda_plan_varlen.restype = ctypes.c_int
    lib.kda_check_cu_seqlens.argtypes = [vp, i32, i32, vp]
    lib.kda_check_cu_seqlens.restype = ctypes.c_int
    lib.kda_fwd_workspace.argtypes = [dp]
    lib.kda_fwd_workspace.restype = sz
    lib.kda_bwd_workspace.argtypes = [dp]
    lib.kda_bwd_workspace.restype = sz
    lib.kda_fwd.argtypes = [dp] + [vp] * 14 + [sz, vp]
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_debug_ws_layout.argtypes = [dp, ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.c_int]
    lib.kda_debug_ws_layout.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = [dp] + [vp] * 14
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_bwd.argtypes = [dp] + [vp] * 22 + [sz, vp]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_step.argtypes = [i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, f32, u32] + [vp] * 10
    lib.kda_step.restype = ctypes.c_int
    lib.kda_status_str.argtypes = [ctypes.c_int]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_timing_enable.argtypes = [ctypes.c_int]
    lib.kda_timing_enable.restype = ctypes.c_int
    lib.kda_timing_collect.argtypes = []
    lib.kda_timing_collect.restype = ctypes.c_int
    lib.kda_timing_count.argtypes = []
    lib.kda_timing_count.restype = ctypes.c_int
    lib.kda_timing_get.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                   ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    lib.kda_timing_get.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.kda_conv_fwd.argtypes = [i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, u32, vp, vp, vp, vp, i32, vp, vp]
    lib.kda_conv_fwd.restype = ctypes.c_int
    lib.kda_conv_bwd_workspace.argtypes = [i32, i32, i32, i32]
    lib.kda_conv_bwd_workspace.restype = sz
    lib.kda_conv_bwd.argtypes = ([i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, u32, vp, vp, vp, vp, i32]
                                 + [vp] * 5 + [sz, vp])
    lib.kda_conv_bwd.restype = ctypes.c_int
    lib.kda_gnorm_fwd.argtypes = [i64, i32, ctypes.c_int, ctypes.c_int, f32, vp, vp, vp, vp, vp]
    lib.kda_gnorm_fwd.restype = ctypes.c_int
    lib.kda_gnorm_bwd_workspace.argtypes = [i64, i32]
    lib.kda_gnorm_bwd_workspace.restype = sz
    lib.kda_gnorm_bwd.argtypes = [i64, i32, ctypes.c_int, ctypes.c_int, f32] + [vp] * 8 + [sz, vp]
    lib.kda_gnorm_bwd.restype = ctypes.c_int
    lib.kda_segment_maps.argtypes = [dp] + [vp] * 12 + [sz, vp]
    lib.kda_segment_maps.restype = ctypes.c_int
    lib.kda_state_scan.argtypes = [i32, i32, i32, i32, i32] + [vp] * 6
    lib.kda_state_scan.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc):
    if rc != KDA_OK:
        lib = load_library()
        raise KdaError(rc, lib.kda_last_error().decode())


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KDA_BF16
    if t == torch.float32:
        return KDA_FP32
    raise ValueError("unsupported dtype %s (bfloat16 or float32)" % t)


def _req(x, name, dtype=None, shape=None, device=None, optional=False):
    if x is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(x, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if not x.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if device is not None and x.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, x.device, device))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous (call .contiguous() explicitly)" % name)
    if dtype is not None and x.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError("%s has dtype %s, expected %s" % (name, x.dtype, dtype))
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), tuple(shape)))
    return x


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def max_chunks(T: int, N: int, chunk: int = CHUNK) -> int:
    return int(load_library().kda_max_chunks(T, N, chunk))


def plan_varlen(cu_seqlens: torch.Tensor, T: int, chunk: int = CHUNK):
    """Device chunk tables for a packed row: (chunk_indices [M,2], chunk_offsets [N+1])."""
    lib = load_library()
    _req(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.numel() - 1
    M = max_chunks(T, N, chunk)
    dev = cu_seqlens.device
    idx = torch.empty((max(M, 1), 2), dtype=torch.int32, device=dev)
    off = torch.empty((N + 1,), dtype=torch.int32, device=dev)
    _check(lib.kda_plan_varlen(_ptr(cu_seqlens), N, T, chunk, _ptr(idx), _ptr(off), _stream(dev)))
    return idx[:M], off


def check_cu_seqlens(cu_seqlens: torch.Tensor, T: int):
    """Synchronising debug check of cu_seqlens (raises KdaError if malformed)."""
    lib = load_library()
    _req(cu_seqlens, "cu_seqlens", torch.int32)
    _check(lib.kda_check_cu_seqlens(_ptr(cu_seqlens), cu_seqlens.numel() - 1, T,
                                    _stream(cu_seqlens.device)))


def _desc(q, v, N, scale, flags, out_dtype):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    return KdaDesc(B, T, H, dk, dv, N, CHUNK, _dt(q.dtype), _dt(out_dtype), float(scale), int(flags))


def _flags(l2norm_qk, gate_in_kernel, beta_logits):
    return (F_QK_L2NORM if l2norm_qk else 0) | (F_GATE_IN_KERNEL if gate_in_kernel else 0) | (
        F_BETA_LOGITS if beta_logits else 0)


def _check_inputs(q, k, v, g, beta, h0, cu_seqlens, plan, A_log, dt_bias, gate_in_kernel):
    _req(q, "q", (torch.bfloat16, torch.float32))
    dev = q.device
    B, T, H, dk = q.shape
    _req(k, "k", q.dtype, q.shape, dev)
    if v.dim() != 4 or tuple(v.shape[:3]) != (B, T, H):
        raise ValueError("v must be [B,T,H,dv] matching q")
    _req(v, "v", q.dtype, None, dev)
    dv = v.shape[-1]
    _req(g, "g", torch.float32, q.shape, dev)
    _req(beta, "beta", torch.float32, (B, T, H), dev)
    if cu_seqlens is not None:
        _req(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        if plan is None:
            raise ValueError("packed rows need plan=plan_varlen(cu_seqlens, T)")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    _req(h0, "h0", torch.float32, (N, H, dk, dv), dev, optional=True)
    if gate_in_kernel:
        _req(A_log, "A_log", torch.float32, (H,), dev)
        _req(dt_bias, "dt_bias", torch.float32, (H, dk), dev)
    return B, T, H, dk, dv, N


def fwd(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, plan=None, *, A_log=None,
        dt_bias=None, l2norm_qk=False, gate_in_kernel=False, beta_logits=False, out_dtype=None,
        output_final_state=True, workspace=None, save_for_bwd=False, fwd_saved=False):
    """kda_fwd.  Returns (o [B,T,H,dv], hT [N,H,dk,dv] or None).

    With save_for_bwd the workspace (which must then be sized for the backward)
    keeps what kda_bwd(..., fwd_saved=True, workspace=same) needs.  With fwd_saved
    the workspace already holds such a forward of the same inputs: only the state
    pass runs again, from this call's h0.
    """
    lib = load_library()
    B, T, H, dk, dv, N = _check_inputs(q, k, v, g, beta, h0, cu_seqlens, plan, A_log, dt_bias,
                                       gate_in_kernel)
    out_dtype = out_dtype or q.dtype
    flags = (_flags(l2norm_qk, gate_in_kernel, beta_logits) | (F_SAVE_FOR_BWD if save_for_bwd else 0)
             | (F_FWD_SAVED if fwd_saved else 0))
    if fwd_saved and workspace is None:
        raise ValueError("fwd_saved needs the saved forward's workspace")
    desc = _desc(q, v, N, scale, flags, out_dtype)
    dev = q.device
    o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    need = (lib.kda_bwd_workspace if (save_for_bwd or fwd_saved) else lib.kda_fwd_workspace)(ctypes.byref(desc))
    if need == 0:
        _check(KDA_ERR_INVALID)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    idx, off = plan if plan is not None else (None, None)
    _check(lib.kda_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                       _ptr(A_log), _ptr(dt_bias), _ptr(h0), _ptr(cu_seqlens), _ptr(idx), _ptr(off),
                       _ptr(o), _ptr(hT), _ptr(ws), ws.numel(), _stream(dev)))
    return o, hT


def fwd_noalloc(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, plan=None, *, A_log=None,
                dt_bias=None, l2norm_qk=False, gate_in_kernel=False, beta_logits=False, out_dtype=None,
                o=None, hT=None):
    """kda_fwd_noalloc: the forward on the library's own fixed scratch (no workspace).
    Writes into `o` / `hT` when given (nothing is allocated then), else into new tensors.
    Returns (o, hT)."""
    lib = load_library()
    B, T, H, dk, dv, N = _check_inputs(q, k, v, g, beta, h0, cu_seqlens, plan, A_log, dt_bias,
                                       gate_in_kernel)
    out_dtype = out_dtype or q.dtype
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    _req(o, "o", out_dtype, (B, T, H, dv), dev)
    _req(hT, "hT", torch.float32, (N, H, dk, dv), dev, optional=True)
    desc = _desc(q, v, N, scale, _flags(l2norm_qk, gate_in_kernel, beta_logits), out_dtype)
    idx, off = plan if plan is not None else (None, None)
    _check(lib.kda_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(A_log), _ptr(dt_bias), _ptr(h0), _ptr(cu_seqlens), _ptr(idx),
                               _ptr(off), _ptr(o), _ptr(hT), _stream(dev)))
    return o, hT


def bwd(q, k, v, g, beta, scale, d_o, h0=None, dhT=None, cu_seqlens=None, plan=None, *,
        A_log=None, dt_bias=None, l2norm_qk=False, gate_in_kernel=False, beta_logits=False,
        out_dtype=None, need_dh0=True, workspace=None, fwd_saved=False, dh0_only=False):
    """kda_bwd.  Returns dict dq, dk, dv, dg, dbeta, dh0 (and dA_log, ddt_bias with the gate).

    dh0_only: only the reverse state pass runs; the result holds dh0 alone.
    fwd_saved: `workspace` holds a kda_fwd(..., save_for_bwd=True) of the same
    inputs, so the forward is not recomputed.
    """
    lib = load_library()
    B, T, H, dk, dv, N = _check_inputs(q, k, v, g, beta, h0, cu_seqlens, plan, A_log, dt_bias,
                                       gate_in_kernel)
    dev = q.device
    _req(d_o, "d_o", q.dtype, (B, T, H, dv), dev)
    _req(dhT, "dhT", torch.float32, (N, H, dk, dv), dev, optional=True)
    out_dtype = out_dtype or q.dtype
    flags = (_flags(l2norm_qk, gate_in_kernel, beta_logits) | (F_FWD_SAVED if fwd_saved else 0)
             | (F_DH0_ONLY if dh0_only else 0))
    if fwd_saved and workspace is None:
        raise ValueError("fwd_saved needs the forward's workspace")
    desc = _desc(q, v, N, scale, flags, out_dtype)
    if dh0_only:
        out = dict(dq=None, dk=None, dv=None, dg=None, dbeta=None,
                   dh0=torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev))
    else:
        out = dict(
            dq=torch.empty((B, T, H, dk), dtype=out_dtype, device=dev),
            dk=torch.empty((B, T, H, dk), dtype=out_dtype, device=dev),
            dv=torch.empty((B, T, H, dv), dtype=out_dtype, device=dev),
            dg=torch.empty((B, T, H, dk), dtype=torch.float32, device=dev),
            dbeta=torch.empty((B, T, H), dtype=torch.float32, device=dev),
            dh0=torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if need_dh0 else None,
        )
    if gate_in_kernel and not dh0_only:
        out["dA_log"] = torch.empty((H,), dtype=torch.float32, device=dev)
        out["ddt_bias"] = torch.empty((H, dk), dtype=torch.float32, device=dev)
    need = lib.kda_bwd_workspace(ctypes.byref(desc))
    if need == 0:
        _check(KDA_ERR_INVALID)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    idx, off = plan if plan is not None else (None, None)
    _check(lib.kda_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                       _ptr(A_log), _ptr(dt_bias), _ptr(h0), _ptr(cu_seqlens), _ptr(idx), _ptr(off),
                       _ptr(d_o), _ptr(dhT), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                       _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]),
                       _ptr(out.get("dA_log")), _ptr(out.get("ddt_bias")), _ptr(ws), ws.numel(),
                       _stream(dev)))
    return out


def workspace_arrays(q_shape, dv, N, backward, dtype=torch.bfloat16):
    """kda_debug_ws_layout: [(name, byte offset, byte size)] of the workspace arrays, in order."""
    lib = load_library()
    B, T, H, dk = q_shape
    desc = KdaDesc(B, T, H, dk, dv, N, CHUNK, _dt(dtype), _dt(dtype), 1.0, 0)
    n = lib.kda_debug_ws_layout(ctypes.byref(desc), int(backward), None, None, None, 0)
    if n < 0:
        _check(KDA_ERR_INVALID)
    names = (ctypes.c_char_p * n)()
    offs = (ctypes.c_size_t * n)()
    nbs = (ctypes.c_size_t * n)()
    lib.kda_debug_ws_layout(ctypes.byref(desc), int(backward), names, offs, nbs, n)
    return [(names[i].decode(), int(offs[i]), int(nbs[i])) for i in range(n)]


def workspace_bytes(q_shape, dv, N, backward, dtype=torch.bfloat16, flags=0):
    lib = load_library()
    B, T, H, dk = q_shape
    desc = KdaDesc(B, T, H, dk, dv, N, CHUNK, _dt(dtype), _dt(dtype), 1.0, flags)
    fn = lib.kda_bwd_workspace if backward else lib.kda_fwd_workspace
    return int(fn(ctypes.byref(desc)))


def step(q, k, v, g, beta, h, scale, *, A_log=None, dt_bias=None, l2norm_qk=False,
         gate_in_kernel=False, beta_logits=False, out_dtype=None, out=None):
    """kda_step: one decode token for B sequences; updates h [B,H,dk,dv] in place, returns o."""
    lib = load_library()
    _req(q, "q", (torch.bfloat16, torch.float32))
    dev = q.device
    B, H, dk = q.shape
    _req(k, "k", q.dtype, q.shape, dev)
    _req(v, "v", q.dtype, None, dev)
    if v.dim() != 3 or tuple(v.shape[:2]) != (B, H):
        raise ValueError("v must be [B,H,dv]")
    dv = v.shape[-1]
    _req(g, "g", torch.float32, (B, H, dk), dev)
    _req(beta, "beta", torch.float32, (B, H), dev)
    _req(h, "h", torch.float32, (B, H, dk, dv), dev)
    if gate_in_kernel:
        _req(A_log, "A_log", torch.float32, (H,), dev)
        _req(dt_bias, "dt_bias", torch.float32, (H, dk), dev)
    out_dtype = out_dtype or q.dtype
    o = out if out is not None else torch.empty((B, H, dv), dtype=out_dtype, device=dev)
    _req(o, "out", out_dtype, (B, H, dv), dev)
    flags = _flags(l2norm_qk, gate_in_kernel, beta_logits)
    _check(lib.kda_step(B, H, dk, dv, _dt(q.dtype), _dt(out_dtype), float(scale), flags, _ptr(q),
                        _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(h),
                        _ptr(o), _stream(dev)))
    return o


def timing_enable(on: bool = True):
    """Start (and clear) or stop the library's per-kernel event timing."""
    _check(load_library().kda_timing_enable(1 if on else 0))


def timing_collect() -> dict:
    """Wait for the recorded events; returns {kernel: (launches, total_ms)} so far."""
    lib = load_library()
    _check(lib.kda_timing_collect())
    out = {}
    for i in range(lib.kda_timing_count()):
        name = ctypes.c_char_p()
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        _check(lib.kda_timing_get(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)))
        out[name.value.decode()] = (int(n.value), float(ms.value))
    return out


# ---------------------------------------------------------------- short convolution
def _conv_inputs(x, w, bias, cu_seqlens):
    _req(x, "x", (torch.bfloat16, torch.float32))
    if x.dim() != 3:
        raise ValueError("x must be [B,T,D]")
    dev = x.device
    B, T, D = x.shape
    _req(w, "w", torch.float32, None, dev)
    if w.dim() != 2 or w.shape[0] != D:
        raise ValueError("w must be [D,W]")
    _req(bias, "bias", torch.float32, (D,), dev, optional=True)
    N = 0
    if cu_seqlens is not None:
        _req(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        N = cu_seqlens.numel() - 1
    return B, T, D, w.shape[1], N


def conv_fwd(x, w, bias=None, cu_seqlens=None, *, silu=False, out_dtype=None):
    """kda_conv_fwd: short causal depthwise convolution of x [B,T,D]; returns y [B,T,D]."""
    lib = load_library()
    B, T, D, W, N = _conv_inputs(x, w, bias, cu_seqlens)
    out_dtype = out_dtype or x.dtype
    y = torch.empty((B, T, D), dtype=out_dtype, device=x.device)
    _check(lib.kda_conv_fwd(B, T, D, W, _dt(x.dtype), _dt(out_dtype), CONV_SILU if silu else 0, _ptr(x), _ptr(w),
                            _ptr(bias), _ptr(cu_seqlens), N, _ptr(y), _stream(x.device)))
    return y


def conv_bwd(x, w, dy, bias=None, cu_seqlens=None, *, silu=False, out_dtype=None, need_dbias=True, workspace=None):
    """kda_conv_bwd: returns dict dx [B,T,D], dw [D,W] fp32, dbias [D] fp32 (or None)."""
    lib = load_library()
    B, T, D, W, N = _conv_inputs(x, w, bias, cu_seqlens)
    dev = x.device
    _req(dy, "dy", x.dtype, (B, T, D), dev)
    out_dtype = out_dtype or x.dtype
    out = dict(dx=torch.empty((B, T, D), dtype=out_dtype, device=dev),
               dw=torch.empty((D, W), dtype=torch.float32, device=dev),
               dbias=torch.empty((D,), dtype=torch.float32, device=dev) if need_dbias else None)
    need = lib.kda_conv_bwd_workspace(B, T, D, W)
    if need == 0:
        _check(KDA_ERR_INVALID)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib.kda_conv_bwd(B, T, D, W, _dt(x.dtype), _dt(out_dtype), CONV_SILU if silu else 0, _ptr(x), _ptr(w),
                            _ptr(bias), _ptr(cu_seqlens), N, _ptr(dy), _ptr(out["dx"]), _ptr(out["dw"]),
                            _ptr(out["dbias"]), _ptr(ws), ws.numel(), _stream(dev)))
    return out


# ---------------------------------------------------------------- gated norm
def _gnorm_inputs(o, gate, weight):
    _req(o, "o", (torch.bfloat16, torch.float32))
    dev = o.device
    dv = o.shape[-1]
    _req(gate, "gate", o.dtype, tuple(o.shape), dev)
    _req(weight, "weight", torch.float32, (dv,), dev)
    return o.numel() // dv if dv else 0, dv


def gnorm_fwd(o, gate, weight, eps=RMS_EPS, *, out_dtype=None):
    """kda_gnorm_fwd: y = rmsnorm(o) * weight * sigmoid(gate) over the last axis (dv)."""
    lib = load_library()
    rows, dv = _gnorm_inputs(o, gate, weight)
    out_dtype = out_dtype or o.dtype
    y = torch.empty(o.shape, dtype=out_dtype, device=o.device)
    _check(lib.kda_gnorm_fwd(rows, dv, _dt(o.dtype), _dt(out_dtype), float(eps), _ptr(o), _ptr(gate), _ptr(weight),
                             _ptr(y), _stream(o.device)))
    return y


def gnorm_bwd(o, gate, weight, dy, eps=RMS_EPS, *, out_dtype=None, workspace=None):
    """kda_gnorm_bwd: returns dict do, dgate (shape of o) and dweight [dv] fp32."""
    lib = load_library()
    rows, dv = _gnorm_inputs(o, gate, weight)
    dev = o.device
    _req(dy, "dy", o.dtype, tuple(o.shape), dev)
    out_dtype = out_dtype or o.dtype
    out = dict(do=torch.empty(o.shape, dtype=out_dtype, device=dev),
               dgate=torch.empty(o.shape, dtype=out_dtype, device=dev),
               dweight=torch.empty((dv,), dtype=torch.float32, device=dev))
    need = lib.kda_gnorm_bwd_workspace(rows, dv)
    if need == 0:
        _check(KDA_ERR_INVALID)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib.kda_gnorm_bwd(rows, dv, _dt(o.dtype), _dt(out_dtype), float(eps), _ptr(o), _ptr(gate), _ptr(weight),
                             _ptr(dy), _ptr(out["do"]), _ptr(out["dgate"]), _ptr(out["dweight"]), _ptr(ws),
                             ws.numel(), _stream(dev)))
    return out


# ---------------------------------------------------------------- context parallelism
def segment_maps(q, k, v, g, beta, cu_seqlens=None, plan=None, *, A_log=None, dt_bias=None, l2norm_qk=False,
                 gate_in_kernel=False, beta_logits=False, workspace=None, fwd_saved=False):
    """kda_segment_maps: the state-transition matrix M [N,H,dk,dk] of every sequence or packed
    document: h_out = M h_in + (its hT from h0 = 0).  fwd_saved: `workspace` holds a
    kda_fwd(..., save_for_bwd=True) of the same inputs, whose chunk transitions are reused."""
    lib = load_library()
    B, T, H, dk, dv, N = _check_inputs(q, k, v, g, beta, None, cu_seqlens, plan, A_log, dt_bias, gate_in_kernel)
    flags = _flags(l2norm_qk, gate_in_kernel, beta_logits) | (F_FWD_SAVED if fwd_saved else 0)
    if fwd_saved and workspace is None:
        raise ValueError("fwd_saved needs the saved forward's workspace")
    desc = _desc(q, v, N, 1.0, flags, q.dtype)
    dev = q.device
    M = torch.empty((N, H, dk, dk), dtype=torch.float32, device=dev)
    need = lib.kda_fwd_workspace(ctypes.byref(desc))
    if need == 0:
        _check(KDA_ERR_INVALID)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    idx, off = plan if plan is not None else (None, None)
    _check(lib.kda_segment_maps(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log),
                                _ptr(dt_bias), _ptr(cu_seqlens), _ptr(idx), _ptr(off), _ptr(M), _ptr(ws), ws.numel(),
                                _stream(dev)))
    return M


def state_scan(M, c, x0=None, *, transpose=False):
    """kda_state_scan: chains R segments; returns (x_in [R,H,dk,dv], x_out [H,dk,dv])."""
    lib = load_library()
    _req(M, "M", torch.float32)
    R, H, dk, _ = M.shape
    dev = M.device
    _req(c, "c", torch.float32, None, dev)
    if c.dim() != 4 or tuple(c.shape[:3]) != (R, H, dk):
        raise ValueError("c must be [R,H,dk,dv]")
    dv = c.shape[-1]
    _req(x0, "x0", torch.float32, (H, dk, dv), dev, optional=True)
    x_in = torch.empty((R, H, dk, dv), dtype=torch.float32, device=dev)
    x_out = torch.empty((H, dk, dv), dtype=torch.float32, device=dev)
    _check(lib.kda_state_scan(R, H, dk, dv, 1 if transpose else 0, _ptr(M), _ptr(c), _ptr(x0), _ptr(x_in),
                              _ptr(x_out), _stream(dev)))
    return x_in, x_out
