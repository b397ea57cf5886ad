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
F_QK_L2NORM, F_GATE_IN_KERNEL, F_BETA_LOGITS, F_SAVE_FOR_BWD, F_FWD_SAVED = 1, 2, 4, 8, 16
CHUNK = 64

EXPORTS = ["kda_max_chunks", "kda_plan_varlen", "kda_check_cu_seqlens", "kda_fwd_workspace",
           "kda_bwd_workspace", "kda_fwd", "kda_bwd", "kda_step", "kda_status_str",
           "kda_last_error", "kda_timing_enable", "kda_timing_collect", "kda_timing_count",
           "kda_timing_get"]


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
        output_final_state=True, workspace=None, save_for_bwd=False):
    """kda_fwd.  Returns (o [B,T,H,dv], hT [N,H,dk,dv] or None).

    With save_for_bwd the workspace (which must then be sized for the backward)
    keeps what kda_bwd(..., fwd_saved=True, workspace=same) needs.
    """
    lib = load_library()
    B, T, H, dk, dv, N = _check_inputs(q, k, v, g, beta, h0, cu_seqlens, plan, A_log, dt_bias,
                                       gate_in_kernel)
    out_dtype = out_dtype or q.dtype
    flags = _flags(l2norm_qk, gate_in_kernel, beta_logits) | (F_SAVE_FOR_BWD if save_for_bwd else 0)
    desc = _desc(q, v, N, scale, flags, out_dtype)
    dev = q.device
    o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    need = (lib.kda_bwd_workspace if save_for_bwd else lib.kda_fwd_workspace)(ctypes.byref(desc))
    if need == 0:
        _check(KDA_ERR_INVALID)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    idx, off = plan if plan is not None else (None, None)
    _check(lib.kda_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                       _ptr(A_log), _ptr(dt_bias), _ptr(h0), _ptr(cu_seqlens), _ptr(idx), _ptr(off),
                       _ptr(o), _ptr(hT), _ptr(ws), ws.numel(), _stream(dev)))
    return o, hT


def bwd(q, k, v, g, beta, scale, d_o, h0=None, dhT=None, cu_seqlens=None, plan=None, *,
        A_log=None, dt_bias=None, l2norm_qk=False, gate_in_kernel=False, beta_logits=False,
        out_dtype=None, need_dh0=True, workspace=None, fwd_saved=False):
    """kda_bwd.  Returns dict dq, dk, dv, dg, dbeta, dh0 (and dA_log, ddt_bias with the gate).

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
    flags = _flags(l2norm_qk, gate_in_kernel, beta_logits) | (F_FWD_SAVED if fwd_saved else 0)
    if fwd_saved and workspace is None:
        raise ValueError("fwd_saved needs the forward's workspace")
    desc = _desc(q, v, N, scale, flags, out_dtype)
    out = dict(
        dq=torch.empty((B, T, H, dk), dtype=out_dtype, device=dev),
        dk=torch.empty((B, T, H, dk), dtype=out_dtype, device=dev),
        dv=torch.empty((B, T, H, dv), dtype=out_dtype, device=dev),
        dg=torch.empty((B, T, H, dk), dtype=torch.float32, device=dev),
        dbeta=torch.empty((B, T, H), dtype=torch.float32, device=dev),
        dh0=torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if need_dh0 else None,
    )
    if gate_in_kernel:
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
