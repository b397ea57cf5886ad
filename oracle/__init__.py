"""Plain fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package.  It shares
no code with the HIP path.

The arithmetic lives in ``kda_oracle.c`` (token-by-token recurrence, its
hand-derived backward, the decode step, the gate preparation and a chunked
fp64 rewrite used for chunk-size invariance).  This module builds it with gcc
and wraps it for numpy float64 arrays.  ``plan_varlen`` (the integer chunk
metadata) is written here in plain Python.

Sources of each definition (page title, section):
  * delta-rule recurrence with a per-channel decay gate: "Pure KDA 300M on
    Primus" guide, "Overview"; openkimi README, "What is implemented" and the
    FlashQLA paragraph (channel-wise decay);
  * document offsets resetting the recurrent state: torchtitan PR #4347
    "[kimi k3] Support sample packing in KDA", "Verification";
  * per-document chunk tables built once per batch: same PR, the paragraph on
    FLA's memoized varlen index helpers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``kda_oracle.c`` into ``liboracle.so`` with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)


def _p(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous, (a.dtype, a.flags)
    return a.ctypes.data_as(_D)


def _pi(a):
    assert a.dtype == np.int64 and a.flags.c_contiguous
    return a.ctypes.data_as(_I64)


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def num_threads() -> int:
    return int(_load().kdo_num_threads())


def segments_from(B: int, T: int, cu_seqlens=None):
    """Sequence table: dense [B,T] rows, or the documents of one packed row."""
    if cu_seqlens is None:
        start = np.arange(B, dtype=np.int64) * T
        length = np.full(B, T, dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        assert B == 1
        start = np.ascontiguousarray(cu[:-1])
        length = np.ascontiguousarray(cu[1:] - cu[:-1])
    return start, length


def forward(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, nthreads=0):
    """Token recurrence.  q,k,g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H].

    Returns (o [B,T,H,dv], hT [N,H,dk,dv]) in float64.
    """
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    start, length = segments_from(B, T, cu_seqlens)
    N = len(start)
    o = np.zeros((B, T, H, dv))
    hT = np.zeros((N, H, dk, dv))
    _load().kdo_forward(ctypes.c_int(N), _pi(start), _pi(length), H, dk, dv, _p(q), _p(k),
                        _p(v), _p(g), _p(beta), ctypes.c_double(scale), _p(h0), _p(o), _p(hT),
                        ctypes.c_int(nthreads))
    return o, hT


def chunked_forward(q, k, v, g, beta, scale, chunk, h0=None, cu_seqlens=None, nthreads=0):
    """The chunked (WY/UT) rewrite in fp64, for any chunk size."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    start, length = segments_from(B, T, cu_seqlens)
    N = len(start)
    o = np.zeros((B, T, H, dv))
    hT = np.zeros((N, H, dk, dv))
    _load().kdo_chunked_forward(ctypes.c_int(N), _pi(start), _pi(length), H, dk, dv, _p(q),
                                _p(k), _p(v), _p(g), _p(beta), ctypes.c_double(scale), _p(h0),
                                ctypes.c_int(chunk), _p(o), _p(hT), ctypes.c_int(nthreads))
    return o, hT


def backward(q, k, v, g, beta, scale, d_o, h0=None, dhT=None, cu_seqlens=None, nthreads=0):
    """Hand-derived backward of ``forward``.

    Returns dict with dq, dk, dv, dg [B,T,H,*], dbeta [B,T,H], dh0 [N,H,dk,dv].
    """
    q, k, v, g, beta, h0, d_o, dhT = map(_f64, (q, k, v, g, beta, h0, d_o, dhT))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    start, length = segments_from(B, T, cu_seqlens)
    N = len(start)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dg=np.zeros_like(g), dbeta=np.zeros_like(beta), dh0=np.zeros((N, H, dk, dv)))
    _load().kdo_backward(ctypes.c_int(N), _pi(start), _pi(length), H, dk, dv, _p(q), _p(k),
                         _p(v), _p(g), _p(beta), ctypes.c_double(scale), _p(h0), _p(d_o),
                         _p(dhT), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dg"]),
                         _p(out["dbeta"]), _p(out["dh0"]), ctypes.c_int(nthreads))
    return out


def step(q, k, v, g, beta, scale, h, nthreads=0):
    """One decode step.  q,k,g [B,H,dk]; v [B,H,dv]; beta [B,H]; h [B,H,dk,dv].

    Returns (o [B,H,dv], h_new) without modifying the argument ``h``.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    hn = np.array(h, dtype=np.float64, copy=True, order="C")
    B, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, dv))
    _load().kdo_step(B, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                     ctypes.c_double(scale), _p(hn), _p(o), ctypes.c_int(nthreads))
    return o, hn


# --------------------------------------------------------------------------
# Gate preparation (fused Q/K norm, decay gate and beta; openkimi README,
# "What is implemented"; decay gate with A_log and dt_bias through softplus,
# Primus guide "Overview").
# --------------------------------------------------------------------------
L2_EPS = 1e-6


def l2norm(x, eps=L2_EPS):
    x = _f64(x)
    d = x.shape[-1]
    y = np.empty_like(x)
    _load().kdo_l2norm_fwd(ctypes.c_int64(x.size // d), d, ctypes.c_double(eps), _p(x), _p(y))
    return y


def l2norm_bwd(x, dy, eps=L2_EPS):
    x, dy = _f64(x), _f64(dy)
    d = x.shape[-1]
    dx = np.empty_like(x)
    _load().kdo_l2norm_bwd(ctypes.c_int64(x.size // d), d, ctypes.c_double(eps), _p(x), _p(dy),
                           _p(dx))
    return dx


def gate(f, A_log, dt_bias):
    """g = -exp(A_log[h]) * softplus(f + dt_bias[h, c]);  f [..., H, dk]."""
    f, A_log, dt_bias = map(_f64, (f, A_log, dt_bias))
    H, dk = f.shape[-2], f.shape[-1]
    g = np.empty_like(f)
    _load().kdo_gate_fwd(ctypes.c_int64(f.size // (H * dk)), H, dk, _p(f), _p(A_log),
                         _p(dt_bias), _p(g))
    return g


def gate_bwd(f, A_log, dt_bias, dg):
    f, A_log, dt_bias, dg = map(_f64, (f, A_log, dt_bias, dg))
    H, dk = f.shape[-2], f.shape[-1]
    df = np.empty_like(f)
    dA = np.empty(H)
    ddt = np.empty((H, dk))
    _load().kdo_gate_bwd(ctypes.c_int64(f.size // (H * dk)), H, dk, _p(f), _p(A_log),
                         _p(dt_bias), _p(dg), _p(df), _p(dA), _p(ddt))
    return df, dA, ddt


def sigmoid(b):
    b = _f64(b)
    y = np.empty_like(b)
    _load().kdo_sigmoid_fwd(ctypes.c_int64(b.size), _p(b), _p(y))
    return y


def sigmoid_bwd(b, dbeta):
    b, dbeta = _f64(b), _f64(dbeta)
    db = np.empty_like(b)
    _load().kdo_sigmoid_bwd(ctypes.c_int64(b.size), _p(b), _p(dbeta), _p(db))
    return db


def prep_forward(q_raw, k_raw, f, A_log, dt_bias, b):
    """Raw inputs -> (q^, k^, g, beta) as the fused preparation defines them."""
    return l2norm(q_raw), l2norm(k_raw), gate(f, A_log, dt_bias), sigmoid(b)


def prep_backward(q_raw, k_raw, f, A_log, dt_bias, b, dq, dk, dg, dbeta):
    """Chain the recurrence gradients back to the raw inputs."""
    df, dA, ddt = gate_bwd(f, A_log, dt_bias, dg)
    return dict(dq=l2norm_bwd(q_raw, dq), dk=l2norm_bwd(k_raw, dk), df=df,
                db=sigmoid_bwd(b, dbeta), dA_log=dA, ddt_bias=ddt)


# --------------------------------------------------------------------------
# Varlen chunk metadata (integer).  Chunks restart at every document, so a
# packed document is tiled exactly as if it were run alone (torchtitan PR
# #4347, "Verification": packed row equals the per-document runs).
# --------------------------------------------------------------------------
def max_chunks(T: int, N: int, chunk: int) -> int:
    """Upper bound on the chunk count of any N documents totalling T tokens."""
    return (T + N * (chunk - 1)) // chunk


def plan_varlen(cu_seqlens, chunk: int):
    """Returns (chunk_indices [M,2] int32 rows (doc, i), chunk_offsets [N+1] int32).

    Written as a plain enumeration over documents and their chunks.
    """
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    offsets = [0]
    rows = []
    for n in range(N):
        length = cu[n + 1] - cu[n]
        count = 0
        start = 0
        while start < length:
            rows.append((n, count))
            count += 1
            start += chunk
        offsets.append(offsets[-1] + count)
    idx = np.array(rows, dtype=np.int32).reshape(-1, 2)
    return idx, np.array(offsets, dtype=np.int32)
