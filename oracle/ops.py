"""Plain fp64 CPU oracle for the two operations next to KDA in its layer: the
short causal depthwise convolution before it and the gated output norm after
it.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It
shares no code with the HIP path.

Sources (page title, section):
  * short convolution: "Pure KDA 300M on Primus" guide, "Overview" (kernel
    size 4, depthwise, on the concatenated q/k/v channels) and
    "Troubleshooting" (the [B, T, D] layout is the native one);
    torchtitan PR #4347 "[kimi k3] Support sample packing in KDA",
    description (with document offsets the convolution window resets at
    document boundaries);
  * gated output norm: openkimi README, "Profiling and H100 acceptance" (the
    KDA output goes through a fused RMSNorm and a sigmoid gate); Primus guide,
    "Overview" (per-head output gate, RMSNorm eps 1e-6) and "Step 7" (one
    g_norm per head, FusedRMSNormGated).

Readings where the pages are silent (each one is listed in the design notes):
  * convolution: y[t, c] = sum_{i < W} w[c, i] x[t - (W - 1) + i, c] over the
    positions of the same document (earlier positions count as zero), plus an
    optional per-channel bias, then an optional SiLU; the pages name neither
    a bias nor an activation, so both are options;
  * gated norm: per (token, head) row of dv values,
    y = o (mean(o^2) + eps)^{-1/2} * weight * sigmoid(gate), with one weight
    vector of dv values shared by the heads (the norm is applied per head).
"""
from __future__ import annotations

import numpy as np

RMS_EPS = 1e-6  # Primus guide, "Overview": RMSNorm with eps = 1e-6


def _f64(x):
    return np.asarray(x.detach().cpu() if hasattr(x, "detach") else x, dtype=np.float64)


def doc_starts(B, T, cu_seqlens=None):
    """For every (b, t): the first position of its document (dense rows: 0)."""
    start = np.zeros((B, T), dtype=np.int64)
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        assert B == 1 and cu[0] == 0 and cu[-1] == T
        for n in range(len(cu) - 1):
            start[0, cu[n]:cu[n + 1]] = cu[n]
    return start


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _dsilu(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def conv_preact(x, w, bias=None, cu_seqlens=None):
    """z[b, t, c] = sum_i w[c, i] x[b, t - (W-1) + i, c] (same document only) + bias[c]."""
    x, w = _f64(x), _f64(w)
    B, T, D = x.shape
    W = w.shape[1]
    start = doc_starts(B, T, cu_seqlens)
    z = np.zeros_like(x)
    for i in range(W):
        lag = W - 1 - i  # tap i reads x at t - lag
        for b in range(B):
            for t in range(T):
                s = t - lag
                if s >= start[b, t]:
                    z[b, t] += w[:, i] * x[b, s]
    if bias is not None:
        z += _f64(bias)[None, None, :]
    return z


def conv_fwd(x, w, bias=None, cu_seqlens=None, silu=False):
    z = conv_preact(x, w, bias, cu_seqlens)
    return _silu(z) if silu else z


def conv_bwd(x, w, dy, bias=None, cu_seqlens=None, silu=False):
    """Gradients of sum(dy * conv_fwd(...)) with respect to x, w and bias.

    With z the pre-activation and dz = dy * act'(z):
      dx[b, s] = sum_i w[:, i] dz[b, s + lag_i]   (t = s + lag_i in the same document)
      dw[:, i] = sum_{b, t} dz[b, t] x[b, t - lag_i]   (same document)
      dbias    = sum_{b, t} dz[b, t]
    """
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    B, T, D = x.shape
    W = w.shape[1]
    z = conv_preact(x, w, bias, cu_seqlens)
    dz = dy * _dsilu(z) if silu else dy
    start = doc_starts(B, T, cu_seqlens)
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    for i in range(W):
        lag = W - 1 - i
        for b in range(B):
            for t in range(T):
                s = t - lag
                if s >= start[b, t]:
                    dx[b, s] += w[:, i] * dz[b, t]
                    dw[:, i] += dz[b, t] * x[b, s]
    dbias = dz.sum(axis=(0, 1))
    return dx, dw, dbias


def gnorm_fwd(o, gate, weight, eps=RMS_EPS):
    """y = o r * weight * sigmoid(gate), r = (mean over the last axis of o^2 + eps)^{-1/2}."""
    o, gate, weight = _f64(o), _f64(gate), _f64(weight)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * weight * (1.0 / (1.0 + np.exp(-gate)))


def gnorm_bwd(o, gate, weight, dy, eps=RMS_EPS):
    """Gradients of sum(dy * gnorm_fwd(...)) with respect to o, gate and weight.

    With n = o r, s = sigmoid(gate), d = the row length:
      dgate   = dy * n * weight * s (1 - s)
      dweight = sum over rows of dy * n * s
      dn      = dy * weight * s
      do      = r (dn - n * mean(dn * n))      (r depends on o through mean(o^2))
    """
    o, gate, weight, dy = _f64(o), _f64(gate), _f64(weight), _f64(dy)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    n = o * r
    s = 1.0 / (1.0 + np.exp(-gate))
    dgate = dy * n * weight * s * (1.0 - s)
    dweight = (dy * n * s).reshape(-1, o.shape[-1]).sum(axis=0)
    dn = dy * weight * s
    do = r * (dn - n * np.mean(dn * n, axis=-1, keepdims=True))
    return do, dgate, dweight
