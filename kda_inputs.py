"""Seeded synthetic input draws for KDA, shared by the tests, the smoke entry
and the bench.

This module holds none of the operator's arithmetic: it only draws raw random
tensors (CPU, float32, ``torch.Generator``) with the shapes and distributions
of the workloads, and document lengths for packed rows.  Everything derived
from them by the method (L2 normalisation, the decay gate, the sigmoid) is
computed by the caller.

Workload shapes: the 300M pure-KDA layer of the "Pure KDA 300M on Primus"
guide, section "Overview" (8 heads, head_k_dim 32, head_v_dim 64, sequence
length 2048); packed documents as in torchtitan PR #4347 ("Verification").
Value distributions: q, k, v, f, b ~ N(0,1); A_log = log U[1,16] per head;
dt_bias ~ N(0, 0.1) per channel; states and upstream gradients as stated per
draw.  Draw order within one seed: q, k, v, f, A_log, dt_bias, b, h0, do, dhT.
"""
from __future__ import annotations

import math

import torch

# A_log ranges: the default draw, and a weak-decay variant that keeps the
# state alive across many chunks (so the state path is actually exercised).
A_LOG_RANGE = (1.0, 16.0)
A_LOG_RANGE_WEAK = (0.01, 0.1)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(gen, shape, std=1.0):
    return torch.randn(*shape, generator=gen, dtype=torch.float32) * std


def _uniform(gen, shape, lo, hi):
    return torch.rand(*shape, generator=gen, dtype=torch.float32) * (hi - lo) + lo


def draw(seed: int, B: int, T: int, H: int, dk: int, dv: int, *, n_states: int | None = None,
         h0_std: float | None = None, upstream: bool = False, dhT: bool = False,
         a_log_range=A_LOG_RANGE) -> dict:
    """Raw draws for one forward(+backward) case.

    Returns float32 CPU tensors: q_raw, k_raw, f [B,T,H,dk]; v [B,T,H,dv];
    A_log [H]; dt_bias [H,dk]; b [B,T,H]; h0 [N,H,dk,dv] or None; do
    [B,T,H,dv] or None; dhT [N,H,dk,dv] or None.  N = ``n_states`` (default B).
    """
    gen = _gen(seed)
    N = B if n_states is None else n_states
    out = {}
    out["q_raw"] = _normal(gen, (B, T, H, dk))
    out["k_raw"] = _normal(gen, (B, T, H, dk))
    out["v"] = _normal(gen, (B, T, H, dv))
    out["f"] = _normal(gen, (B, T, H, dk))
    out["A_log"] = torch.log(_uniform(gen, (H,), *a_log_range))
    out["dt_bias"] = _normal(gen, (H, dk), 0.1)
    out["b"] = _normal(gen, (B, T, H))
    out["h0"] = _normal(gen, (N, H, dk, dv), h0_std) if h0_std is not None else None
    out["do"] = _normal(gen, (B, T, H, dv)) if upstream else None
    out["dhT"] = _normal(gen, (N, H, dk, dv)) if (upstream and dhT) else None
    return out


def draw_device(seed: int, B: int, T: int, H: int, dk: int, dv: int, device, dtype=torch.bfloat16, *,
                n_states: int | None = None, h0_std: float | None = None, upstream: bool = False,
                dhT: bool = False) -> dict:
    """The draws of ``draw`` made on the device (a device ``torch.Generator``), for
    rows too large to draw on the host: q_raw, k_raw, v (and do) come out in
    ``dtype``, the rest in float32.  Same distributions as ``draw``; the values
    differ from it (another generator)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    N = B if n_states is None else n_states

    def normal(shape, std=1.0, out_dtype=torch.float32):
        x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
        if std != 1.0:
            x.mul_(std)
        return x if out_dtype == torch.float32 else x.to(out_dtype)

    out = {}
    out["q_raw"] = normal((B, T, H, dk), out_dtype=dtype)
    out["k_raw"] = normal((B, T, H, dk), out_dtype=dtype)
    out["v"] = normal((B, T, H, dv), out_dtype=dtype)
    out["f"] = normal((B, T, H, dk))
    lo, hi = A_LOG_RANGE
    out["A_log"] = torch.log(torch.rand(H, generator=gen, dtype=torch.float32, device=device) * (hi - lo) + lo)
    out["dt_bias"] = normal((H, dk), 0.1)
    out["b"] = normal((B, T, H))
    out["h0"] = normal((N, H, dk, dv), h0_std) if h0_std is not None else None
    out["do"] = normal((B, T, H, dv), out_dtype=dtype) if upstream else None
    out["dhT"] = normal((N, H, dk, dv)) if (upstream and dhT) else None
    return out


def draw_decode(seed: int, steps: int, B: int, H: int, dk: int, dv: int, h_std: float = 0.1,
                a_log_range=A_LOG_RANGE) -> dict:
    """Raw draws for ``steps`` consecutive one-token decode steps.

    q_raw, k_raw, f [steps,B,H,dk]; v [steps,B,H,dv]; b [steps,B,H];
    A_log [H]; dt_bias [H,dk]; h [B,H,dk,dv] ~ N(0, h_std).
    """
    gen = _gen(seed)
    out = {}
    out["q_raw"] = _normal(gen, (steps, B, H, dk))
    out["k_raw"] = _normal(gen, (steps, B, H, dk))
    out["v"] = _normal(gen, (steps, B, H, dv))
    out["f"] = _normal(gen, (steps, B, H, dk))
    out["A_log"] = torch.log(_uniform(gen, (H,), *a_log_range))
    out["dt_bias"] = _normal(gen, (H, dk), 0.1)
    out["b"] = _normal(gen, (steps, B, H))
    out["h"] = _normal(gen, (B, H, dk, dv), h_std)
    return out


def geometric_cu_seqlens(seed: int, total: int = 65536, mean: int = 512,
                         force_single: bool = True) -> torch.Tensor:
    """Document offsets of one packed row of ``total`` tokens.

    Lengths are i.i.d. geometric on {1, 2, ...} with the given mean (inverse
    CDF of a uniform draw); the last document is truncated so the row is
    exactly ``total`` long.  If no length-1 document occurs and
    ``force_single`` is set, the first token of document 0 is split off as a
    document of its own, so length-1 documents are always present.
    Returns int32 cu_seqlens [N+1] with cu[0] = 0 and cu[N] = total.
    """
    gen = _gen(seed)
    p = 1.0 / mean
    lengths = []
    acc = 0
    while acc < total:
        u = float(torch.rand((), generator=gen, dtype=torch.float64))
        u = max(u, 1e-300)
        n = max(1, int(math.ceil(math.log(u) / math.log1p(-p))))
        n = min(n, total - acc)
        lengths.append(n)
        acc += n
    if force_single and 1 not in lengths and lengths[0] > 1:
        lengths = [1, lengths[0] - 1] + lengths[1:]
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    return torch.tensor(cu, dtype=torch.int32)
