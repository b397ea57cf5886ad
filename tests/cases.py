"""Input construction and comparison helpers for the parity tests.

Raw draws come from kda_inputs (no arithmetic of the method).  Prepared
inputs -- L2-normalised q, k, the decay gate g and beta -- are computed by the
oracle's preparation functions in fp64, then rounded to the dtype handed to
the GPU.  The oracle is always fed exactly the values the GPU receives,
widened to fp64.

Tolerances (stated once, used by every GPU test):
  * fp32 inputs: max |x - ref| / max |ref| <= 1e-4 per tensor (normwise
    relative error; elementwise relative error is ill-posed where the decay
    drives entries towards 0);
  * bf16 inputs, fp32 outputs: max |x - ref| <= 2e-2 * rms(ref) per tensor;
  * bf16 outputs: the bf16 tensor must equal the round-to-nearest-even of
    the fp32-output run of the same call, bit for bit, so it inherits the
    fp32-output bound up to its own final rounding.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import kda_inputs
import oracle

FP32_TOL = 1e-4
BF16_TOL = 2e-2


def to_np(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu", torch.float64).numpy()


def check_close(name, got, ref, in_dtype):
    """Assert the per-tensor bound for `in_dtype`; returns the measured ratio to the bound."""
    got = to_np(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s has non-finite values" % name
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    if in_dtype == torch.float32:
        scale = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1e-30)
        ratio = err / (FP32_TOL * scale)
        assert ratio <= 1.0, "%s: max rel err %.3e > %.1e" % (name, err / scale, FP32_TOL)
    else:
        rms = max(float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0, 1e-30)
        ratio = err / (BF16_TOL * rms)
    log = os.environ.get("KDA_RATIO_LOG")
    if log:  # the measured fraction of the bound, per tensor, for tolerance studies
        with open(log, "a") as fh:
            fh.write("%s %s %s %.4g\n" % (os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], name,
                                           "fp32" if in_dtype == torch.float32 else "bf16", ratio))
    if in_dtype != torch.float32:
        assert ratio <= 1.0, "%s: max abs err %.3e > %.1e * rms %.3e" % (name, err, BF16_TOL, rms)
    return ratio


def prepared(seed, B, T, H, dk, dv, dtype, *, weak=False, h0_std=None, n_states=None,
             upstream=False, dhT=False, variant=None):
    """Returns (gpu_inputs dict of CPU torch tensors, raw dict).

    gpu_inputs: q, k [B,T,H,dk] dtype (normalised); v dtype; g, beta fp32; h0;
    do (dtype), dhT.  Variants: 'g0' (no decay), 'beta1_unit' (beta = 1),
    None (the default distributions).
    """
    raw = kda_inputs.draw(seed, B, T, H, dk, dv, n_states=n_states, h0_std=h0_std,
                          upstream=upstream, dhT=dhT,
                          a_log_range=kda_inputs.A_LOG_RANGE_WEAK if weak else kda_inputs.A_LOG_RANGE)
    qh, kh, g, beta = oracle.prep_forward(raw["q_raw"], raw["k_raw"], raw["f"], raw["A_log"],
                                          raw["dt_bias"], raw["b"])
    if variant == "g0":
        g = np.zeros_like(g)
    elif variant == "beta1_unit":
        beta = np.ones_like(beta)
    elif variant is not None:
        raise ValueError(variant)
    out = dict(
        q=torch.tensor(qh, dtype=torch.float32).to(dtype),
        k=torch.tensor(kh, dtype=torch.float32).to(dtype),
        v=raw["v"].to(dtype),
        g=torch.tensor(g, dtype=torch.float32),
        beta=torch.tensor(beta, dtype=torch.float32),
        h0=raw["h0"],
        do=raw["do"].to(dtype) if raw["do"] is not None else None,
        dhT=raw["dhT"],
    )
    return out, raw


def raw_inputs(raw, dtype):
    """Inputs for the fused-preparation mode: raw q, k (dtype), f, b, A_log, dt_bias (fp32)."""
    return dict(q=raw["q_raw"].to(dtype), k=raw["k_raw"].to(dtype), v=raw["v"].to(dtype),
                g=raw["f"].clone(), beta=raw["b"].clone(), A_log=raw["A_log"].clone(),
                dt_bias=raw["dt_bias"].clone(), h0=raw["h0"],
                do=raw["do"].to(dtype) if raw["do"] is not None else None, dhT=raw["dhT"])


def to_dev(d, device="cuda"):
    return {k: (v.to(device).contiguous() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def oracle_fwd(inp, scale, cu=None):
    h0 = to_np(inp["h0"]) if inp.get("h0") is not None else None
    return oracle.forward(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g"]),
                          to_np(inp["beta"]), scale, h0=h0,
                          cu_seqlens=None if cu is None else to_np(cu).astype(np.int64))


def oracle_fwd_raw(rin, scale, cu=None):
    """Oracle forward in the fused-preparation mode (prep in fp64 from the same raw values)."""
    qh, kh, g, beta = oracle.prep_forward(to_np(rin["q"]), to_np(rin["k"]), to_np(rin["g"]),
                                          to_np(rin["A_log"]), to_np(rin["dt_bias"]),
                                          to_np(rin["beta"]))
    h0 = to_np(rin["h0"]) if rin.get("h0") is not None else None
    return oracle.forward(qh, kh, to_np(rin["v"]), g, beta, scale, h0=h0,
                          cu_seqlens=None if cu is None else to_np(cu).astype(np.int64))


def oracle_bwd(inp, scale, cu=None):
    h0 = to_np(inp["h0"]) if inp.get("h0") is not None else None
    dhT = to_np(inp["dhT"]) if inp.get("dhT") is not None else None
    return oracle.backward(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g"]),
                           to_np(inp["beta"]), scale, to_np(inp["do"]), h0=h0, dhT=dhT,
                           cu_seqlens=None if cu is None else to_np(cu).astype(np.int64))


def oracle_bwd_raw(rin, scale, cu=None):
    q_raw, k_raw, f, A_log, dt, b = (to_np(rin[x]) for x in ("q", "k", "g", "A_log", "dt_bias", "beta"))
    qh, kh, g, beta = oracle.prep_forward(q_raw, k_raw, f, A_log, dt, b)
    h0 = to_np(rin["h0"]) if rin.get("h0") is not None else None
    dhT = to_np(rin["dhT"]) if rin.get("dhT") is not None else None
    gr = oracle.backward(qh, kh, to_np(rin["v"]), g, beta, scale, to_np(rin["do"]), h0=h0, dhT=dhT,
                         cu_seqlens=None if cu is None else to_np(cu).astype(np.int64))
    pr = oracle.prep_backward(q_raw, k_raw, f, A_log, dt, b, gr["dq"], gr["dk"], gr["dg"],
                              gr["dbeta"])
    return dict(dq=pr["dq"], dk=pr["dk"], dv=gr["dv"], dg=pr["df"], dbeta=pr["db"], dh0=gr["dh0"],
                dA_log=pr["dA_log"], ddt_bias=pr["ddt_bias"])


def bf16_rne(x: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even of an fp32 tensor to bf16 (torch's conversion)."""
    return x.to(torch.bfloat16)
