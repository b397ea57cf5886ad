#!/usr/bin/env python3
"""KDA forward+backward throughput on one MI355X.

One step = kda_fwd + kda_bwd over one batch of the 300M pure-KDA layer shape
("Pure KDA 300M on Primus" guide, Overview: 8 heads, head_k_dim 32,
head_v_dim 64; sequence length 2048), bf16 q/k/v, fp32 decay/beta/state,
with the fused preparation on (raw q/k L2-normalised in-kernel, the decay gate
from f, A_log and dt_bias, beta from logits) so every step of the hot path
runs: gate preparation, intra-chunk, state passing, output, the mirrored
backward and the preparation chain.  Inputs are synthetic (kda_inputs), drawn
on the CPU and copied to HBM before the timed region.

Prints one JSON line.  `roofline` reports the kernel that takes the most
time, with its algorithmic work per launch (see kda_work below) divided by
its average duration measured with HIP events on the launch stream.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "KDA fwd+bwd tokens/s at H=8,dk=32,dv=64,T=2048; % of MI355X roofline"

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3


def kda_work(B, T, H, dk, dv, C=64):
    """Algorithmic work per kernel launch of one step, from the chunk algebra.

    Bytes: what the operator must read and write at least once
      forward   q,k (bf16) + v (bf16) + f (fp32) + b (fp32) -> o (bf16)
      backward  the forward inputs + do -> dq, dk, dv (bf16), df (fp32), db (fp32)
    FLOPs (2 per multiply-add) of the products each kernel performs per
    chunk-head, Gram/pair terms counted on their triangles:
    """
    th = B * T * H                      # token-heads
    ch = B * ((T + C - 1) // C) * H     # chunk-heads
    tri = C * (C + 1) // 2              # lower triangle incl. diagonal
    f = {}
    # fwd_intra: Akk and Aqk pairwise (tri*dk each), UT inverse (~C^3/6), w (tri*dk), u (tri*dv)
    f["fwd_intra"] = 2 * ch * (2 * tri * dk + C ** 3 // 6 + tri * dk + tri * dv)
    # fwd_state: v_new = u - w h (C*dk*dv), h' = Kh^T v_new (C*dk*dv)
    f["fwd_state"] = 2 * ch * (2 * C * dk * dv)
    # fwd_output: Qg h (C*dk*dv) + Aqk v_new (tri*dv)
    f["fwd_output"] = 2 * ch * (C * dk * dv + tri * dv)
    # bwd_dh: Aqk^T dO (tri*dv), Kh D (C*dk*dv), Qg^T dO (C*dk*dv), w^T dvn (C*dk*dv)
    f["bwd_dh"] = 2 * ch * (tri * dv + 3 * C * dk * dv)
    # bwd_dv: dQg, dKh, dw (3*C*dk*dv), dAqk, dT_v (2*C*C*dv), T^T dvn (tri*dv)
    f["bwd_dv"] = 2 * ch * (3 * C * dk * dv + 2 * C * C * dv + tri * dv)
    # bwd_dk: dT += dw Kg^T (C*C*dk), T^T dw (tri*dk), dT T^T and T^T Y (2*C^3/2),
    #         four decayed pair sums (4*tri*dk)
    f["bwd_dk"] = 2 * ch * (C * C * dk + tri * dk + C ** 3 + 4 * tri * dk)
    fwd_bytes = th * (2 * 2 * dk + 2 * dv + 4 * dk + 4 + 2 * dv)
    bwd_bytes = th * (2 * 2 * dk + 2 * dv + 4 * dk + 4 + 2 * dv + 2 * 2 * dk + 2 * dv + 4 * dk + 4)
    return f, fwd_bytes, bwd_bytes


def cpu_baseline(B, T, H, dk, dv, seconds):
    """The fp64 oracle (as it stands) on a bounded sample: whole sequences of the
    same workload, all heads, repeated until about `seconds` of CPU work."""
    import numpy as np

    import kda_inputs
    import oracle

    import torch

    threads = oracle.num_threads()
    nseq = max(1, min(B, threads // H))  # enough (sequence, head) pairs for every thread
    raw = kda_inputs.draw(1, nseq, T, H, dk, dv, upstream=True)
    as_bf16 = lambda x: raw[x].to(torch.bfloat16).double().numpy()  # same values the GPU receives
    q, k, v, do = (as_bf16(x) for x in ("q_raw", "k_raw", "v", "do"))
    f, b = (raw[x].double().numpy() for x in ("f", "b"))
    A_log = raw["A_log"].numpy().astype(np.float64)
    dtb = raw["dt_bias"].numpy().astype(np.float64)
    scale = dk ** -0.5
    reps = 0
    t0 = time.perf_counter()
    while True:
        qh, kh, g, beta = oracle.prep_forward(q, k, f, A_log, dtb, b)
        o, hT = oracle.forward(qh, kh, v, g, beta, scale)
        gr = oracle.backward(qh, kh, v, g, beta, scale, do)
        oracle.prep_backward(q, k, f, A_log, dtb, b, gr["dq"], gr["dk"], gr["dg"], gr["dbeta"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": nseq * T * reps / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d x (%d sequences x %d tokens x %d heads), prep+fwd+bwd+prep-bwd in fp64, %.1f s"
                      % (reps, nseq, T, H, el)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--seq", type=int, default=2048)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out-dtype", choices=["bf16", "fp32"], default="bf16")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the operator shards by sequence and head with no communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import kda_inputs
    import kimi_delta_attention_chunk_amd as kda

    B, T, H, dk, dv = args.batch, args.seq, 8, 32, 64
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    out_dtype = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    raw = kda_inputs.draw(1, B, T, H, dk, dv, upstream=True)
    bf = torch.bfloat16
    q = raw["q_raw"].to(bf).to(dev)
    k = raw["k_raw"].to(bf).to(dev)
    v = raw["v"].to(bf).to(dev)
    f = raw["f"].to(dev)
    b = raw["b"].to(dev)
    A_log = raw["A_log"].to(dev)
    dtb = raw["dt_bias"].to(dev)
    do = raw["do"].to(bf).to(dev)
    scale = dk ** -0.5
    flags = dict(A_log=A_log, dt_bias=dtb, l2norm_qk=True, gate_in_kernel=True, beta_logits=True,
                 out_dtype=out_dtype)
    # one workspace: the forward keeps what the backward needs (save-for-backward)
    ws = torch.empty(kda.workspace_bytes((B, T, H, dk), dv, B, True), dtype=torch.uint8, device=dev)

    def step():
        o, hT = kda.fwd(q, k, v, f, b, scale, workspace=ws, save_for_bwd=True, **flags)
        g = kda.bwd(q, k, v, f, b, scale, do, workspace=ws, fwd_saved=True, need_dh0=False, **flags)
        return o, g

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps; per-kernel HIP events on the launch stream
    kda.timing_enable(True)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    per_kernel = kda.timing_collect()
    kda.timing_enable(False)

    tokens = B * T
    value = tokens / (ms * 1e-3)
    flops, fwd_bytes, bwd_bytes = kda_work(B, T, H, dk, dv)
    kernels = {name: {"launches_per_step": n / args.steps, "avg_us": 1e3 * tot / n,
                      "share": tot / (ms * args.steps)} for name, (n, tot) in per_kernel.items()}
    dom = max(per_kernel, key=lambda nm: per_kernel[nm][1])
    n_dom, tot_dom = per_kernel[dom]
    avg_s = tot_dom / n_dom * 1e-3
    achieved = flops.get(dom, 0) / avg_s / 1e12
    roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS, "traffic": None,
            "avg_us": avg_s * 1e6, "work_per_launch": flops.get(dom, 0), "precision": "fp32"}
    step_bytes = fwd_bytes + bwd_bytes
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded draws; no dataset)",
        "config": {"workload": "KDA fwd+bwd, 300M layer shape: B=%d T=%d H=%d dk=%d dv=%d chunk=64, "
                               "bf16 q/k/v, fused q/k L2-norm + decay gate + sigmoid beta" % (B, T, H, dk, dv),
                   "global_batch": B, "seq_len": T, "heads": H, "dk": dk, "dv": dv,
                   "out_dtype": args.out_dtype, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "step_hbm_roofline": {"algorithmic_bytes": step_bytes,
                              "achieved_GBs": step_bytes / (ms * 1e-3) / 1e9,
                              "frac_of_8TBs": step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(B, T, H, dk, dv, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
