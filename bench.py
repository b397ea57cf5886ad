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

Prints one JSON line.  `value` and `ms_per_step` come from K steps timed with
nothing else on the stream.  `roofline` reports the kernel that takes the most
time, with its algorithmic work per launch (see kda_work below) divided by
its average duration, measured with a HIP-event pair around every launch on
the launch stream during a second pass of the same K steps.  `cpu_baseline`
times the fp64 oracle on the same draw: forward, forward + backward, and a
single-thread leg.
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
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3

HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "bwd_chunk_layer300M_B16_hbm_traffic.txt")


def kda_work(B, T, H, dk, dv, C=64):
    """Algorithmic work per launch of each kernel of one step.

    Per token-head (dk=32, dv=64, bf16 q/k/v/o/do/dq/dk/dv, fp32 f/b/df/db):
      bytes  forward  read q, k, v, f, b; write o         -> fwd_intra reads the inputs,
                                                             fwd_scan writes o and the final state
             backward read q, k, v, f, b, do; write dq, dk, dv, df, db
                                                          -> all of it in bwd_chunk
      FLOPs  what each kernel computes (2 per multiply-add, triangles counted as halves),
             per token-head, i.e. per chunk / C:
             fwd_intra  Akk, Aqk, w (3 C dk), u (C dv), the unit-triangular inverse (C^2/3),
                        and the affine chunk form: P, P^T (4 dk^2), hh (2 dk dv),
                        qh, qh^T (2 C dk), ol (C dv)
             fwd_scan   h' = P h + hh (2 dk^2 dv / C), o = ol + qh h (2 dk dv)
             bwd_dh     D = P^T D' + qh^T dO (2 dk^2 dv / C + 2 dk dv)
             bwd_chunk  v_new = T (beta V - beta Kg h), dv_new = Kh D' + Aqk^T dO
                        (4 dk dv + 2 C dv); dO h^T, vn D^T, dvn h^T (6 dk dv);
                        dAqk, dT_v, T^T dvn (3 C dv); dw (bKg)^T, T^T dw (2 C dk);
                        dA = -T^T dT T^T (2 C^2/3); four decayed pair sums (4 C dk)
    Intermediates the kernels pass to each other (T, the affine form, states, ...)
    are not algorithmic bytes; the measured traffic shows them.
    """
    th = B * T * H  # token-heads
    per = {
        "fwd_intra": (2 * 2 * dk + 2 * dv + 4 * dk + 4,
                      3 * C * dk + C * dv + C * C / 3 + 4 * dk * dk + 2 * dk * dv + 2 * C * dk + C * dv),
        "fwd_scan": (2 * dv + 4 * dk * dv / T, 2 * dk * dk * dv / C + 2 * dk * dv),
        "bwd_dh": (0.0, 2 * dk * dk * dv / C + 2 * dk * dv),
        "bwd_chunk": (2 * 2 * dk + 2 * dv + 4 * dk + 4 + 2 * dv + 2 * 2 * dk + 2 * dv + 4 * dk + 4,
                      4 * dk * dv + 2 * C * dv + 6 * dk * dv + 3 * C * dv + 2 * C * dk + 2 * C * C / 3 + 4 * C * dk),
        "bwd_gate_sum": (0.0, 0.0),
    }
    return {k: (th * b, th * f) for k, (b, f) in per.items()}


def kernel_source_hash():
    """Hash of the HIP sources, so measured counters are used only for the code they measured."""
    import hashlib

    d = os.path.join(HERE, "kimi_delta_attention_chunk_amd", "csrc")
    hsh = hashlib.sha256()
    for nm in sorted(os.listdir(d)):
        with open(os.path.join(d, nm), "rb") as fh:
            hsh.update(nm.encode() + b"\0" + fh.read())
    return hsh.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed PMC summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by the same counter on a copy of known size), or None when
    there is none for this kernel or the sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = [json.loads(l) for l in fh if l.startswith("{")][-1]
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("csrc_sha") != kernel_source_hash():
        return None
    return rec["fetch_bytes"] / rec["fetch_factor"] + rec["write_bytes"] / rec["write_factor"]


def copy_calibration(mb):
    """A plain device copy of `mb` MiB (torch copy_), 5 times: the reference reading for the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = mb * (1 << 20) // 4
    x = torch.randn(n, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "launches": 5}), flush=True)


def cpu_threads():
    """Host threads for the oracle: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when the environment sets it (the host's share per GPU)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return (min(n, int(cap)) if cap.isdigit() and int(cap) > 0 else n), n


def cpu_baseline(raw, T, H, dk, dv, single_seqs=1):
    """The fp64 oracle (as it stands, never tuned) on the same draw the GPU times:
    forward (prep + recurrence) and forward + backward (prep, recurrence, its
    backward, prep backward) over the whole batch on all host threads, and
    forward + backward on `single_seqs` sequences on one thread; each leg one
    warm-up and three timed repetitions, median wall clock."""
    import statistics

    import numpy as np

    import oracle

    import torch

    threads, affinity = cpu_threads()
    as_bf16 = lambda x: raw[x].to(torch.bfloat16).double().numpy()  # the values the GPU receives
    q, k, v, do = (as_bf16(x) for x in ("q_raw", "k_raw", "v", "do"))
    f, b = (raw[x].double().numpy() for x in ("f", "b"))
    A_log = raw["A_log"].numpy().astype(np.float64)
    dtb = raw["dt_bias"].numpy().astype(np.float64)
    scale = dk ** -0.5
    B = q.shape[0]

    def fwd(sl, nt):
        qh, kh, g, beta = oracle.prep_forward(q[sl], k[sl], f[sl], A_log, dtb, b[sl])
        oracle.forward(qh, kh, v[sl], g, beta, scale, nthreads=nt)

    def fwd_bwd(sl, nt):
        qh, kh, g, beta = oracle.prep_forward(q[sl], k[sl], f[sl], A_log, dtb, b[sl])
        oracle.forward(qh, kh, v[sl], g, beta, scale, nthreads=nt)
        gr = oracle.backward(qh, kh, v[sl], g, beta, scale, do[sl], nthreads=nt)
        oracle.prep_backward(q[sl], k[sl], f[sl], A_log, dtb, b[sl], gr["dq"], gr["dk"], gr["dg"], gr["dbeta"])

    def median_s(fn, *a):
        fn(*a)
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn(*a)
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    everything = slice(0, B)
    one = slice(0, min(single_seqs, B))
    t_f = median_s(fwd, everything, threads)
    t_fb = median_s(fwd_bwd, everything, threads)
    t_1 = median_s(fwd_bwd, one, 1)
    n1 = one.stop - one.start
    return {"value": B * T / t_fb, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "the whole timed batch (%d x %d tokens x %d heads, the GPU's own draw) on %d threads; "
                      "the single-thread leg on %d sequence(s); fp64, 1 warm-up + 3 timed, median"
                      % (B, T, H, threads, n1),
            "fwd_tokens_per_s": B * T / t_f, "fwd_bwd_tokens_per_s": B * T / t_fb,
            "fwd_s": t_f, "fwd_bwd_s": t_fb,
            "single_thread_fwd_bwd_tokens_per_s": n1 * T / t_1, "single_thread_fwd_bwd_s": t_1,
            "affinity_cpus": affinity}


def flushed_median(step, dev, reps):
    """Median step time with the 256 MB Infinity Cache flushed before every rep
    (a 512 MB buffer written between reps), so no input or workspace line is
    served from it."""
    import torch

    buf = torch.empty(512 << 18, dtype=torch.float32, device=dev)  # 512 MiB
    times = []
    for _ in range(reps):
        buf.fill_(1.0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    med = times[len(times) // 2]
    return {"median_ms": med, "reps": reps, "flush_bytes": 512 << 20, "tokens_per_s": None}


def secondary_run(q, k, v, f, b, do, scale, flags, B, T, H, dk, dv, dev, mult=8, steps=3):
    """One GPU's data-parallel share at the pages' per-GPU micro-batch: B*mult
    sequences (the headline draw repeated along the batch), fwd+bwd, mean of
    `steps` after one warm-up."""
    import torch

    import kimi_delta_attention_chunk_amd as kda

    rep = lambda x: x.repeat(mult, *([1] * (x.dim() - 1))).contiguous()
    q2, k2, v2, f2, b2, do2 = (rep(x) for x in (q, k, v, f, b, do))
    B2 = B * mult
    ws2 = torch.empty(kda.workspace_bytes((B2, T, H, dk), dv, B2, True), dtype=torch.uint8, device=dev)

    def step2():
        kda.fwd(q2, k2, v2, f2, b2, scale, workspace=ws2, save_for_bwd=True, **flags)
        kda.bwd(q2, k2, v2, f2, b2, scale, do2, workspace=ws2, fwd_saved=True, need_dh0=False, **flags)

    step2()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step2()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"global_batch": B2, "seq_len": T, "ms_per_step": ms, "tokens_per_s": B2 * T / (ms * 1e-3),
            "steps": steps, "data": "the headline draw repeated %dx along the batch" % mult}


def io_bytes(B, T, H, dk, dv, N, esz, h0, dhT, backward):
    """Algorithmic HBM bytes of one kda_fwd (+ kda_bwd) call: the inputs read and
    outputs written once, at their own element sizes (esz for q/k/v/o/do/dq/dk/dv,
    4 for f, b, df, db and every state)."""
    th = B * T * H
    fwd = th * (2 * esz * dk + esz * dv + 4 * dk + 4 + esz * dv)
    st = N * H * dk * dv * 4
    fwd += st * ((1 if h0 else 0) + 1)  # h0 read, hT written
    if not backward:
        return fwd
    bwd = th * (2 * esz * dk + esz * dv + 4 * dk + 4 + esz * dv) + th * (2 * esz * dk + esz * dv + 4 * dk + 4)
    bwd += st * ((1 if h0 else 0) + (1 if dhT else 0) + (1 if h0 else 0))  # h0, dhT read, dh0 written
    return fwd + bwd


def chunked_flops(dk, dv, C=64):
    """FLOPs per token-head of the chunked forward + backward (2 per multiply-add,
    triangles as halves): forward 3C dk + 2C dv + C^2/3 + 6 dk dv, backward
    recompute + gradients (3C dk + C dv + C^2/3 + 4 dk dv) + (6C dk + 4C dv +
    2C^2/3 + 12 dk dv)."""
    fwd = 3 * C * dk + 2 * C * dv + C * C / 3 + 6 * dk * dv
    bwd = (3 * C * dk + C * dv + C * C / 3 + 4 * dk * dv) + (6 * C * dk + 4 * C * dv + 2 * C * C / 3 + 12 * dk * dv)
    return fwd + bwd


def timed_ms(fn, reps, warm=2):
    """Mean milliseconds of fn() over reps, HIP events on the current stream."""
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def fwd_bwd_workload(name, dev, B, T, H, dk, dv, seed, packed=False, reps=10):
    """fwd+bwd of another configuration: tokens/s and the fraction of its binding
    roofline, max(bytes / HBM peak, 3 x FLOPs / bf16 MFMA peak) (products issued as
    three bf16 MFMAs, hi/lo split)."""
    import torch

    import kda_inputs
    import kimi_delta_attention_chunk_amd as kda

    bf = torch.bfloat16
    cu = plan = None
    if packed:
        cu = kda_inputs.geometric_cu_seqlens(seed, total=T).to(dev)
        N = cu.numel() - 1
        plan = kda.plan_varlen(cu, T)
    else:
        N = B
    raw = kda_inputs.draw(seed, B, T, H, dk, dv, n_states=N, h0_std=0.1 if packed else None,
                          upstream=True, dhT=packed)
    q, k, v, do = (raw[x].to(bf).to(dev) for x in ("q_raw", "k_raw", "v", "do"))
    f, b, A_log, dtb = (raw[x].to(dev) for x in ("f", "b", "A_log", "dt_bias"))
    h0 = raw["h0"].to(dev) if raw["h0"] is not None else None
    dhT = raw["dhT"].to(dev) if raw["dhT"] is not None else None
    scale = dk ** -0.5
    flags = dict(A_log=A_log, dt_bias=dtb, l2norm_qk=True, gate_in_kernel=True, beta_logits=True)
    ws = torch.empty(kda.workspace_bytes((B, T, H, dk), dv, N, True), dtype=torch.uint8, device=dev)

    def step():
        kda.fwd(q, k, v, f, b, scale, h0=h0, cu_seqlens=cu, plan=plan, workspace=ws, save_for_bwd=True,
                **flags)
        kda.bwd(q, k, v, f, b, scale, do, h0=h0, dhT=dhT, cu_seqlens=cu, plan=plan, workspace=ws,
                fwd_saved=True, need_dh0=packed, **flags)

    ms = timed_ms(step, reps)
    nbytes = io_bytes(B, T, H, dk, dv, N, 2, h0 is not None, dhT is not None, True)
    flops = chunked_flops(dk, dv) * B * T * H
    t_hbm, t_mfma = nbytes / (PEAK_HBM_GBS * 1e9), 3 * flops / (PEAK_BF16_TFLOPS * 1e12)
    t_roof = max(t_hbm, t_mfma)
    return {"workload": name, "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "documents": N,
            "ms_per_step": ms, "tokens_per_s": B * T / (ms * 1e-3), "reps": reps,
            "algorithmic_bytes": nbytes, "flops": flops, "bound": "hbm" if t_hbm >= t_mfma else "mfma",
            "roofline_us": t_roof * 1e6, "frac": t_roof / (ms * 1e-3)}


def decode_workload(dev, steps=1000, B=256, H=8, dk=32, dv=64, seed=2):
    """kda_step for `steps` consecutive tokens of B sequences (bf16 q/k/v, fp32 f/b and
    state, fused preparation), captured once in a HIP graph and replayed: microseconds
    per step and effective GB/s of its algorithmic bytes (state read and written, the
    token's inputs and output).  The 16.8 MB state stays in the 256 MB Infinity Cache
    between steps, so the warm figure can pass the HBM peak; `cold_step_us` is the
    median of single steps each after a 512 MB cache flush."""
    import torch

    import kda_inputs
    import kimi_delta_attention_chunk_amd as kda

    bf = torch.bfloat16
    raw = kda_inputs.draw_decode(seed, steps, B, H, dk, dv)
    q, k, v = (raw[x].to(bf).to(dev) for x in ("q_raw", "k_raw", "v"))
    f, b, A_log, dtb = (raw[x].to(dev) for x in ("f", "b", "A_log", "dt_bias"))
    h = raw["h"].to(dev)
    o = torch.empty((steps, B, H, dv), dtype=bf, device=dev)
    scale = dk ** -0.5
    flags = dict(A_log=A_log, dt_bias=dtb, l2norm_qk=True, gate_in_kernel=True, beta_logits=True)

    def one(t):
        kda.step(q[t], k[t], v[t], f[t], b[t], h, scale, out=o[t], **flags)

    for t in range(8):
        one(t)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(steps):
            one(t)
    ms = timed_ms(graph.replay, 5, warm=1)
    per = ms * 1e3 / steps
    nbytes = B * H * (2 * dk * dv * 4 + 2 * 2 * dk + 2 * dv + 4 * dk + 4 + 2 * dv)
    buf = torch.empty(512 << 18, dtype=torch.float32, device=dev)
    cold = []
    for t in range(21):
        buf.fill_(1.0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        one(t)
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    cold.sort()
    del graph, buf
    # a stack of layers: each layer's output is the next layer's v (written straight into
    # it), every (token, layer) step in one graph; each layer has its own state, so the
    # stack's states (L x 16.8 MB) no longer stay in the Infinity Cache between steps
    # (12 layers, 201 MB, partly; 24 layers, 403 MB, not at all: each step streams its
    # state from HBM)
    def stack_us(L, lsteps):
        hs = [h.clone() for _ in range(L)]
        outs = [torch.empty((lsteps, B, H, dv), dtype=bf, device=dev) for _ in range(L)]

        def stack():
            for t in range(lsteps):
                for l in range(L):
                    vin = v[t] if l == 0 else outs[l - 1][t]
                    kda.step(q[t], k[t], vin, f[t], b[t], hs[l], scale, out=outs[l][t], **flags)

        stack()
        torch.cuda.synchronize()
        lgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(lgraph):
            stack()
        us = timed_ms(lgraph.replay, 5, warm=1) * 1e3 / (L * lsteps)
        del lgraph, hs, outs
        return us

    L, lsteps = 12, 32
    lper = stack_us(L, lsteps)
    L2, lsteps2 = 24, 16
    lper2 = stack_us(L2, lsteps2)
    return {"workload": "kda_step decode: B=%d H=%d dk=%d dv=%d, %d steps in one HIP graph" % (B, H, dk, dv, steps),
            "us_per_step": per, "tokens_per_s": B / (per * 1e-6), "algorithmic_bytes_per_step": nbytes,
            "effective_GBs": nbytes / (per * 1e-6) / 1e9, "frac_of_8TBs": nbytes / (per * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "roofline_us": nbytes / (PEAK_HBM_GBS * 1e9) * 1e6, "cold_step_us": cold[len(cold) // 2],
            "layer_stack": {"layers": L, "tokens": lsteps, "us_per_layer_step": lper,
                            "effective_GBs": nbytes / (lper * 1e-6) / 1e9,
                            "frac_of_8TBs": nbytes / (lper * 1e-6) / 1e9 / PEAK_HBM_GBS},
            "layer_stack_from_hbm": {"layers": L2, "tokens": lsteps2, "us_per_layer_step": lper2,
                                     "effective_GBs": nbytes / (lper2 * 1e-6) / 1e9,
                                     "frac_of_8TBs": nbytes / (lper2 * 1e-6) / 1e9 / PEAK_HBM_GBS}}


def layer_ops_workload(dev, B=16, T=2048, H=8, dk=32, dv=64, W=4, reps=20):
    """The two operations next to KDA in the layer, fwd+bwd at the 300M layer shape, bf16:
    the short convolution over the concatenated q/k/v channels (D = H (2 dk + dv), kernel
    W, SiLU) and the gated output norm over H heads of dv values.  Both are HBM-bound:
    algorithmic bytes = every input read once and every output written once."""
    import torch

    import kimi_delta_attention_chunk_amd as kda

    bf = torch.bfloat16
    g = torch.Generator().manual_seed(9)
    D = H * (2 * dk + dv)
    x = torch.randn(B, T, D, generator=g).to(bf).to(dev)
    w = (torch.randn(D, W, generator=g) * 0.5).to(dev)
    dy = torch.randn(B, T, D, generator=g).to(bf).to(dev)
    o, gate, dyo = (torch.randn(B, T, H, dv, generator=g).to(bf).to(dev) for _ in range(3))
    wt = torch.ones(dv, device=dev)
    ws_c = torch.empty(kda.load_library().kda_conv_bwd_workspace(B, T, D, W), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(kda.load_library().kda_gnorm_bwd_workspace(B * T * H, dv), dtype=torch.uint8, device=dev)
    out = []
    conv_ms = timed_ms(lambda: (kda.conv_fwd(x, w, silu=True),
                                kda.conv_bwd(x, w, dy, silu=True, need_dbias=False, workspace=ws_c)), reps)
    nbytes = 2 * B * T * D * 2 + 3 * B * T * D * 2  # fwd: x, y; bwd: x, dy, dx
    out.append({"workload": "short conv fwd+bwd: [%d, %d, %d] bf16, kernel %d, SiLU" % (B, T, D, W),
                "ms_per_step": conv_ms, "tokens_per_s": B * T / (conv_ms * 1e-3), "algorithmic_bytes": nbytes,
                "achieved_GBs": nbytes / (conv_ms * 1e-3) / 1e9, "bound": "hbm",
                "frac": nbytes / (conv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS})
    gn_ms = timed_ms(lambda: (kda.gnorm_fwd(o, gate, wt), kda.gnorm_bwd(o, gate, wt, dyo, workspace=ws_g)), reps)
    n = B * T * H * dv
    nbytes = 3 * n * 2 + 5 * n * 2  # fwd: o, gate, y; bwd: o, gate, dy, do, dgate
    out.append({"workload": "gated output norm fwd+bwd: [%d, %d, %d, %d] bf16" % (B, T, H, dv),
                "ms_per_step": gn_ms, "tokens_per_s": B * T / (gn_ms * 1e-3), "algorithmic_bytes": nbytes,
                "achieved_GBs": nbytes / (gn_ms * 1e-3) / 1e9, "bound": "hbm",
                "frac": nbytes / (gn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS})
    return out


def long_document_workload(dev, T=65536, H=8, dk=32, dv=64, seg=1024, reps=5, seed=5):
    """One document of T tokens, fwd+bwd: directly (its state pass is H * dv / 32 chains of
    T / 64 chunks each) and segment-parallel on the same GPU (T / seg segments run from a zero
    state, chained by their transition matrices, then rerun from their true states; the
    context-parallel scheme, with the ranks' segments on one device)."""
    import torch

    import kda_inputs
    import kimi_delta_attention_chunk_amd as kda

    bf = torch.bfloat16
    raw = kda_inputs.draw(seed, 1, T, H, dk, dv, h0_std=0.1, upstream=True, dhT=True)
    q, k, v, do = (raw[x].to(bf).to(dev) for x in ("q_raw", "k_raw", "v", "do"))
    f, b, A_log, dtb = (raw[x].to(dev) for x in ("f", "b", "A_log", "dt_bias"))
    h0, dhT = raw["h0"].to(dev), raw["dhT"].to(dev)
    scale = dk ** -0.5
    flags = dict(A_log=A_log, dt_bias=dtb, l2norm_qk=True, gate_in_kernel=True, beta_logits=True)
    args = (q, k, v, f, b)
    ws = torch.empty(kda.workspace_bytes((1, T, H, dk), dv, 1, True), dtype=torch.uint8, device=dev)

    def direct():
        kda.fwd(*args, scale, h0=h0, workspace=ws, save_for_bwd=True, **flags)
        kda.bwd(*args, scale, do, h0=h0, dhT=dhT, workspace=ws, fwd_saved=True, **flags)

    R = T // seg
    cu = torch.arange(0, T + 1, seg, dtype=torch.int32, device=dev)
    plan = kda.plan_varlen(cu, T)
    wsc = torch.empty(kda.workspace_bytes((1, T, H, dk), dv, R, True), dtype=torch.uint8, device=dev)
    pk = dict(cu_seqlens=cu, plan=plan, **flags)

    def segmented():
        # chunk quantities formed once; the second state passes and the maps reuse them
        _, c = kda.fwd(*args, scale, workspace=wsc, save_for_bwd=True, **pk)
        M = kda.segment_maps(*args, workspace=wsc, fwd_saved=True, **pk)
        h_in, _ = kda.state_scan(M, c, h0[0])
        kda.fwd(*args, scale, h0=h_in, workspace=wsc, save_for_bwd=True, fwd_saved=True, **pk)
        e = kda.bwd(*args, scale, do, h0=h_in, workspace=wsc, fwd_saved=True, dh0_only=True, **pk)["dh0"]
        D, _ = kda.state_scan(M, e, dhT[0], transpose=True)
        kda.bwd(*args, scale, do, h0=h_in, dhT=D, workspace=wsc, fwd_saved=True, **pk)

    ms_d = timed_ms(direct, reps, warm=1)
    ms_s = timed_ms(segmented, reps, warm=1)
    return {"workload": "KDA fwd+bwd, one document of %d tokens, H=%d dk=%d dv=%d, bf16" % (T, H, dk, dv),
            "direct_ms": ms_d, "direct_tokens_per_s": T / (ms_d * 1e-3),
            "segment_parallel_ms": ms_s, "segment_parallel_tokens_per_s": T / (ms_s * 1e-3),
            "segments": R, "segment_tokens": seg}


def other_workloads(dev):
    """The decode step, the packed 65,536-token row, the dk = dv = 128 heads, one long
    document (dk = 32 and dk = dv = 128) in one pass and segment-parallel, and the short
    convolution and gated output norm of the layer."""
    return layer_ops_workload(dev) + [
        decode_workload(dev),
        fwd_bwd_workload("KDA fwd+bwd, one packed row of 65536 tokens (geometric document lengths, "
                         "mean 512), per-document h0 and dhT", dev, 1, 65536, 8, 32, 64, 3, packed=True),
        fwd_bwd_workload("KDA fwd+bwd, larger heads: B=2 T=8192 H=16 dk=dv=128", dev, 2, 8192, 16, 128, 128, 4),
        long_document_workload(dev),
        long_document_workload(dev, T=16384, H=16, dk=128, dv=128, seg=1024),
    ]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--seq", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cache-flushed median and the B=128 run (keeps profiler traces to the timed steps)")
    ap.add_argument("--out-dtype", choices=["bf16", "fp32"], default="bf16")
    ap.add_argument("--only-extras", action="store_true",
                    help="run only the other workloads (decode, packed row, dk=128) and print them")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the operator shards by sequence and head with no communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_mb:
        copy_calibration(args.copy_mb)
        return

    import torch

    import kda_inputs
    import kimi_delta_attention_chunk_amd as kda

    B, T, H, dk, dv = args.batch, args.seq, 8, 32, 64
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only_extras:
        for w in other_workloads(dev):
            print(json.dumps(w), flush=True)
        return
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

    # timed region: K steps with nothing else on the stream
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    # per-kernel durations: the same K steps again, each launch between a pair of HIP
    # events on its own stream (the events are kept out of the headline loop above)
    kda.timing_enable(True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_instrumented = ev0.elapsed_time(ev1) / args.steps
    per_kernel = kda.timing_collect()
    kda.timing_enable(False)

    tokens = B * T
    value = tokens / (ms * 1e-3)
    work = kda_work(B, T, H, dk, dv)
    kernels = {name: {"launches_per_step": n / args.steps, "avg_us": 1e3 * tot / n,
                      "share": tot / (ms_instrumented * args.steps)} for name, (n, tot) in per_kernel.items()}
    dom = max(per_kernel, key=lambda nm: per_kernel[nm][1])
    n_dom, tot_dom = per_kernel[dom]
    avg_s = tot_dom / n_dom * 1e-3
    bytes_dom, flops_dom = work.get(dom, (0.0, 0.0))
    # the binding roofline of the dominant kernel: its bytes at HBM peak against its
    # products, issued as bf16 MFMA three times each (hi/lo split), at the bf16 peak
    t_hbm = bytes_dom / (PEAK_HBM_GBS * 1e9)
    t_mfma = 3 * flops_dom / (PEAK_BF16_TFLOPS * 1e12)
    traffic = measured_traffic(dom)
    if t_hbm >= t_mfma:
        achieved = bytes_dom / avg_s / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}
    else:
        achieved = 3 * flops_dom / avg_s / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic}
    roof.update({"avg_us": avg_s * 1e6, "algorithmic_bytes": bytes_dom, "flops": flops_dom,
                 "fp32_equiv_tflops": flops_dom / avg_s / 1e12})
    step_bytes = sum(b for b, _ in work.values())
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
        "instrumented_ms_per_step": ms_instrumented,
    }
    if not args.no_extras:
        line["flushed"] = flushed_median(step, dev, reps=21)
        line["flushed"]["tokens_per_s"] = B * T / (line["flushed"]["median_ms"] * 1e-3)
        line["secondary_B128"] = secondary_run(q, k, v, f, b, do, scale, flags, B, T, H, dk, dv, dev)
        line["other_workloads"] = other_workloads(dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(raw, T, H, dk, dv)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
