"""Decode step (kda_step) against the oracle's token step."""
import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunk_amd as kda
import oracle
from cases import check_close, to_np

pytestmark = pytest.mark.gpu


def _decode_inputs(seed, steps, B, H, dk, dv, dtype, weak=False):
    raw = kda_inputs.draw_decode(seed, steps, B, H, dk, dv,
                                 a_log_range=kda_inputs.A_LOG_RANGE_WEAK if weak else kda_inputs.A_LOG_RANGE)
    qh, kh, g, beta = oracle.prep_forward(raw["q_raw"], raw["k_raw"], raw["f"], raw["A_log"],
                                          raw["dt_bias"], raw["b"])
    inp = dict(q=torch.tensor(qh, dtype=torch.float32).to(dtype),
               k=torch.tensor(kh, dtype=torch.float32).to(dtype), v=raw["v"].to(dtype),
               g=torch.tensor(g, dtype=torch.float32), beta=torch.tensor(beta, dtype=torch.float32))
    return inp, raw


@pytest.mark.parametrize("dtype,dk,dv", [(torch.float32, 32, 64), (torch.bfloat16, 32, 64),
                                         (torch.bfloat16, 128, 128), (torch.float32, 64, 64),
                                         (torch.bfloat16, 64, 64), (torch.float32, 128, 128)])
def test_step_matches_oracle(dtype, dk, dv):
    B, H, steps = 64, 4, 24
    inp, raw = _decode_inputs(3, steps, B, H, dk, dv, dtype, weak=True)
    dev = {k: v.cuda() for k, v in inp.items()}
    h = raw["h"].clone().cuda()
    href = to_np(raw["h"])
    scale = dk ** -0.5
    for t in range(steps):
        o = kda.step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], h, scale,
                     out_dtype=torch.float32)
        oref, href = oracle.step(to_np(inp["q"][t]), to_np(inp["k"][t]), to_np(inp["v"][t]),
                                 to_np(inp["g"][t]), to_np(inp["beta"][t]), scale, href)
        check_close("o[%d]" % t, o, oref, dtype)
    check_close("h", h, href, dtype)


def test_step_decode_config_shape_with_prep():
    """B=256, H=8, dk=32, dv=64 (the decode configuration), fused preparation, bf16."""
    B, H, dk, dv, steps = 256, 8, 32, 64, 16
    raw = kda_inputs.draw_decode(2, steps, B, H, dk, dv)
    dt = torch.bfloat16
    q, k, v = (raw[x].to(dt).cuda() for x in ("q_raw", "k_raw", "v"))
    f, b = raw["f"].cuda(), raw["b"].cuda()
    A_log, dtb = raw["A_log"].cuda(), raw["dt_bias"].cuda()
    h = raw["h"].clone().cuda()
    href = to_np(raw["h"])
    scale = dk ** -0.5
    for t in range(steps):
        o = kda.step(q[t], k[t], v[t], f[t], b[t], h, scale, A_log=A_log, dt_bias=dtb, l2norm_qk=True,
                     gate_in_kernel=True, beta_logits=True, out_dtype=torch.float32)
        qh, kh, g, beta = oracle.prep_forward(to_np(q[t]), to_np(k[t]), to_np(f[t]), to_np(A_log),
                                              to_np(dtb), to_np(b[t]))
        oref, href = oracle.step(qh, kh, to_np(v[t]), g, beta, scale, href)
        check_close("o[%d]" % t, o, oref, dt)
    check_close("h", h, href, dt)


def test_step_decode_config_1000_steps():
    """The decode configuration as specified: B=256, H=8, dk=32, dv=64, bf16 q/k/v, prepared
    fp32 g and beta (default distributions, seed 2), fp32 state ~ N(0, 0.1) updated in place,
    1000 consecutive steps.  The oracle runs the same 1000-step chain in fp64 from the same
    initial state (it never sees a GPU value); every 50th output and the final state are
    compared at the bf16-input bound."""
    B, H, dk, dv, steps = 256, 8, 32, 64, 1000
    inp, raw = _decode_inputs(2, steps, B, H, dk, dv, torch.bfloat16)
    dev = {k: v.cuda() for k, v in inp.items()}
    h = raw["h"].clone().cuda()
    href = to_np(raw["h"])
    scale = dk ** -0.5
    checked = 0
    for t in range(steps):
        o = kda.step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], h, scale,
                     out_dtype=torch.float32)
        oref, href = oracle.step(to_np(inp["q"][t]), to_np(inp["k"][t]), to_np(inp["v"][t]),
                                 to_np(inp["g"][t]), to_np(inp["beta"][t]), scale, href)
        if t % 50 == 49:
            check_close("o[%d]" % t, o, oref, torch.bfloat16)
            checked += 1
    check_close("h after %d steps" % steps, h, href, torch.bfloat16)
    assert checked == steps // 50


def test_step_continuation_is_bitwise():
    """500 + 500 steps with the state copied out in between equal 1000 straight steps."""
    B, H, dk, dv, steps = 32, 8, 32, 64, 1000
    inp, raw = _decode_inputs(4, steps, B, H, dk, dv, torch.bfloat16)
    dev = {k: v.cuda() for k, v in inp.items()}
    scale = dk ** -0.5
    h1 = raw["h"].clone().cuda()
    for t in range(steps):
        o1 = kda.step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], h1, scale)
    h2 = raw["h"].clone().cuda()
    for t in range(500):
        kda.step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], h2, scale)
    saved = h2.cpu().clone()
    h3 = saved.cuda()
    for t in range(500, steps):
        o3 = kda.step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], h3, scale)
    torch.cuda.synchronize()
    assert torch.equal(h1, h3)
    assert torch.equal(o1, o3)


def test_step_bf16_output_is_rounded_fp32_output():
    B, H, dk, dv = 16, 8, 32, 64
    inp, raw = _decode_inputs(5, 1, B, H, dk, dv, torch.bfloat16)
    dev = {k: v[0].cuda() for k, v in inp.items()}
    ha, hb = raw["h"].clone().cuda(), raw["h"].clone().cuda()
    oa = kda.step(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], ha, 0.17, out_dtype=torch.float32)
    ob = kda.step(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], hb, 0.17, out_dtype=torch.bfloat16)
    assert torch.equal(oa.to(torch.bfloat16), ob)
    assert torch.equal(ha, hb)


def test_step_graph_replay_equals_eager():
    """Consecutive decode steps captured in one HIP graph: every replay reproduces the
    eager steps bit for bit (outputs of every step and the final state), with other
    eager work and synchronisations between the replays."""
    B, H, dk, dv, steps = 64, 8, 32, 64, 12
    raw = kda_inputs.draw_decode(5, steps, B, H, dk, dv)
    dt = torch.bfloat16
    q, k, v = (raw[x].to(dt).cuda() for x in ("q_raw", "k_raw", "v"))
    f, b = raw["f"].cuda(), raw["b"].cuda()
    A_log, dtb = raw["A_log"].cuda(), raw["dt_bias"].cuda()
    flags = dict(A_log=A_log, dt_bias=dtb, l2norm_qk=True, gate_in_kernel=True, beta_logits=True)
    scale = dk ** -0.5
    h_init = raw["h"].cuda()

    h_eager = h_init.clone()
    o_eager = torch.empty((steps, B, H, dv), dtype=dt, device="cuda")
    for t in range(steps):
        kda.step(q[t], k[t], v[t], f[t], b[t], h_eager, scale, out=o_eager[t], **flags)
    torch.cuda.synchronize()

    h = h_init.clone()
    o = torch.empty_like(o_eager)
    kda.step(q[0], k[0], v[0], f[0], b[0], h.clone(), scale, **flags)  # warm the launch path
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(steps):
            kda.step(q[t], k[t], v[t], f[t], b[t], h, scale, out=o[t], **flags)
    other = h_init.clone()
    for rep in range(3):
        h.copy_(h_init)
        o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), "replay %d: outputs differ from the eager steps" % rep
        assert torch.equal(h, h_eager), "replay %d: state differs from the eager steps" % rep
        kda.step(q[rep], k[rep], v[rep], f[rep], b[rep], other, scale, **flags)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_multi_layer_decode_graph(dtype):
    """Decode through a stack of layers, the output of each layer's step being the v input
    of the next (written straight into it), every (token, layer) step captured in one HIP
    graph: the eager chain matches the oracle's chain, and every replay reproduces the
    eager chain bit for bit."""
    L, B, H, dk, dv, steps = 3, 32, 4, 32, 64, 5
    scale = dk ** -0.5
    layers = [kda_inputs.draw_decode(40 + l, steps, B, H, dk, dv, a_log_range=kda_inputs.A_LOG_RANGE_WEAK)
              for l in range(L)]
    dev = []
    for raw in layers:
        dev.append(dict(q=raw["q_raw"].to(dtype).cuda(), k=raw["k_raw"].to(dtype).cuda(), f=raw["f"].cuda(),
                        b=raw["b"].cuda(), h=raw["h"].cuda(),
                        flags=dict(A_log=raw["A_log"].cuda(), dt_bias=raw["dt_bias"].cuda(), l2norm_qk=True,
                                   gate_in_kernel=True, beta_logits=True)))
    v0 = layers[0]["v"].to(dtype).cuda()

    def run(hs, outs, check_rne=False):
        for t in range(steps):
            for l, d in enumerate(dev):
                vin = v0[t] if l == 0 else outs[l - 1][t]
                if check_rne:  # the same call with an fp32 output, on a copy of the state
                    o32 = kda.step(d["q"][t], d["k"][t], vin, d["f"][t], d["b"][t], hs[l].clone(), scale,
                                   out_dtype=torch.float32, **d["flags"])
                kda.step(d["q"][t], d["k"][t], vin, d["f"][t], d["b"][t], hs[l], scale, out=outs[l][t],
                         **d["flags"])
                if check_rne:
                    assert torch.equal(outs[l][t], o32.to(dtype)), "t=%d layer=%d: not RNE(fp32)" % (t, l)

    h_e = [d["h"].clone() for d in dev]
    o_e = [torch.empty((steps, B, H, dv), dtype=dtype, device="cuda") for _ in range(L)]
    run(h_e, o_e, check_rne=dtype == torch.bfloat16)
    torch.cuda.synchronize()

    # the oracle's chain, in fp64 throughout (the GPU's outputs are never fed to it)
    href = [to_np(raw["h"]) for raw in layers]
    prev = None
    for t in range(steps):
        for l, raw in enumerate(layers):
            qh, kh, g, beta = oracle.prep_forward(to_np(dev[l]["q"][t]), to_np(dev[l]["k"][t]), to_np(raw["f"][t]),
                                                  to_np(raw["A_log"]), to_np(raw["dt_bias"]), to_np(raw["b"][t]))
            vin = to_np(v0[t]) if l == 0 else prev
            prev, href[l] = oracle.step(qh, kh, vin, g, beta, scale, href[l])
            if dtype == torch.float32:
                check_close("o[t=%d, layer=%d]" % (t, l), o_e[l][t], prev, dtype)
            else:
                # a bf16 output is the rounding of the fp32 one (checked above): the bound of an
                # fp32 output plus its own final rounding, at most 2^-8 of each value (bf16 keeps 8 significant bits)
                got = to_np(o_e[l][t])
                excess = np.max(np.abs(got - prev) - 2.0 ** -8 * np.abs(prev))
                assert excess <= 2e-2 * np.sqrt(np.mean(prev ** 2)), "o[t=%d, layer=%d]" % (t, l)
    for l in range(L):
        check_close("h[layer=%d]" % l, h_e[l], href[l], dtype)

    hs = [d["h"].clone() for d in dev]
    outs = [torch.empty_like(o) for o in o_e]
    run([h.clone() for h in hs], [torch.empty_like(o) for o in o_e])  # warm the launch path
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(hs, outs)
    for rep in range(3):
        for l in range(L):
            hs[l].copy_(dev[l]["h"])
            outs[l].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(outs[l], o_e[l]), "replay %d: layer %d outputs differ" % (rep, l)
            assert torch.equal(hs[l], h_e[l]), "replay %d: layer %d state differs" % (rep, l)
