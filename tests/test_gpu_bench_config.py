"""Parity of the exact launch configurations bench.py times, element by element
against the oracle: the 300M layer shape (B=16, T=2048, H=8, dk=32, dv=64) and the
larger-head workload (B=2, T=8192, H=16, dk=dv=128), both with bf16 q/k/v, fused
preparation, one workspace with save-for-backward and bf16 outputs.

bf16 outputs: the same calls with fp32 outputs are checked against the oracle at
the bf16-input bound, and the bf16 outputs must be their round-to-nearest-even,
bit for bit."""
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunk_amd as kda
from cases import check_close, oracle_bwd_raw, oracle_fwd_raw, raw_inputs, to_dev

pytestmark = pytest.mark.gpu


def _run(d, out_dtype):
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    kw = dict(A_log=d["A_log"], dt_bias=d["dt_bias"], l2norm_qk=True, gate_in_kernel=True,
              beta_logits=True, out_dtype=out_dtype)
    ws = torch.empty(kda.workspace_bytes((B, T, H, dk), dv, B, True), dtype=torch.uint8, device="cuda")
    o, hT = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dk ** -0.5, workspace=ws,
                    save_for_bwd=True, **kw)
    g = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dk ** -0.5, d["do"], workspace=ws,
                fwd_saved=True, need_dh0=False, **kw)
    return o, hT, g


@pytest.mark.parametrize("shape,seed", [((16, 2048, 8, 32, 64), 1), ((2, 8192, 16, 128, 128), 4)],
                         ids=["layer300M_B16", "dk128_B2_T8192_H16"])
def test_bench_configuration(shape, seed):
    B, T, H, dk, dv = shape
    raw = kda_inputs.draw(seed, B, T, H, dk, dv, upstream=True)   # the bench's own draw
    rin = raw_inputs(raw, torch.bfloat16)
    d = to_dev(rin)
    o32, h32, g32 = _run(d, torch.float32)
    o16, h16, g16 = _run(d, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(h32, h16)
    for nm in ("dq", "dk", "dv"):
        assert torch.equal(g32[nm].to(torch.bfloat16), g16[nm]), nm
    for nm in ("dg", "dbeta", "dA_log", "ddt_bias"):
        assert torch.equal(g32[nm], g16[nm]), nm
    scale = dk ** -0.5
    oref, href = oracle_fwd_raw(rin, scale)
    check_close("o", o32, oref, torch.bfloat16)
    check_close("hT", h32, href, torch.bfloat16)
    gref = oracle_bwd_raw(rin, scale)
    for nm in ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "ddt_bias"):
        check_close(nm, g32[nm], gref[nm], torch.bfloat16)
