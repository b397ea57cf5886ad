"""kda_fwd_noalloc -- the forward on the library's fixed per-GPU scratch, for callers
that cannot allocate -- against kda_fwd with a caller workspace, through the C ABI:
two calls in a row (the second on a smaller problem, so it runs on what the first
left in the scratch), each equal to kda_fwd bit for bit and within the oracle bound."""
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunk_amd as kda
from cases import check_close, oracle_fwd, oracle_fwd_raw, prepared, raw_inputs, to_dev

pytestmark = pytest.mark.gpu


def test_noalloc_forward_equals_workspace_forward_twice():
    dev = torch.device("cuda:0")
    # first call: 4 x 2048 tokens, 8 heads, bf16 raw inputs with the fused preparation
    raw = kda_inputs.draw(90, 4, 2048, 8, 32, 64, h0_std=0.1, a_log_range=kda_inputs.A_LOG_RANGE_WEAK)
    rin = raw_inputs(raw, torch.bfloat16)
    d = to_dev(rin, dev)
    kw = dict(h0=d["h0"], A_log=d["A_log"], dt_bias=d["dt_bias"], l2norm_qk=True, gate_in_kernel=True,
              beta_logits=True, out_dtype=torch.float32)
    o_ref, h_ref = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], 32 ** -0.5, **kw)
    o, hT = kda.fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], 32 ** -0.5,
                            hT=torch.empty_like(h_ref), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
    oref, href = oracle_fwd_raw(rin, 32 ** -0.5)
    check_close("o (first call)", o, oref, torch.bfloat16)
    check_close("hT (first call)", hT, href, torch.bfloat16)

    # second call, smaller: 1 x 300 tokens, 2 heads, fp32 prepared inputs, partial last chunk
    inp, _ = prepared(91, 1, 300, 2, 32, 64, torch.float32, weak=True, h0_std=0.1)
    d2 = to_dev(inp, dev)
    o_ref2, h_ref2 = kda.fwd(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], 32 ** -0.5, h0=d2["h0"])
    o2, hT2 = kda.fwd_noalloc(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], 32 ** -0.5, h0=d2["h0"],
                              hT=torch.empty_like(h_ref2))
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref2) and torch.equal(hT2, h_ref2)
    oref2, href2 = oracle_fwd(inp, 32 ** -0.5)
    check_close("o (second call)", o2, oref2, torch.float32)
    check_close("hT (second call)", hT2, href2, torch.float32)


def test_noalloc_forward_rejects_oversized_problem():
    inp, _ = prepared(92, 16, 2048, 8, 32, 64, torch.bfloat16)
    d = to_dev(inp)
    with pytest.raises(kda.KdaError) as ei:
        kda.fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], 32 ** -0.5)
    assert ei.value.status == 2  # KDA_ERR_UNSUPPORTED
