"""A packed row past 2^31 elements: H=32, dk=32, dv=64 and 2,228,261 tokens, so q, k
and the log-decay hold T*H*dk > 2^31 values and v, o, dO twice that, and the
workspace runs to tens of GB.  Every offset of the row is 64-bit on the device
side; this checks it where 32-bit arithmetic would wrap.  fwd+bwd with the fused
preparation, bf16 inputs; the first document and the last three (which lie past
element 2^31 of q) are compared with the oracle run on each document alone.

Outputs in fp32 (checked at the bf16-input bound).  Runs last among the GPU tests
(it holds about 190 GB of device memory while it runs and frees it at the end)."""
import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunk_amd as kda
import oracle
from cases import check_close, to_np

pytestmark = pytest.mark.gpu


def test_packed_row_past_2e31_elements():
    free, _ = torch.cuda.mem_get_info()
    if free < (200 << 30):
        pytest.skip("needs about 200 GB of free device memory (%.0f GB free)" % (free / 2 ** 30))
    H, dk, dv = 32, 32, 64
    lens = [4096] + [65536] * 33 + [57343, 4096, 37, 1]
    T = int(sum(lens))
    assert T * H * dk > 2 ** 31
    N = len(lens)
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    assert cu_h[-3] * H * dk > 2 ** 31  # the last three documents start past element 2^31 of q
    d = kda_inputs.draw_device(21, 1, T, H, dk, dv, "cuda", n_states=N, h0_std=0.1, upstream=True, dhT=True)
    cu = torch.tensor(cu_h, dtype=torch.int32, device="cuda")
    plan = kda.plan_varlen(cu, T)
    scale = dk ** -0.5
    kw = dict(A_log=d["A_log"], dt_bias=d["dt_bias"], l2norm_qk=True, gate_in_kernel=True, beta_logits=True)
    args = (d["q_raw"], d["k_raw"], d["v"], d["f"], d["b"])
    ws = torch.empty(kda.workspace_bytes((1, T, H, dk), dv, N, True), dtype=torch.uint8, device="cuda")
    o, hT = kda.fwd(*args, scale, h0=d["h0"], cu_seqlens=cu, plan=plan, workspace=ws, save_for_bwd=True,
                    out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    check = [0, N - 3, N - 2, N - 1]
    o_s = {n: o[:, cu_h[n]:cu_h[n + 1]].cpu() for n in check}
    del o
    g = kda.bwd(*args, scale, d["do"], h0=d["h0"], dhT=d["dhT"], cu_seqlens=cu, plan=plan, workspace=ws,
                fwd_saved=True, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    del ws
    for n in check:
        a, b = int(cu_h[n]), int(cu_h[n + 1])
        sl = lambda x: to_np(x[:, a:b])
        q_raw, k_raw, f, bl = sl(d["q_raw"]), sl(d["k_raw"]), sl(d["f"]), sl(d["b"])
        A_log, dtb = to_np(d["A_log"]), to_np(d["dt_bias"])
        qh, kh, gg, beta = oracle.prep_forward(q_raw, k_raw, f, A_log, dtb, bl)
        h0 = to_np(d["h0"][n:n + 1])
        dhT = to_np(d["dhT"][n:n + 1])
        oref, href = oracle.forward(qh, kh, sl(d["v"]), gg, beta, scale, h0=h0)
        check_close("o[doc %d]" % n, o_s[n], oref, torch.bfloat16)
        check_close("hT[doc %d]" % n, hT[n:n + 1], href, torch.bfloat16)
        gr = oracle.backward(qh, kh, sl(d["v"]), gg, beta, scale, sl(d["do"]), h0=h0, dhT=dhT)
        pr = oracle.prep_backward(q_raw, k_raw, f, A_log, dtb, bl, gr["dq"], gr["dk"], gr["dg"], gr["dbeta"])
        check_close("dq[doc %d]" % n, g["dq"][:, a:b], pr["dq"], torch.bfloat16)
        check_close("dk[doc %d]" % n, g["dk"][:, a:b], pr["dk"], torch.bfloat16)
        check_close("dv[doc %d]" % n, g["dv"][:, a:b], gr["dv"], torch.bfloat16)
        check_close("df[doc %d]" % n, g["dg"][:, a:b], pr["df"], torch.bfloat16)
        check_close("db[doc %d]" % n, g["dbeta"][:, a:b], pr["db"], torch.bfloat16)
        check_close("dh0[doc %d]" % n, g["dh0"][n:n + 1], gr["dh0"], torch.bfloat16)
    del g, d
    torch.cuda.empty_cache()
