"""Empty inputs (no tokens, no rows): states pass through unchanged (hT = h0,
dh0 = dhT), parameter gradients are zeros, nothing else is touched."""
import pytest
import torch

import kimi_delta_attention_chunk_amd as kda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dk,dv", [(32, 64), (128, 128)])
def test_fwd_bwd_without_tokens(dk, dv):
    B, H = 2, 3
    g = torch.Generator().manual_seed(0)
    bf = torch.bfloat16
    q, k = (torch.empty((B, 0, H, dk), dtype=bf, device="cuda") for _ in range(2))
    v, do = (torch.empty((B, 0, H, dv), dtype=bf, device="cuda") for _ in range(2))
    f = torch.empty((B, 0, H, dk), device="cuda")
    b = torch.empty((B, 0, H), device="cuda")
    h0 = torch.randn((B, H, dk, dv), generator=g).cuda()
    dhT = torch.randn((B, H, dk, dv), generator=g).cuda()
    kw = dict(A_log=torch.zeros(H, device="cuda"), dt_bias=torch.zeros((H, dk), device="cuda"), l2norm_qk=True,
              gate_in_kernel=True, beta_logits=True)
    o, hT = kda.fwd(q, k, v, f, b, 0.2, h0=h0, **kw)
    gr = kda.bwd(q, k, v, f, b, 0.2, do, h0=h0, dhT=dhT, **kw)
    torch.cuda.synchronize()
    assert o.shape == (B, 0, H, dv) and gr["dq"].shape == (B, 0, H, dk)
    assert torch.equal(hT, h0)
    assert torch.equal(gr["dh0"], dhT)
    assert not torch.any(gr["dA_log"]) and not torch.any(gr["ddt_bias"])


def test_conv_and_gnorm_without_rows():
    D, W = 64, 4
    x = torch.empty((1, 0, D), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((D, W), device="cuda")
    bias = torch.randn(D, device="cuda")
    y = kda.conv_fwd(x, w, bias, silu=True)
    r = kda.conv_bwd(x, w, torch.empty_like(x), bias, silu=True)
    o = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    wt = torch.randn(64, device="cuda")
    yn = kda.gnorm_fwd(o, torch.empty_like(o), wt)
    rn = kda.gnorm_bwd(o, torch.empty_like(o), wt, torch.empty_like(o))
    torch.cuda.synchronize()
    assert y.shape == (1, 0, D) and yn.shape == (0, 4, 64)
    assert not torch.any(r["dw"]) and not torch.any(r["dbias"]) and r["dx"].shape == (1, 0, D)
    assert not torch.any(rn["dweight"]) and rn["do"].shape == (0, 4, 64)
