"""Short convolution and gated output norm (kda_conv_*, kda_gnorm_*) through the C
ABI against the fp64 oracle (oracle/ops.py): fp32 inputs within a normwise
relative error of 1e-4, bf16 inputs within 2e-2 * rms(reference), the oracle fed
the same bf16-rounded values."""
import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunk_amd as kda
from cases import check_close, to_np
from oracle import ops

pytestmark = pytest.mark.gpu


def _conv_case(seed, B, T, D, W, dtype, packed_lens=None, bias=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, T, D, generator=g).to(dtype)
    w = (torch.randn(D, W, generator=g) * 0.5).float()
    b = (torch.randn(D, generator=g) * 0.1).float() if bias else None
    dy = torch.randn(B, T, D, generator=g).to(dtype)
    cu = None
    if packed_lens is not None:
        cu = torch.tensor(np.cumsum([0] + list(packed_lens)), dtype=torch.int32)
    return x, w, b, dy, cu


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("W,silu,bias", [(4, True, True), (4, False, False), (3, True, False), (2, False, True),
                                         (1, True, True)])
def test_conv_dense_matches_oracle(dtype, W, silu, bias):
    # T = 77 is not a multiple of the 16-token run; D = 96 leaves most of a workgroup's channel groups idle
    x, w, b, dy, _ = _conv_case(1, 2, 77, 96, W, dtype, bias=bias)
    dev = lambda t: None if t is None else t.cuda()
    y = kda.conv_fwd(dev(x), dev(w), dev(b), silu=silu, out_dtype=torch.float32)
    gr = kda.conv_bwd(dev(x), dev(w), dev(dy), dev(b), silu=silu, out_dtype=torch.float32, need_dbias=bias)
    torch.cuda.synchronize()
    xr, dyr = to_np(x), to_np(dy)
    check_close("y", y, ops.conv_fwd(xr, to_np(w), None if b is None else to_np(b), silu=silu), dtype)
    dx, dw, db = ops.conv_bwd(xr, to_np(w), dyr, None if b is None else to_np(b), silu=silu)
    check_close("dx", gr["dx"], dx, dtype)
    check_close("dw", gr["dw"], dw, dtype)
    if bias:
        check_close("dbias", gr["dbias"], db, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_conv_packed_row_resets_at_documents(dtype):
    # length-1 documents, a document shorter than the window, runs crossing boundaries
    lens = [1, 2, 17, 1, 40, 3, 1, 30, 16, 5]
    x, w, b, dy, cu = _conv_case(2, 1, sum(lens), 64, 4, dtype, packed_lens=lens)
    y = kda.conv_fwd(x.cuda(), w.cuda(), b.cuda(), cu.cuda(), silu=True, out_dtype=torch.float32)
    gr = kda.conv_bwd(x.cuda(), w.cuda(), dy.cuda(), b.cuda(), cu.cuda(), silu=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    c = cu.numpy()
    check_close("y", y, ops.conv_fwd(to_np(x), to_np(w), to_np(b), c, silu=True), dtype)
    dx, dw, db = ops.conv_bwd(to_np(x), to_np(w), to_np(dy), to_np(b), c, silu=True)
    check_close("dx", gr["dx"], dx, dtype)
    check_close("dw", gr["dw"], dw, dtype)
    check_close("dbias", gr["dbias"], db, dtype)
    # packed = separate runs, bit for bit, document by document
    for n in range(len(lens)):
        a, e = int(c[n]), int(c[n + 1])
        ys = kda.conv_fwd(x[:, a:e].contiguous().cuda(), w.cuda(), b.cuda(), silu=True, out_dtype=torch.float32)
        gs = kda.conv_bwd(x[:, a:e].contiguous().cuda(), w.cuda(), dy[:, a:e].contiguous().cuda(), b.cuda(),
                          silu=True, out_dtype=torch.float32)
        assert torch.equal(ys, y[:, a:e]), n
        assert torch.equal(gs["dx"], gr["dx"][:, a:e]), n


def test_conv_layer_shape_bf16():
    """The layer's convolution: B=16 rows of 2048 tokens, D = 2*256 + 512 = 1024 channels
    (q, k, v of 8 heads), kernel 4, SiLU; the oracle on the whole tensor."""
    B, T, D, W = 16, 2048, 1024, 4
    x, w, b, dy, _ = _conv_case(3, B, T, D, W, torch.bfloat16, bias=False)
    xc, wc, dyc = x.cuda(), w.cuda(), dy.cuda()
    # the arithmetic against the oracle at fp32 output; the bf16 output is its rounding, bit for
    # bit (the output's tails reach ~15 rms, where one bf16 rounding alone passes 2e-2 * rms)
    y32 = kda.conv_fwd(xc, wc, silu=True, out_dtype=torch.float32)
    g32 = kda.conv_bwd(xc, wc, dyc, silu=True, need_dbias=False, out_dtype=torch.float32)
    y = kda.conv_fwd(xc, wc, silu=True)
    gr = kda.conv_bwd(xc, wc, dyc, silu=True, need_dbias=False)
    torch.cuda.synchronize()
    check_close("y", y32, ops.conv_fwd(to_np(x), to_np(w), silu=True), torch.bfloat16)
    dx, dw, _ = ops.conv_bwd(to_np(x), to_np(w), to_np(dy), silu=True)
    check_close("dx", g32["dx"], dx, torch.bfloat16)
    check_close("dw", g32["dw"], dw, torch.bfloat16)
    assert torch.equal(y32.to(torch.bfloat16), y) and torch.equal(g32["dx"].to(torch.bfloat16), gr["dx"])
    # deterministic weight gradient
    gr2 = kda.conv_bwd(xc, wc, dyc, silu=True, need_dbias=False)
    assert torch.equal(gr["dw"], gr2["dw"]) and torch.equal(gr["dx"], gr2["dx"])


def test_conv_packed_config_row():
    """One packed row of 65,536 tokens with geometric document lengths (mean 512, with
    length-1 documents), D = 1024, bf16."""
    cu = kda_inputs.geometric_cu_seqlens(3)
    T, D = int(cu[-1]), 1024
    x, w, b, dy, _ = _conv_case(4, 1, T, D, 4, torch.bfloat16)
    y = kda.conv_fwd(x.cuda(), w.cuda(), b.cuda(), cu.cuda(), silu=True, out_dtype=torch.float32)
    gr = kda.conv_bwd(x.cuda(), w.cuda(), dy.cuda(), b.cuda(), cu.cuda(), silu=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    c = cu.numpy()
    check_close("y", y, ops.conv_fwd(to_np(x), to_np(w), to_np(b), c, silu=True), torch.bfloat16)
    dx, dw, db = ops.conv_bwd(to_np(x), to_np(w), to_np(dy), to_np(b), c, silu=True)
    check_close("dx", gr["dx"], dx, torch.bfloat16)
    check_close("dw", gr["dw"], dw, torch.bfloat16)
    check_close("dbias", gr["dbias"], db, torch.bfloat16)


def test_conv_bf16_output_is_rounded_fp32_output():
    x, w, b, dy, _ = _conv_case(5, 2, 100, 128, 4, torch.bfloat16)
    y32 = kda.conv_fwd(x.cuda(), w.cuda(), b.cuda(), silu=True, out_dtype=torch.float32)
    y16 = kda.conv_fwd(x.cuda(), w.cuda(), b.cuda(), silu=True)
    g32 = kda.conv_bwd(x.cuda(), w.cuda(), dy.cuda(), b.cuda(), silu=True, out_dtype=torch.float32)
    g16 = kda.conv_bwd(x.cuda(), w.cuda(), dy.cuda(), b.cuda(), silu=True)
    assert torch.equal(y32.to(torch.bfloat16), y16)
    assert torch.equal(g32["dx"].to(torch.bfloat16), g16["dx"])
    assert torch.equal(g32["dw"], g16["dw"])


# ---------------------------------------------------------------- gated norm
def _gn_case(seed, shape, dtype):
    g = torch.Generator().manual_seed(seed)
    o = torch.randn(*shape, generator=g).to(dtype)
    gate = torch.randn(*shape, generator=g).to(dtype)
    wt = (1.0 + 0.1 * torch.randn(shape[-1], generator=g)).float()
    dy = torch.randn(*shape, generator=g).to(dtype)
    return o, gate, wt, dy


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("dv", [32, 64, 128])
def test_gnorm_matches_oracle(dtype, dv):
    # 1001 rows: the last workgroup is partly empty
    o, gate, wt, dy = _gn_case(6, (7, 11, 13, dv), dtype)
    y = kda.gnorm_fwd(o.cuda(), gate.cuda(), wt.cuda(), out_dtype=torch.float32)
    gr = kda.gnorm_bwd(o.cuda(), gate.cuda(), wt.cuda(), dy.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_close("y", y, ops.gnorm_fwd(to_np(o), to_np(gate), to_np(wt)), dtype)
    do, dg, dw = ops.gnorm_bwd(to_np(o), to_np(gate), to_np(wt), to_np(dy))
    check_close("do", gr["do"], do, dtype)
    check_close("dgate", gr["dgate"], dg, dtype)
    check_close("dweight", gr["dweight"], dw, dtype)


def test_gnorm_layer_shape_bf16():
    """The layer's output norm: B=16, T=2048, H=8 heads of dv = 64, bf16; the oracle on
    the whole tensor; bf16 output = rounded fp32 output; deterministic dweight."""
    o, gate, wt, dy = _gn_case(7, (16, 2048, 8, 64), torch.bfloat16)
    oc, gc, wc, dc = o.cuda(), gate.cuda(), wt.cuda(), dy.cuda()
    y = kda.gnorm_fwd(oc, gc, wc)
    y32 = kda.gnorm_fwd(oc, gc, wc, out_dtype=torch.float32)
    gr = kda.gnorm_bwd(oc, gc, wc, dc)
    gr32 = kda.gnorm_bwd(oc, gc, wc, dc, out_dtype=torch.float32)
    gr2 = kda.gnorm_bwd(oc, gc, wc, dc)
    torch.cuda.synchronize()
    # the arithmetic against the oracle at fp32 output; the bf16 output is its rounding, bit for bit
    check_close("y", y32, ops.gnorm_fwd(to_np(o), to_np(gate), to_np(wt)), torch.bfloat16)
    do, dg, dw = ops.gnorm_bwd(to_np(o), to_np(gate), to_np(wt), to_np(dy))
    check_close("do", gr32["do"], do, torch.bfloat16)
    check_close("dgate", gr32["dgate"], dg, torch.bfloat16)
    check_close("dweight", gr32["dweight"], dw, torch.bfloat16)
    assert torch.equal(y32.to(torch.bfloat16), y)
    assert torch.equal(gr32["do"].to(torch.bfloat16), gr["do"])
    assert torch.equal(gr32["dgate"].to(torch.bfloat16), gr["dgate"])
    assert torch.equal(gr["dweight"], gr2["dweight"])
