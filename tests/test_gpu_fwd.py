"""Forward (kda_fwd) against the fp64 oracle, element by element."""
import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunk_amd as kda
from cases import (check_close, oracle_fwd, oracle_fwd_raw, prepared, raw_inputs, to_dev, to_np)

pytestmark = pytest.mark.gpu


def run_fwd(d, scale, cu=None, out_dtype=torch.float32, **kw):
    plan = kda.plan_varlen(d["cu"], d["q"].shape[1]) if cu is not None else None
    return kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, h0=d.get("h0"),
                   cu_seqlens=d.get("cu"), plan=plan, out_dtype=out_dtype, **kw)


CASES = [
    # (name, B, T, H, dk, dv, dtype, kwargs)
    ("small_fp32", 1, 128, 1, 32, 64, torch.float32, {}),
    ("small_fp32_weak_h0", 2, 200, 2, 32, 64, torch.float32, dict(weak=True, h0_std=0.1)),
    ("small_fp32_g0", 1, 160, 2, 32, 64, torch.float32, dict(variant="g0", h0_std=0.1)),
    ("small_fp32_beta1", 1, 130, 2, 32, 64, torch.float32, dict(variant="beta1_unit", weak=True)),
    ("partial_T100", 3, 100, 2, 32, 64, torch.float32, dict(weak=True, h0_std=0.1)),
    ("single_token", 2, 1, 3, 32, 64, torch.float32, dict(h0_std=0.1)),
    ("bf16_weak", 2, 300, 4, 32, 64, torch.bfloat16, dict(weak=True, h0_std=0.1)),
    ("bf16_default", 2, 256, 8, 32, 64, torch.bfloat16, {}),
    ("dk64_fp32", 1, 150, 2, 64, 64, torch.float32, dict(weak=True, h0_std=0.1)),
    ("dk64_bf16_weak_h0", 2, 150, 2, 64, 64, torch.bfloat16, dict(weak=True, h0_std=0.1)),
    ("dk64_bf16_default", 2, 256, 4, 64, 64, torch.bfloat16, {}),
    ("dk128_fp32", 1, 200, 2, 128, 128, torch.float32, dict(weak=True, h0_std=0.1)),
    ("dk128_bf16", 2, 190, 2, 128, 128, torch.bfloat16, dict(weak=True)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fwd_matches_oracle(case):
    name, B, T, H, dk, dv, dtype, kw = case
    inp, _ = prepared(10 + len(name), B, T, H, dk, dv, dtype, **kw)
    d = to_dev(inp)
    scale = dk ** -0.5
    o, hT = run_fwd(d, scale)
    oref, href = oracle_fwd(inp, scale)
    check_close("o", o, oref, dtype)
    check_close("hT", hT, href, dtype)


def test_fwd_config0_seed0():
    """The small forward configuration exactly as specified: fp32, B=1, H=1, T=128, dk=32,
    dv=64, scale = dk^-0.5, the default distributions, h0 = 0, drawn with seed 0."""
    inp, _ = prepared(0, 1, 128, 1, 32, 64, torch.float32)
    assert inp["h0"] is None
    d = to_dev(inp)
    o, hT = run_fwd(d, 32 ** -0.5)
    oref, href = oracle_fwd(inp, 32 ** -0.5)
    check_close("o", o, oref, torch.float32)
    check_close("hT", hT, href, torch.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("variant", ["g0", "beta1_unit"])
def test_fwd_layer_shape_adversarial(variant, dtype):
    """The layer shape (T=2048, H=8, dk=32, dv=64; B=2) with no decay (g = 0: the pure
    delta rule, the state carries across all 32 chunks) or with beta = 1 on unit keys
    (every write replaces the key's old value), h0 ~ N(0, 0.1)."""
    inp, _ = prepared(60 + len(variant), 2, 2048, 8, 32, 64, dtype, variant=variant, h0_std=0.1)
    d = to_dev(inp)
    o, hT = run_fwd(d, 32 ** -0.5)
    oref, href = oracle_fwd(inp, 32 ** -0.5)
    check_close("o", o, oref, dtype)
    check_close("hT", hT, href, dtype)


def test_fwd_bf16_output_is_rounded_fp32_output():
    inp, _ = prepared(7, 2, 200, 4, 32, 64, torch.bfloat16, weak=True, h0_std=0.1)
    d = to_dev(inp)
    o32, h32 = run_fwd(d, 0.17, out_dtype=torch.float32)
    o16, h16 = run_fwd(d, 0.17, out_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(h32, h16)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fwd_fused_preparation(dtype):
    raw = kda_inputs.draw(21, 2, 180, 4, 32, 64, h0_std=0.1, a_log_range=kda_inputs.A_LOG_RANGE_WEAK)
    rin = raw_inputs(raw, dtype)
    d = to_dev(rin)
    o, hT = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], 32 ** -0.5, h0=d["h0"], A_log=d["A_log"],
                    dt_bias=d["dt_bias"], l2norm_qk=True, gate_in_kernel=True, beta_logits=True,
                    out_dtype=torch.float32)
    oref, href = oracle_fwd_raw(rin, 32 ** -0.5)
    check_close("o", o, oref, dtype)
    check_close("hT", hT, href, dtype)


def test_fwd_layer_shape_full():
    """The 300M layer shape: B=16, T=2048, H=8, dk=32, dv=64, bf16, h0 = 0."""
    inp, _ = prepared(1, 16, 2048, 8, 32, 64, torch.bfloat16)
    d = to_dev(inp)
    o, hT = run_fwd(d, 32 ** -0.5)
    oref, href = oracle_fwd(inp, 32 ** -0.5)
    check_close("o", o, oref, torch.bfloat16)
    check_close("hT", hT, href, torch.bfloat16)


def test_fwd_layer_shape_weak_decay():
    """Same shape with weak decay, so the state crosses all 32 chunks."""
    inp, _ = prepared(11, 4, 2048, 8, 32, 64, torch.bfloat16, weak=True, h0_std=0.1)
    d = to_dev(inp)
    o, hT = run_fwd(d, 32 ** -0.5)
    oref, href = oracle_fwd(inp, 32 ** -0.5)
    check_close("o", o, oref, torch.bfloat16)
    check_close("hT", hT, href, torch.bfloat16)


def _packed(seed, lens, H=2, dk=32, dv=64, dtype=torch.float32, weak=True):
    T = int(sum(lens))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    inp, _ = prepared(seed, 1, T, H, dk, dv, dtype, weak=weak, h0_std=0.1, n_states=len(lens))
    inp["cu"] = cu
    return inp


def test_packed_equals_separate_bitwise():
    """Documents of 96 and 160 tokens packed with offsets (0, 96, 256) reproduce their
    separate runs bitwise; without offsets the second document differs."""
    for dtype in (torch.float32, torch.bfloat16):
        inp = _packed(5, [96, 160], dtype=dtype)
        d = to_dev(inp)
        o, hT = run_fwd(d, 0.2, cu=d["cu"])
        cu = [0, 96, 256]
        for n in range(2):
            sl = slice(cu[n], cu[n + 1])
            part = {k: d[k][:, sl].contiguous() for k in ("q", "k", "v", "g", "beta")}
            part["h0"] = d["h0"][n:n + 1].contiguous()
            on, hn = run_fwd(part, 0.2)
            assert torch.equal(on, o[:, sl]), (dtype, n)
            assert torch.equal(hn[0], hT[n]), (dtype, n)
        whole = {k: d[k] for k in ("q", "k", "v", "g", "beta")}
        whole["h0"] = d["h0"][:1].contiguous()
        o2, _ = run_fwd(whole, 0.2)
        assert torch.equal(o2[:, :96], o[:, :96])
        assert not torch.allclose(o2[:, 96:], o[:, 96:])


def test_packed_matches_oracle_with_short_and_empty_documents():
    lens = [1, 0, 64, 65, 1, 1, 130, 3, 0, 200]
    inp = _packed(8, lens, H=3)
    d = to_dev(inp)
    o, hT = run_fwd(d, 0.2, cu=d["cu"])
    oref, href = oracle_fwd(inp, 0.2, cu=inp["cu"])
    check_close("o", o, oref, torch.float32)
    check_close("hT", hT, href, torch.float32)
    # empty documents: hT = h0
    assert torch.equal(hT[1], d["h0"][1]) and torch.equal(hT[8], d["h0"][8])


def test_packed_config_row_forward():
    """65,536-token packed row, geometric document lengths (mean 512, length-1 documents
    included), H=8, bf16, per-document h0 ~ N(0, 0.1)."""
    cu = kda_inputs.geometric_cu_seqlens(3)
    N = cu.numel() - 1
    inp, _ = prepared(3, 1, 65536, 8, 32, 64, torch.bfloat16, h0_std=0.1, n_states=N)
    inp["cu"] = cu
    d = to_dev(inp)
    o, hT = run_fwd(d, 32 ** -0.5, cu=d["cu"])
    oref, href = oracle_fwd(inp, 32 ** -0.5, cu=cu)
    check_close("o", o, oref, torch.bfloat16)
    check_close("hT", hT, href, torch.bfloat16)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128)], ids=["dk64", "dk128"])
def test_packed_larger_heads_with_short_and_empty_documents(dims, dtype):
    """Packed rows at dk = 64 and 128: empty, one-token and partial-chunk documents,
    per-document h0, against the oracle; and the 96 + 160 pair equals its separate runs
    bit for bit."""
    dk, dv = dims
    lens = [1, 0, 64, 65, 1, 1, 130, 3, 0, 200]
    inp = _packed(18, lens, H=2, dk=dk, dv=dv, dtype=dtype)
    d = to_dev(inp)
    o, hT = run_fwd(d, dk ** -0.5, cu=d["cu"])
    oref, href = oracle_fwd(inp, dk ** -0.5, cu=inp["cu"])
    check_close("o", o, oref, dtype)
    check_close("hT", hT, href, dtype)
    assert torch.equal(hT[1], d["h0"][1]) and torch.equal(hT[8], d["h0"][8])
    inp = _packed(19, [96, 160], dk=dk, dv=dv, dtype=dtype)
    d = to_dev(inp)
    o, hT = run_fwd(d, 0.2, cu=d["cu"])
    cu = [0, 96, 256]
    for n in range(2):
        sl = slice(cu[n], cu[n + 1])
        part = {k: d[k][:, sl].contiguous() for k in ("q", "k", "v", "g", "beta")}
        part["h0"] = d["h0"][n:n + 1].contiguous()
        on, hn = run_fwd(part, 0.2)
        assert torch.equal(on, o[:, sl]), n
        assert torch.equal(hn[0], hT[n]), n
