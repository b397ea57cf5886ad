"""Backward (kda_bwd) against the oracle's hand-derived backward, element by element."""
import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunk_amd as kda
from cases import (check_close, oracle_bwd, oracle_bwd_raw, prepared, raw_inputs, to_dev)

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def run_bwd(d, scale, out_dtype=torch.float32, **kw):
    cu = d.get("cu")
    plan = kda.plan_varlen(cu, d["q"].shape[1]) if cu is not None else None
    return kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, d["do"], h0=d.get("h0"),
                   dhT=d.get("dhT"), cu_seqlens=cu, plan=plan, out_dtype=out_dtype, **kw)


def compare(got, ref, dtype, names=GRADS):
    for nm in names:
        check_close(nm, got[nm], ref[nm], dtype)


CASES = [
    ("small_fp32", 1, 128, 1, 32, 64, torch.float32, dict(h0_std=0.1, dhT=True)),
    ("fp32_weak", 2, 200, 2, 32, 64, torch.float32, dict(weak=True, h0_std=0.1, dhT=True)),
    ("fp32_g0", 1, 150, 2, 32, 64, torch.float32, dict(variant="g0", h0_std=0.1, dhT=True)),
    ("fp32_beta1", 1, 130, 2, 32, 64, torch.float32, dict(variant="beta1_unit", weak=True, dhT=True)),
    ("partial_T100", 3, 100, 2, 32, 64, torch.float32, dict(weak=True, h0_std=0.1, dhT=True)),
    ("single_token", 2, 1, 3, 32, 64, torch.float32, dict(h0_std=0.1, dhT=True)),
    ("no_state_grads", 2, 70, 2, 32, 64, torch.float32, dict(weak=True)),
    ("bf16_weak", 2, 300, 4, 32, 64, torch.bfloat16, dict(weak=True, h0_std=0.1, dhT=True)),
    ("bf16_default", 2, 256, 8, 32, 64, torch.bfloat16, {}),
    ("dk64_fp32", 1, 150, 2, 64, 64, torch.float32, dict(weak=True, h0_std=0.1, dhT=True)),
    ("dk64_bf16_weak_h0", 2, 150, 2, 64, 64, torch.bfloat16, dict(weak=True, h0_std=0.1, dhT=True)),
    ("dk64_bf16_default", 2, 256, 4, 64, 64, torch.bfloat16, {}),
    ("dk128_fp32", 1, 200, 2, 128, 128, torch.float32, dict(weak=True, h0_std=0.1, dhT=True)),
    ("dk128_bf16", 2, 190, 2, 128, 128, torch.bfloat16, dict(weak=True, dhT=True)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_oracle(case):
    name, B, T, H, dk, dv, dtype, kw = case
    inp, _ = prepared(40 + len(name), B, T, H, dk, dv, dtype, upstream=True, **kw)
    d = to_dev(inp)
    scale = dk ** -0.5
    got = run_bwd(d, scale)
    ref = oracle_bwd(inp, scale)
    compare(got, ref, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("variant", ["g0", "beta1_unit"])
def test_bwd_layer_shape_adversarial(variant, dtype):
    """The layer shape (T=2048, H=8, dk=32, dv=64; B=2) with no decay or with beta = 1 on
    unit keys, h0 ~ N(0, 0.1), upstream do and dhT ~ N(0, 1): with g = 0 every chunk's
    state gradient reaches the first chunk."""
    inp, _ = prepared(70 + len(variant), 2, 2048, 8, 32, 64, dtype, variant=variant, h0_std=0.1,
                      upstream=True, dhT=True)
    d = to_dev(inp)
    got = run_bwd(d, 32 ** -0.5)
    ref = oracle_bwd(inp, 32 ** -0.5)
    compare(got, ref, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128)], ids=["dk64", "dk128"])
def test_bwd_packed_larger_heads(dims, dtype):
    """Packed rows at dk = 64 and 128 with empty, one-token and partial-chunk documents,
    per-document h0 and dhT, against the oracle; the 96 + 160 pair equals its separate
    runs bit for bit."""
    dk, dv = dims
    lens = [1, 0, 64, 65, 1, 1, 130, 3, 0, 200]
    inp = _packed(28, lens, H=2, dk=dk, dv=dv, dtype=dtype)
    d = to_dev(inp)
    got = run_bwd(d, dk ** -0.5)
    ref = oracle_bwd(inp, dk ** -0.5, cu=inp["cu"])
    compare(got, ref, dtype)
    assert torch.equal(got["dh0"][1], d["dhT"][1]) and torch.equal(got["dh0"][8], d["dhT"][8])
    inp = _packed(29, [96, 160], dk=dk, dv=dv, dtype=dtype)
    d = to_dev(inp)
    got = run_bwd(d, 0.2)
    cu = [0, 96, 256]
    for n in range(2):
        sl = slice(cu[n], cu[n + 1])
        part = {k: d[k][:, sl].contiguous() for k in ("q", "k", "v", "g", "beta", "do")}
        part["h0"] = d["h0"][n:n + 1].contiguous()
        part["dhT"] = d["dhT"][n:n + 1].contiguous()
        gn = run_bwd(part, 0.2)
        for nm in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(gn[nm], got[nm][:, sl]), (n, nm)
        assert torch.equal(gn["dh0"][0], got["dh0"][n]), n


def test_bwd_bf16_outputs_are_rounded_fp32_outputs():
    inp, _ = prepared(8, 2, 200, 4, 32, 64, torch.bfloat16, weak=True, h0_std=0.1, upstream=True, dhT=True)
    d = to_dev(inp)
    g32 = run_bwd(d, 0.17, out_dtype=torch.float32)
    g16 = run_bwd(d, 0.17, out_dtype=torch.bfloat16)
    for nm in ("dq", "dk", "dv"):
        assert torch.equal(g32[nm].to(torch.bfloat16), g16[nm]), nm
    for nm in ("dg", "dbeta", "dh0"):
        assert torch.equal(g32[nm], g16[nm]), nm


def test_bwd_is_deterministic():
    inp, _ = prepared(9, 2, 256, 4, 32, 64, torch.bfloat16, weak=True, h0_std=0.1, upstream=True, dhT=True)
    d = to_dev(inp)
    a = run_bwd(d, 0.17)
    b = run_bwd(d, 0.17)
    for nm in GRADS:
        assert torch.equal(a[nm], b[nm]), nm


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bwd_fused_preparation(dtype):
    raw = kda_inputs.draw(22, 2, 180, 4, 32, 64, h0_std=0.1, upstream=True, dhT=True,
                          a_log_range=kda_inputs.A_LOG_RANGE_WEAK)
    rin = raw_inputs(raw, dtype)
    d = to_dev(rin)
    got = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], 32 ** -0.5, d["do"], h0=d["h0"],
                  dhT=d["dhT"], A_log=d["A_log"], dt_bias=d["dt_bias"], l2norm_qk=True,
                  gate_in_kernel=True, beta_logits=True, out_dtype=torch.float32)
    ref = oracle_bwd_raw(rin, 32 ** -0.5)
    compare(got, ref, dtype, GRADS + ("dA_log", "ddt_bias"))


def test_bwd_layer_shape_full():
    """The 300M layer shape, B=16, T=2048, H=8, dk=32, dv=64, bf16, do ~ N(0,1), no state grads."""
    inp, _ = prepared(1, 16, 2048, 8, 32, 64, torch.bfloat16, upstream=True)
    d = to_dev(inp)
    got = run_bwd(d, 32 ** -0.5)
    ref = oracle_bwd(inp, 32 ** -0.5)
    compare(got, ref, torch.bfloat16)


def test_bwd_layer_shape_weak_decay_with_prep():
    """Same shape (B=4), weak decay, fused preparation, upstream dhT."""
    raw = kda_inputs.draw(12, 4, 2048, 8, 32, 64, h0_std=0.1, upstream=True, dhT=True,
                          a_log_range=kda_inputs.A_LOG_RANGE_WEAK)
    rin = raw_inputs(raw, torch.bfloat16)
    d = to_dev(rin)
    got = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], 32 ** -0.5, d["do"], h0=d["h0"],
                  dhT=d["dhT"], A_log=d["A_log"], dt_bias=d["dt_bias"], l2norm_qk=True,
                  gate_in_kernel=True, beta_logits=True, out_dtype=torch.float32)
    ref = oracle_bwd_raw(rin, 32 ** -0.5)
    compare(got, ref, torch.bfloat16, GRADS + ("dA_log", "ddt_bias"))


def _packed(seed, lens, H=2, dk=32, dv=64, dtype=torch.float32, weak=True):
    T = int(sum(lens))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    inp, _ = prepared(seed, 1, T, H, dk, dv, dtype, weak=weak, h0_std=0.1, n_states=len(lens),
                      upstream=True, dhT=True)
    inp["cu"] = cu
    return inp


def test_bwd_packed_equals_separate_bitwise():
    for dtype in (torch.float32, torch.bfloat16):
        inp = _packed(6, [96, 160], dtype=dtype)
        d = to_dev(inp)
        got = run_bwd(d, 0.2)
        cu = [0, 96, 256]
        for n in range(2):
            sl = slice(cu[n], cu[n + 1])
            part = {k: d[k][:, sl].contiguous() for k in ("q", "k", "v", "g", "beta", "do")}
            part["h0"] = d["h0"][n:n + 1].contiguous()
            part["dhT"] = d["dhT"][n:n + 1].contiguous()
            gn = run_bwd(part, 0.2)
            for nm in ("dq", "dk", "dv", "dg", "dbeta"):
                assert torch.equal(gn[nm], got[nm][:, sl]), (dtype, n, nm)
            assert torch.equal(gn["dh0"][0], got["dh0"][n]), (dtype, n)


def test_bwd_packed_short_and_empty_documents():
    lens = [1, 0, 64, 65, 1, 1, 130, 3, 0, 200]
    inp = _packed(9, lens, H=3)
    d = to_dev(inp)
    got = run_bwd(d, 0.2)
    ref = oracle_bwd(inp, 0.2, cu=inp["cu"])
    compare(got, ref, torch.float32)
    assert torch.equal(got["dh0"][1], d["dhT"][1])  # empty document: dh0 = dhT


def test_bwd_packed_config_row():
    """65,536-token packed row, geometric lengths (mean 512), H=8, bf16, per-document h0,
    upstream do and dhT ~ N(0,1)."""
    cu = kda_inputs.geometric_cu_seqlens(3)
    N = cu.numel() - 1
    inp, _ = prepared(3, 1, 65536, 8, 32, 64, torch.bfloat16, h0_std=0.1, n_states=N, upstream=True,
                      dhT=True)
    inp["cu"] = cu
    d = to_dev(inp)
    got = run_bwd(d, 32 ** -0.5)
    ref = oracle_bwd(inp, 32 ** -0.5, cu=cu)
    compare(got, ref, torch.bfloat16)


@pytest.mark.parametrize("dtype,dims", [(torch.bfloat16, (32, 64)), (torch.float32, (32, 64)),
                                        (torch.bfloat16, (128, 128)), (torch.float32, (64, 64))])
def test_bwd_from_saved_forward_equals_recompute(dtype, dims):
    """kda_fwd(save_for_bwd) + kda_bwd(fwd_saved) gives bitwise the same gradients as a
    backward that recomputes the forward, and the same forward outputs."""
    dk, dv = dims
    raw = kda_inputs.draw(31, 2, 200, 4, dk, dv, h0_std=0.1, upstream=True, dhT=True,
                          a_log_range=kda_inputs.A_LOG_RANGE_WEAK)
    rin = raw_inputs(raw, dtype)
    d = to_dev(rin)
    kw = dict(A_log=d["A_log"], dt_bias=d["dt_bias"], l2norm_qk=True, gate_in_kernel=True,
              beta_logits=True, out_dtype=torch.float32)
    scale = dk ** -0.5
    o1, h1 = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, h0=d["h0"], **kw)
    ws = torch.empty(kda.workspace_bytes(tuple(d["q"].shape), dv, 2, True), dtype=torch.uint8,
                     device="cuda")
    o2, h2 = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, h0=d["h0"], workspace=ws,
                     save_for_bwd=True, **kw)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    g_saved = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, d["do"], h0=d["h0"],
                      dhT=d["dhT"], workspace=ws, fwd_saved=True, **kw)
    g_rec = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, d["do"], h0=d["h0"],
                    dhT=d["dhT"], **kw)
    for nm in GRADS + ("dA_log", "ddt_bias"):
        assert torch.equal(g_saved[nm], g_rec[nm]), nm
    ref = oracle_bwd_raw(rin, scale)
    compare(g_saved, ref, dtype, GRADS + ("dA_log", "ddt_bias"))
