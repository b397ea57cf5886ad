"""Context parallelism on one GPU (every supported dk, dv): one long document split into segments
that run independently, chained by their transition matrices (kda_segment_maps,
kda_state_scan), and rerun with their true entering states / end gradients,
reproduces the single pass over the whole document (the oracle's), forward and
backward.  Weak decay, nonzero h0 and dhT, so the state carries across every
segment boundary."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_chunk_amd as kda
from cases import check_close, oracle_bwd, oracle_fwd, prepared, to_dev

pytestmark = pytest.mark.gpu


def _cp_run_saved(d, scale, cu):
    """The same scheme without repeated work: the chunk quantities are formed once (the
    first forward keeps them), the maps and the second state pass reuse them, and the
    first backward pass runs the reverse state pass alone."""
    T, H = d["q"].shape[1], d["q"].shape[2]
    cuc = torch.tensor(cu, dtype=torch.int32, device="cuda")
    plan = kda.plan_varlen(cuc, T)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    R = len(cu) - 1
    ws = torch.empty(kda.workspace_bytes(tuple(d["q"].shape), d["v"].shape[-1], R, True, d["q"].dtype),
                     dtype=torch.uint8, device="cuda")
    pk = dict(cu_seqlens=cuc, plan=plan, workspace=ws)
    _, c = kda.fwd(*args, scale, save_for_bwd=True, out_dtype=torch.float32, **pk)
    M = kda.segment_maps(*args, fwd_saved=True, **pk)
    h_in, hT = kda.state_scan(M, c, d["h0"][0])
    o, _ = kda.fwd(*args, scale, h0=h_in, fwd_saved=True, save_for_bwd=True, out_dtype=torch.float32, **pk)
    e = kda.bwd(*args, scale, d["do"], h0=h_in, fwd_saved=True, dh0_only=True, **pk)["dh0"]
    D, dh0 = kda.state_scan(M, e, d["dhT"][0], transpose=True)
    gr = kda.bwd(*args, scale, d["do"], h0=h_in, dhT=D, fwd_saved=True, out_dtype=torch.float32, **pk)
    gr["dh0"] = dh0
    return o, hT, gr


def _cp_run(d, scale, cu, backward):
    T = d["q"].shape[1]
    cuc = torch.tensor(cu, dtype=torch.int32, device="cuda")
    plan = kda.plan_varlen(cuc, T)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    # 1. every segment from a zero state: its final state c_r, and its transition matrix M_r
    _, c = kda.fwd(*args, scale, cu_seqlens=cuc, plan=plan, out_dtype=torch.float32)
    M = kda.segment_maps(*args, cu_seqlens=cuc, plan=plan)
    # 2. the chain: each segment's true entering state, and the row's final state
    h_in, hT = kda.state_scan(M, c, d["h0"][0])
    # 3. every segment again from its true entering state
    o, _ = kda.fwd(*args, scale, h0=h_in, cu_seqlens=cuc, plan=plan, out_dtype=torch.float32)
    if not backward:
        return o, hT, None
    # 4. each segment's own gradient with respect to its entering state, the reverse chain
    #    (each segment's true end gradient, and the row's dh0), then the gradients
    e = kda.bwd(*args, scale, d["do"], h0=h_in, cu_seqlens=cuc, plan=plan, out_dtype=torch.float32)["dh0"]
    D, dh0 = kda.state_scan(M, e, d["dhT"][0], transpose=True)
    gr = kda.bwd(*args, scale, d["do"], h0=h_in, dhT=D, cu_seqlens=cuc, plan=plan, out_dtype=torch.float32)
    gr["dh0"] = dh0
    return o, hT, gr


DIMS = [(32, 64), (64, 64), (128, 128)]


def _row(dk):
    """Row length and its aligned / ragged segment offsets (shorter rows at the larger
    heads keep the oracle's fp64 pass to seconds)."""
    T = 2048 if dk == 32 else 1024
    q = T // 4
    return T, {"aligned": [0, q, 2 * q, 3 * q, T], "ragged": [0, 300, q + 300, q + 301, T]}


@pytest.mark.parametrize("dims", DIMS, ids=["dk32", "dk64", "dk128"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("split", ["aligned", "ragged"])
def test_context_parallel_equals_single_pass(dtype, split, dims):
    dk, dv = dims
    T, cus = _row(dk)
    cu = cus[split]
    H = 4
    inp, _ = prepared(11, 1, T, H, dk, dv, dtype, weak=True, h0_std=0.1, upstream=True, dhT=True)
    d = to_dev(inp, "cuda:0")
    scale = dk ** -0.5
    o, hT, gr = _cp_run(d, scale, cu, backward=True)
    torch.cuda.synchronize()
    oref, href = oracle_fwd(inp, scale)
    gref = oracle_bwd(inp, scale)
    check_close("o", o, oref, dtype)
    check_close("hT", hT[None], href, dtype)
    for nm in ("dq", "dk", "dv", "dg", "dbeta"):
        check_close(nm, gr[nm], gref[nm], dtype)
    check_close("dh0", gr["dh0"][None], gref["dh0"], dtype)


@pytest.mark.parametrize("dims", DIMS, ids=["dk32", "dk64", "dk128"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_context_parallel_from_saved_forward(dtype, dims):
    """The scheme with the chunk quantities formed once: same results as the plain one,
    bit for bit, and as the oracle's single pass."""
    dk, dv = dims
    T, cus = _row(dk)
    cu = cus["ragged"]
    H = 4
    inp, _ = prepared(13, 1, T, H, dk, dv, dtype, weak=True, h0_std=0.1, upstream=True, dhT=True)
    d = to_dev(inp, "cuda:0")
    scale = dk ** -0.5
    o1, h1, g1 = _cp_run(d, scale, cu, backward=True)
    o2, h2, g2 = _cp_run_saved(d, scale, cu)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    for nm in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(g1[nm], g2[nm]), nm
    oref, href = oracle_fwd(inp, scale)
    gref = oracle_bwd(inp, scale)
    check_close("o", o2, oref, dtype)
    check_close("dk", g2["dk"], gref["dk"], dtype)
    check_close("dh0", g2["dh0"][None], gref["dh0"], dtype)


@pytest.mark.parametrize("dims", DIMS, ids=["dk32", "dk64", "dk128"])
def test_segment_map_of_one_document_is_its_state_map(dims):
    """M h0 + hT(h0 = 0) = hT(h0) for every document of a packed row, and an empty
    document's map is the identity."""
    lens = [700, 0, 1, 64, 1283]
    cu = np.cumsum([0] + lens).tolist()
    dk, dv = dims
    T, H = cu[-1], 2
    inp, _ = prepared(12, 1, T, H, dk, dv, torch.float32, weak=True, h0_std=0.1, n_states=len(lens))
    d = to_dev(inp, "cuda:0")
    cuc = torch.tensor(cu, dtype=torch.int32, device="cuda")
    plan = kda.plan_varlen(cuc, T)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    M = kda.segment_maps(*args, cu_seqlens=cuc, plan=plan)
    _, c = kda.fwd(*args, 0.1, cu_seqlens=cuc, plan=plan)
    _, hT = kda.fwd(*args, 0.1, h0=d["h0"], cu_seqlens=cuc, plan=plan)
    torch.cuda.synchronize()
    pred = torch.matmul(M, d["h0"]) + c
    check_close("M h0 + c", pred, hT.double().cpu().numpy(), torch.float32)
    assert torch.equal(M[1], torch.eye(dk, device="cuda").expand(H, dk, dk))


@pytest.mark.parametrize("dims", DIMS, ids=["dk32", "dk64", "dk128"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_context_parallel_packed_row_of_two_documents(dtype, dims):
    """A packed row of two documents, each cut into segments (three, and two with a
    one-token segment); the segments run as one packed row, each document's chain is
    scanned on its own from its own h0 / dhT, and the result equals the oracle's pass
    over the two-document row."""
    dk, dv = dims
    H = 4
    if dk == 32:
        T, docs, seg = 2200, [0, 1500, 2200], [0, 512, 1100, 1500, 1501, 2200]
    else:
        T, docs, seg = 1100, [0, 750, 1100], [0, 256, 550, 750, 751, 1100]
    chains = [(0, 3), (3, 5)]  # the segments of each document
    inp, _ = prepared(14, 1, T, H, dk, dv, dtype, weak=True, h0_std=0.1, n_states=2, upstream=True, dhT=True)
    d = to_dev(inp, "cuda:0")
    scale = dk ** -0.5
    cuc = torch.tensor(seg, dtype=torch.int32, device="cuda")
    plan = kda.plan_varlen(cuc, T)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    R = len(seg) - 1
    ws = torch.empty(kda.workspace_bytes((1, T, H, dk), dv, R, True, dtype), dtype=torch.uint8, device="cuda")
    pk = dict(cu_seqlens=cuc, plan=plan, workspace=ws)
    _, c = kda.fwd(*args, scale, save_for_bwd=True, out_dtype=torch.float32, **pk)
    M = kda.segment_maps(*args, fwd_saved=True, **pk)
    h_in = torch.empty_like(c)
    hT = torch.empty((2, H, dk, dv), dtype=torch.float32, device="cuda")
    for n, (a, b) in enumerate(chains):
        h_in[a:b], hT[n] = kda.state_scan(M[a:b], c[a:b], d["h0"][n])
    o, _ = kda.fwd(*args, scale, h0=h_in, fwd_saved=True, save_for_bwd=True, out_dtype=torch.float32, **pk)
    e = kda.bwd(*args, scale, d["do"], h0=h_in, fwd_saved=True, dh0_only=True, **pk)["dh0"]
    D = torch.empty_like(e)
    dh0 = torch.empty((2, H, dk, dv), dtype=torch.float32, device="cuda")
    for n, (a, b) in enumerate(chains):
        D[a:b], dh0[n] = kda.state_scan(M[a:b], e[a:b], d["dhT"][n], transpose=True)
    gr = kda.bwd(*args, scale, d["do"], h0=h_in, dhT=D, fwd_saved=True, out_dtype=torch.float32, **pk)
    torch.cuda.synchronize()
    cu_docs = torch.tensor(docs, dtype=torch.int32)
    oref, href = oracle_fwd(inp, scale, cu=cu_docs)
    gref = oracle_bwd(inp, scale, cu=cu_docs)
    check_close("o", o, oref, dtype)
    check_close("hT", hT, href, dtype)
    for nm in ("dq", "dk", "dv", "dg", "dbeta"):
        check_close(nm, gr[nm], gref[nm], dtype)
    check_close("dh0", dh0, gref["dh0"], dtype)
