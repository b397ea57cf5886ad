"""Host-side checks of libkda.so: it loads, exports every function declared in
include/kda.h, and rejects bad arguments before launching anything (no GPU
needed: every call here returns from argument validation)."""
import ctypes
import os
import re

import pytest

import kimi_delta_attention_chunk_amd as kda
from kimi_delta_attention_chunk_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = kda.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_max_chunks_formula():
    lib = kda.load_library()
    assert lib.kda_max_chunks(256, 2, 64) == (256 + 2 * 63) // 64
    assert lib.kda_max_chunks(0, 1, 64) == 0
    assert lib.kda_max_chunks(-1, 1, 64) == -1
    assert lib.kda_max_chunks(10, 1, 0) == -1


def _desc(**kw):
    d = dict(B=1, T=128, H=1, dk=32, dv=64, N=1, chunk=64, dtype=B.KDA_FP32, out_dtype=B.KDA_FP32,
             scale=0.1767767, flags=0)
    d.update(kw)
    return B.KdaDesc(**d)


def _ws(desc, backward=False):
    lib = kda.load_library()
    return (lib.kda_bwd_workspace if backward else lib.kda_fwd_workspace)(ctypes.byref(desc))


def test_workspace_sizes():
    assert _ws(_desc()) > 0
    assert _ws(_desc(), True) > _ws(_desc())
    # packed row of 3 documents
    assert _ws(_desc(N=3)) >= _ws(_desc())


@pytest.mark.parametrize("bad,code", [
    (dict(dk=48), B.KDA_ERR_UNSUPPORTED),
    (dict(chunk=32), B.KDA_ERR_UNSUPPORTED),
    (dict(T=-1), B.KDA_ERR_INVALID),
    (dict(H=0), B.KDA_ERR_INVALID),
    (dict(dtype=7), B.KDA_ERR_INVALID),
    (dict(flags=1 << 9), B.KDA_ERR_INVALID),
    (dict(B=2, N=3), B.KDA_ERR_INVALID),
])
def test_invalid_descriptor_rejected(bad, code):
    lib = kda.load_library()
    d = _desc(**bad)
    assert _ws(d) == 0
    fake = ctypes.c_void_p(0x10000)
    rc = lib.kda_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, None, None, None,
                     None, fake, None, fake, 1 << 40, None)
    assert rc == code, lib.kda_last_error()
    assert lib.kda_last_error().decode()


def test_null_and_misaligned_pointers_rejected():
    lib = kda.load_library()
    d = _desc()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10004)
    ws = _ws(d)
    args = [fake] * 5 + [None, None, None, None, None, None, fake, None, fake, ws, None]
    bad_null = list(args)
    bad_null[0] = None
    assert lib.kda_fwd(ctypes.byref(d), *bad_null) == B.KDA_ERR_INVALID
    assert b"q must not be null" in lib.kda_last_error()
    bad_al = list(args)
    bad_al[2] = odd
    assert lib.kda_fwd(ctypes.byref(d), *bad_al) == B.KDA_ERR_INVALID
    assert b"aligned" in lib.kda_last_error()
    small = list(args)
    small[-2] = ws - 1
    assert lib.kda_fwd(ctypes.byref(d), *small) == B.KDA_ERR_WORKSPACE
    # gate in kernel needs A_log and dt_bias
    dg = _desc(flags=B.F_GATE_IN_KERNEL)
    assert lib.kda_fwd(ctypes.byref(dg), *args) == B.KDA_ERR_INVALID
    assert b"A_log" in lib.kda_last_error()
    # packed needs all three tables and B == 1
    part = list(args)
    part[8] = fake  # cu_seqlens only
    assert lib.kda_fwd(ctypes.byref(d), *part) == B.KDA_ERR_INVALID
    d2 = _desc(B=2, N=2)
    full = list(args)
    full[8] = full[9] = full[10] = fake
    assert lib.kda_fwd(ctypes.byref(d2), *full) == B.KDA_ERR_INVALID
    assert b"B == 1" in lib.kda_last_error()


def test_step_and_plan_validation():
    lib = kda.load_library()
    fake = ctypes.c_void_p(0x10000)
    rc = lib.kda_step(4, 2, 32, 48, 0, 0, 1.0, 0, *([fake] * 5), None, None, fake, fake, None)
    assert rc == B.KDA_ERR_UNSUPPORTED
    rc = lib.kda_step(4, 2, 32, 64, 0, 0, 1.0, 0, *([fake] * 5), None, None, None, fake, None)
    assert rc == B.KDA_ERR_INVALID and b"h must not be null" in lib.kda_last_error()
    assert lib.kda_plan_varlen(None, 2, 10, 64, fake, fake, None) == B.KDA_ERR_INVALID
    assert lib.kda_plan_varlen(fake, 0, 10, 64, fake, fake, None) == B.KDA_ERR_INVALID
    assert lib.kda_status_str(B.KDA_ERR_WORKSPACE) == b"workspace missing or too small"


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError):
        kda.fwd(x, x, torch.zeros(1, 4, 1, 64), x, torch.zeros(1, 4, 1), 1.0)


# ---------------------------------------------------------------- short convolution, gated norm
def _fake(i=1):
    return ctypes.c_void_p(0x100000 * i)  # 16-byte aligned, never dereferenced (validation fails first)


@pytest.mark.parametrize("kw,code", [
    (dict(D=12), B.KDA_ERR_INVALID),
    (dict(D=0), B.KDA_ERR_INVALID),
    (dict(W=5), B.KDA_ERR_UNSUPPORTED),
    (dict(W=0), B.KDA_ERR_UNSUPPORTED),
    (dict(flags=2), B.KDA_ERR_INVALID),
    (dict(cu=True, Bn=2), B.KDA_ERR_INVALID),
    (dict(x=None), B.KDA_ERR_INVALID),
    (dict(x=ctypes.c_void_p(0x100008)), B.KDA_ERR_INVALID),
])
def test_conv_fwd_rejects(kw, code):
    lib = kda.load_library()
    a = dict(Bn=1, T=64, D=64, W=4, flags=0, x=_fake(1), cu=False)
    a.update(kw)
    rc = lib.kda_conv_fwd(a["Bn"], a["T"], a["D"], a["W"], B.KDA_BF16, B.KDA_BF16, a["flags"], a["x"], _fake(2),
                          None, _fake(3) if a["cu"] else None, 3, _fake(4), None)
    assert rc == code, lib.kda_last_error()


def test_conv_bwd_workspace_checked():
    lib = kda.load_library()
    need = lib.kda_conv_bwd_workspace(1, 64, 64, 4)
    assert need > 0 and lib.kda_conv_bwd_workspace(1, 64, 12, 4) == 0
    rc = lib.kda_conv_bwd(1, 64, 64, 4, B.KDA_BF16, B.KDA_BF16, 0, _fake(1), _fake(2), None, None, 0, _fake(3),
                          _fake(4), _fake(5), None, _fake(6), need - 1, None)
    assert rc == B.KDA_ERR_WORKSPACE


@pytest.mark.parametrize("rows,dv,eps,code", [(10, 48, 1e-6, B.KDA_ERR_UNSUPPORTED), (-1, 64, 1e-6, B.KDA_ERR_INVALID),
                                              (10, 64, 0.0, B.KDA_ERR_INVALID)])
def test_gnorm_rejects(rows, dv, eps, code):
    lib = kda.load_library()
    rc = lib.kda_gnorm_fwd(rows, dv, B.KDA_BF16, B.KDA_BF16, eps, _fake(1), _fake(2), _fake(3), _fake(4), None)
    assert rc == code, lib.kda_last_error()
    need = lib.kda_gnorm_bwd_workspace(1000, 64)
    assert need > 0
    rc = lib.kda_gnorm_bwd(1000, 64, B.KDA_BF16, B.KDA_BF16, 1e-6, _fake(1), _fake(2), _fake(3), _fake(4), _fake(5),
                           _fake(6), _fake(7), _fake(8), need - 1, None)
    assert rc == B.KDA_ERR_WORKSPACE


# ---------------------------------------------------------------- context parallelism
def test_segment_maps_and_state_scan_reject():
    lib = kda.load_library()
    d = _desc(dk=64, dv=128)  # not a supported pair
    rc = lib.kda_segment_maps(ctypes.byref(d), *([_fake(1)] * 5), None, None, None, None, None, _fake(2), _fake(3),
                              1 << 30, None)
    assert rc == B.KDA_ERR_UNSUPPORTED, lib.kda_last_error()
    for dk, dv in ((32, 64), (64, 64), (128, 128)):  # every supported pair: the workspace is checked
        d = _desc(dk=dk, dv=dv)
        rc = lib.kda_segment_maps(ctypes.byref(d), *([_fake(1)] * 5), None, None, None, None, None, _fake(2),
                                  _fake(3), 16, None)
        assert rc == B.KDA_ERR_WORKSPACE, lib.kda_last_error()
    for dk, dv in ((64, 128), (128, 64), (32, 32)):
        assert lib.kda_state_scan(4, 2, dk, dv, 0, _fake(1), _fake(2), None, _fake(3), None, None) == \
            B.KDA_ERR_UNSUPPORTED
    assert lib.kda_state_scan(0, 2, 32, 64, 0, _fake(1), _fake(2), None, _fake(3), None, None) == B.KDA_ERR_INVALID
    assert lib.kda_state_scan(4, 2, 32, 64, 2, _fake(1), _fake(2), None, _fake(3), None, None) == B.KDA_ERR_INVALID
    assert lib.kda_state_scan(4, 2, 32, 64, 0, None, _fake(2), None, _fake(3), None, None) == B.KDA_ERR_INVALID


def test_state_pass_only_and_saved_forward_flags():
    lib = kda.load_library()
    fake = _fake(1)
    # kda_fwd: the state-pass-only flag belongs to the backward
    d = _desc(flags=B.F_DH0_ONLY)
    rc = lib.kda_fwd(ctypes.byref(d), *([fake] * 5), None, None, None, None, None, None, fake, None, fake, 1 << 40,
                     None)
    assert rc == B.KDA_ERR_INVALID and b"backward flag" in lib.kda_last_error()
    # kda_fwd with a saved forward sizes its workspace like the saving forward
    d = _desc(flags=B.F_FWD_SAVED)
    need = _ws(d, backward=True)
    assert need > _ws(_desc())
    rc = lib.kda_fwd(ctypes.byref(d), *([fake] * 5), None, None, None, None, None, None, fake, None, fake, need - 1,
                     None)
    assert rc == B.KDA_ERR_WORKSPACE
    # kda_bwd with the state pass only: dh0 is required, the per-token gradients may be null
    d = _desc(flags=B.F_DH0_ONLY | B.F_FWD_SAVED)
    head = [fake] * 5 + [None, None, None, None, None, None]
    rc = lib.kda_bwd(ctypes.byref(d), *head, fake, None, None, None, None, None, None, None, None, None, fake, 16,
                     None)
    assert rc == B.KDA_ERR_INVALID and b"dh0" in lib.kda_last_error()
    rc = lib.kda_bwd(ctypes.byref(d), *head, fake, None, None, None, None, None, None, _fake(2), None, None, fake, 16,
                     None)
    assert rc == B.KDA_ERR_WORKSPACE, lib.kda_last_error()
    # gate parameters are not needed when no gate gradient is formed
    d = _desc(flags=B.F_DH0_ONLY | B.F_GATE_IN_KERNEL)
    head_g = [fake] * 5 + [fake, fake, None, None, None, None]
    rc = lib.kda_bwd(ctypes.byref(d), *head_g, fake, None, None, None, None, None, None, _fake(2), None, None, fake,
                     16, None)
    assert rc == B.KDA_ERR_WORKSPACE, lib.kda_last_error()


def test_empty_inputs_need_no_token_pointers():
    lib = kda.load_library()
    fake = _fake(1)
    d = _desc(T=0)
    # no tokens: null q, k, v, g, beta and o pass the checks (the tiny workspace is what fails)
    rc = lib.kda_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None, None, None, fake,
                     fake, 16, None)
    assert rc == B.KDA_ERR_WORKSPACE, lib.kda_last_error()
    rc = lib.kda_bwd(ctypes.byref(d), *([None] * 11), None, None, None, None, None, None, None, _fake(2), None, None,
                     fake, 16, None)
    assert rc == B.KDA_ERR_WORKSPACE, lib.kda_last_error()
    # with tokens the same call is rejected for the missing q
    d = _desc(T=64)
    rc = lib.kda_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None, None, None, fake,
                     fake, 16, None)
    assert rc == B.KDA_ERR_INVALID and b"q must not be null" in lib.kda_last_error()
    # gated norm without rows: the row arrays may be null, the workspace is still checked
    rc = lib.kda_gnorm_bwd(0, 64, B.KDA_BF16, B.KDA_BF16, 1e-6, None, None, _fake(3), None, None, None, _fake(4),
                           _fake(5), 0, None)
    assert rc == B.KDA_ERR_WORKSPACE, lib.kda_last_error()


def test_noalloc_forward_validation():
    """kda_fwd_noalloc refuses the save/saved/dh0 flags and problems whose workspace would
    not fit its fixed scratch, before any device call."""
    lib = kda.load_library()
    fake = ctypes.c_void_p(0x10000)
    args = [fake] * 5 + [None, None, None, None, None, None, fake, None, None]
    for fl in (B.F_SAVE_FOR_BWD, B.F_FWD_SAVED, B.F_DH0_ONLY):
        d = _desc(flags=fl)
        assert lib.kda_fwd_noalloc(ctypes.byref(d), *args) == B.KDA_ERR_INVALID
        assert b"noalloc" in lib.kda_last_error()
    big = _desc(B=16, T=2048, H=8, N=16)
    assert _ws(big) > 64 << 20
    assert lib.kda_fwd_noalloc(ctypes.byref(big), *args) == B.KDA_ERR_UNSUPPORTED
    assert b"scratch" in lib.kda_last_error()
    fits = _desc(B=4, T=2048, H=8, N=4)
    assert _ws(fits) <= 64 << 20
    bad_null = list(args)
    bad_null[0] = None
    assert lib.kda_fwd_noalloc(ctypes.byref(fits), *bad_null) == B.KDA_ERR_INVALID


# The arrays each kernel family writes (a missing one would send its stores to the
# absent marker, offset 0).
_WRITTEN = {
    (32, False): {"hs", "pm", "pmT", "hh", "qh", "qhT", "ol"},
    (32, True): {"hs", "pm", "pmT", "hh", "qh", "qhT", "ol", "aqT", "tm", "dhs", "part_a", "part_dt"},
    (64, False): {"w", "u", "aqk", "hs", "vn", "qg", "khT", "gl"},
}
_WRITTEN[(64, True)] = _WRITTEN[(64, False)] | {"tm", "aqT", "qgT", "khb", "wT", "dhs", "dvn", "dqt", "dkh", "dwv",
                                                  "daq", "dtv", "dgl", "dbv", "dkt", "dxq", "dxk", "part_a", "part_dt"}


@pytest.mark.parametrize("dims", [(32, 64), (64, 64), (128, 128)])
@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
@pytest.mark.parametrize("shape", [(1, 130, 3, 1), (2, 2048, 8, 2), (1, 1000, 2, 7), (1, 1, 1, 1)],
                         ids=["dense1", "dense2", "packed7", "one_token"])
def test_workspace_layout_has_no_array_at_offset_zero(dims, backward, shape):
    """Every array of every layout lies past the 256-byte sink, 256-byte aligned, inside the
    size the workspace query reports, with no overlap; and every array the kernels write is
    present (this pins the layout fix after an array once sat at offset 0, the absent
    marker, and a kernel's stores went to a null pointer)."""
    dk, dv = dims
    B, T, H, N = shape
    arrays = kda.binding.workspace_arrays((B, T, H, dk), dv, N, backward)
    total = kda.workspace_bytes((B, T, H, dk), dv, N, backward)
    end = 256
    for name, off, nb in arrays:
        assert off >= 256 and off % 256 == 0 and nb > 0, (name, off, nb)
        assert off >= end, (name, off, end)  # in order, disjoint
        end = off + nb
    assert end <= total
    names = {n for n, _, _ in arrays}
    need = _WRITTEN[(min(dk, 64), backward)]
    assert need <= names, need - names
