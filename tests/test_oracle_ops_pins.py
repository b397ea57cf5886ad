"""Pins of the short-convolution and gated-norm oracle (oracle/ops.py) to facts
outside itself: an impulse response and numpy's own convolution, the document
reset (packed row = separate runs), torch's RMS norm, scale invariance, and
central finite differences of every gradient.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import ops



def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- short convolution
def test_conv_impulse_response_is_the_kernel_reversed_in_time():
    # a unit impulse at t0 in channel c reaches y[t0 + lag] through tap W - 1 - lag
    B, T, D, W = 1, 12, 3, 4
    w = _rng(0).normal(size=(D, W))
    x = np.zeros((B, T, D))
    x[0, 5, 1] = 1.0
    y = ops.conv_fwd(x, w)
    for lag in range(W):
        assert y[0, 5 + lag, 1] == w[1, W - 1 - lag]
    y[0, 5:5 + W, 1] = 0.0
    assert not np.any(y)


def test_conv_single_document_equals_numpy_convolve():
    B, T, D, W = 2, 40, 5, 4
    r = _rng(1)
    x, w = r.normal(size=(B, T, D)), r.normal(size=(D, W))
    y = ops.conv_fwd(x, w)
    for b in range(B):
        for c in range(D):
            # causal: y[t] = sum_j w_rev[j] x[t - j], w_rev[j] = w[W - 1 - j]
            ref = np.convolve(x[b, :, c], w[c, ::-1], mode="full")[:T]
            np.testing.assert_allclose(y[b, :, c], ref, rtol=0, atol=1e-13)


def test_conv_bias_and_silu():
    B, T, D, W = 1, 9, 4, 3
    r = _rng(2)
    x, w, bias = r.normal(size=(B, T, D)), r.normal(size=(D, W)), r.normal(size=D)
    z = ops.conv_fwd(x, w) + bias
    np.testing.assert_allclose(ops.conv_fwd(x, w, bias), z, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ops.conv_fwd(x, w, bias, silu=True), z / (1 + np.exp(-z)), rtol=1e-15, atol=1e-15)
    # silu(0) = 0: a zero input with zero bias stays zero
    assert not np.any(ops.conv_fwd(np.zeros((1, 5, 2)), w[:2], silu=True))


def test_conv_packed_row_equals_separate_documents():
    lens = [1, 5, 2, 9, 1, 3]
    cu = np.cumsum([0] + lens)
    T, D, W = int(cu[-1]), 6, 4
    r = _rng(3)
    x, w, dy = r.normal(size=(1, T, D)), r.normal(size=(D, W)), r.normal(size=(1, T, D))
    y = ops.conv_fwd(x, w, cu_seqlens=cu, silu=True)
    dx, dw, db = ops.conv_bwd(x, w, dy, cu_seqlens=cu, silu=True)
    dw_sum, db_sum = np.zeros_like(w), np.zeros(D)
    for n in range(len(lens)):
        a, e = cu[n], cu[n + 1]
        ys = ops.conv_fwd(x[:, a:e], w, silu=True)
        np.testing.assert_array_equal(y[:, a:e], ys)
        dxs, dws, dbs = ops.conv_bwd(x[:, a:e], w, dy[:, a:e], silu=True)
        np.testing.assert_allclose(dx[:, a:e], dxs, rtol=0, atol=1e-14)
        dw_sum += dws
        db_sum += dbs
    np.testing.assert_allclose(dw, dw_sum, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(db, db_sum, rtol=1e-13, atol=1e-13)
    # negative control: without the offsets the second document sees the first
    assert not np.allclose(ops.conv_fwd(x, w, silu=True)[:, cu[1]:cu[2]], y[:, cu[1]:cu[2]])


@pytest.mark.parametrize("silu,packed", [(False, False), (True, False), (True, True)])
def test_conv_backward_finite_differences(silu, packed):
    B, T, D, W = (1, 11, 3, 4) if packed else (2, 7, 3, 4)
    cu = np.array([0, 4, 5, 11]) if packed else None
    r = _rng(4)
    x, w, bias, dy = r.normal(size=(B, T, D)), r.normal(size=(D, W)), r.normal(size=D), r.normal(size=(B, T, D))
    dx, dw, db = ops.conv_bwd(x, w, dy, bias, cu, silu)
    loss = lambda x_, w_, b_: float(np.sum(dy * ops.conv_fwd(x_, w_, b_, cu, silu)))
    h = 1e-6
    for arr, grad, wrap in ((x, dx, lambda a: loss(a, w, bias)), (w, dw, lambda a: loss(x, a, bias)),
                            (bias, db, lambda a: loss(x, w, a))):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            p, m = arr.copy(), arr.copy()
            p[i] += h
            m[i] -= h
            fd[i] = (wrap(p) - wrap(m)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-7, atol=1e-8)


# ----------------------------------------------------------------- gated norm
def test_gnorm_equals_torch_rms_norm_times_sigmoid_gate():
    r = _rng(5)
    o, g, wt = r.normal(size=(3, 4, 64)), r.normal(size=(3, 4, 64)), r.normal(size=64)
    y = ops.gnorm_fwd(o, g, wt)
    ref = torch.nn.functional.rms_norm(torch.tensor(o), (64,), torch.tensor(wt), eps=ops.RMS_EPS) * torch.sigmoid(
        torch.tensor(g))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-14)


def test_gnorm_closed_forms():
    d = 32
    wt = np.linspace(0.5, 1.5, d)
    # a constant row c: mean(o^2) = c^2, so n = c / sqrt(c^2 + eps); gate 0 halves it
    c = 3.0
    y = ops.gnorm_fwd(np.full((1, d), c), np.zeros((1, d)), wt)
    np.testing.assert_allclose(y[0], 0.5 * wt * c / np.sqrt(c * c + ops.RMS_EPS), rtol=1e-15)
    # scale invariance (eps negligible at this scale)
    o = _rng(6).normal(size=(5, d)) * 10
    g = _rng(7).normal(size=(5, d))
    np.testing.assert_allclose(ops.gnorm_fwd(7.0 * o, g, wt, eps=0.0), ops.gnorm_fwd(o, g, wt, eps=0.0), rtol=1e-14)


def test_gnorm_backward_finite_differences():
    r = _rng(8)
    o, g, wt, dy = r.normal(size=(2, 3, 8)), r.normal(size=(2, 3, 8)), r.normal(size=8), r.normal(size=(2, 3, 8))
    do, dg, dw = ops.gnorm_bwd(o, g, wt, dy)
    loss = lambda o_, g_, w_: float(np.sum(dy * ops.gnorm_fwd(o_, g_, w_)))
    h = 1e-6
    for arr, grad, wrap in ((o, do, lambda a: loss(a, g, wt)), (g, dg, lambda a: loss(o, a, wt)),
                            (wt, dw, lambda a: loss(o, g, a))):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            p, m = arr.copy(), arr.copy()
            p[i] += h
            m[i] -= h
            fd[i] = (wrap(p) - wrap(m)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-7, atol=1e-8)
