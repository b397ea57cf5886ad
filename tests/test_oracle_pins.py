"""Pins of the fp64 oracle against facts fixed independently of it.

Each test checks the oracle against something other than itself: hand-worked
fixtures (tests/golden/), closed forms, invariants of the delta rule, a
brute-force O(T^2) sum, textbook causal linear attention, library routines,
chunk-size invariance of the algebraic rewrite, packed-vs-separate runs, and
central finite differences for every gradient.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand(*shape, rng=RNG, std=1.0):
    return rng.standard_normal(shape) * std


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _gates(shape, rng=RNG, lo=-0.3, hi=-0.001):
    """Log-decays in [lo, hi] (weak enough that the state survives)."""
    return rng.uniform(lo, hi, size=shape)


def _case(B=1, T=9, H=2, dk=3, dv=4, rng=RNG, h0=True, weak=True):
    q = _unit(_rand(B, T, H, dk, rng=rng))
    k = _unit(_rand(B, T, H, dk, rng=rng))
    v = _rand(B, T, H, dv, rng=rng)
    g = _gates((B, T, H, dk), rng) if weak else -rng.uniform(0.1, 30, size=(B, T, H, dk))
    beta = rng.uniform(0.05, 0.95, size=(B, T, H))
    hh = _rand(B, H, dk, dv, rng=rng, std=0.5) if h0 else None
    return q, k, v, g, beta, hh


def relerr(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- fixtures
@pytest.mark.parametrize("name", ["scalar_two_tokens.json", "matrix_one_token.json"])
def test_hand_worked_fixture(name):
    fx = json.load(open(os.path.join(GOLD, name)))
    dk, dv = fx["dk"], fx["dv"]
    a = np.array(fx["a"])
    T = a.shape[0]
    g = np.log(a).reshape(1, T, 1, dk)
    q = np.array(fx["q"]).reshape(1, T, 1, dk)
    k = np.array(fx["k"]).reshape(1, T, 1, dk)
    v = np.array(fx["v"]).reshape(1, T, 1, dv)
    beta = np.array(fx["beta"]).reshape(1, T, 1)
    h0 = np.array(fx["h0"]).reshape(1, 1, dk, dv)
    o, hT = oracle.forward(q, k, v, g, beta, fx["scale"], h0=h0)
    np.testing.assert_allclose(o.reshape(T, dv), np.array(fx["o"]), rtol=1e-14, atol=1e-14)
    key = "hT_after_2" if "hT_after_2" in fx else "hT"
    np.testing.assert_allclose(hT.reshape(dk, dv), np.array(fx[key]), rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- forward pins
def test_delta_invariant_beta_one_unit_keys():
    """beta = 1 and |k| = 1: the write makes S_t^T k_t = v_t exactly.

    Read through the output with q_t = k_t: o_t = scale * S_t^T k_t = scale * v_t.
    """
    q, k, v, g, beta, h0 = _case(B=2, T=17, H=2, dk=5, dv=3)
    beta = np.ones_like(beta)
    o, hT = oracle.forward(k, k, v, g, beta, 0.7, h0=h0)
    assert relerr(o, 0.7 * v) < 1e-12
    kT = k[:, -1]  # [B,H,dk]
    pred = np.einsum("bhc,bhcj->bhj", kT, hT)
    assert relerr(pred, v[:, -1]) < 1e-12


def test_beta_zero_closed_form():
    """beta = 0: no writes, the state only decays.

    o_t = scale * sum_c q_tc exp(sum_{s<=t} g_sc) h0[c,:], hT = Diag(exp(sum g)) h0.
    """
    q, k, v, g, beta, h0 = _case(B=2, T=13, H=3, dk=4, dv=5)
    beta = np.zeros_like(beta)
    o, hT = oracle.forward(q, k, v, g, beta, 0.3, h0=h0)
    cum = np.cumsum(g, axis=1)  # [B,T,H,dk]
    ref = 0.3 * np.einsum("bthc,bhcj->bthj", q * np.exp(cum), h0)
    assert relerr(o, ref) < 1e-13
    refT = np.exp(cum[:, -1])[..., None] * h0
    assert relerr(hT, refT) < 1e-13


def test_small_beta_is_decayed_linear_attention():
    """h0 = 0, beta = eps: o / eps -> decayed causal linear attention.

    Brute-force O(T^2) sum: scale * sum_{s<=t} sum_c q_tc exp(G_tc - G_sc) k_sc v_s,
    with G the running sum of g (the write at s is decayed by s+1..t only).
    """
    q, k, v, g, beta, _ = _case(B=1, T=23, H=2, dk=4, dv=3, h0=False)
    eps = 1e-7
    o, _ = oracle.forward(q, k, v, g, np.full_like(beta, eps), 0.5)
    G = np.cumsum(g, axis=1)
    B, T, H, dk = q.shape
    ref = np.zeros_like(o)
    for t in range(T):
        for s in range(t + 1):
            w = np.sum(q[:, t] * k[:, s] * np.exp(G[:, t] - G[:, s]), axis=-1)  # [B,H]
            ref[:, t] += 0.5 * w[..., None] * v[:, s]
    assert relerr(o / eps, ref) < 1e-5


def test_orthonormal_keys_no_decay_is_linear_attention():
    """g = 0, beta = 1, orthonormal keys (T <= dk): textbook causal linear attention."""
    T, dk, dv = 6, 8, 5
    Qm, _ = np.linalg.qr(RNG.standard_normal((dk, dk)))
    k = Qm[:, :T].T.reshape(1, T, 1, dk)
    q = RNG.standard_normal((1, T, 1, dk))
    v = RNG.standard_normal((1, T, 1, dv))
    o, hT = oracle.forward(q, k, v, np.zeros_like(q), np.ones((1, T, 1)), 1.0)
    scores = np.tril(q[0, :, 0] @ k[0, :, 0].T)
    ref = scores @ v[0, :, 0]
    assert relerr(o[0, :, 0], ref) < 1e-13
    assert relerr(hT[0, 0], k[0, :, 0].T @ v[0, :, 0]) < 1e-13


@pytest.mark.parametrize("weak", [True, False])
def test_chunk_size_invariance(weak):
    """The chunked rewrite equals the token loop for any chunk size, partial chunks included."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, h0 = _case(B=2, T=100, H=2, dk=6, dv=5, rng=rng, weak=weak)
    o, hT = oracle.forward(q, k, v, g, beta, 0.4, h0=h0)
    for C in (1, 2, 3, 16, 64, 128):
        oc, hc = oracle.chunked_forward(q, k, v, g, beta, 0.4, C, h0=h0)
        assert relerr(oc, o) < 1e-12, C
        assert relerr(hc, hT) < 1e-12, C


def test_packed_row_equals_separate_runs():
    """Offsets reset the state: a packed row reproduces each document's own run exactly,
    and the same row without offsets does not (torchtitan PR #4347, Verification)."""
    rng = np.random.default_rng(11)
    lens = [96, 160]
    T = sum(lens)
    q, k, v, g, beta, _ = _case(B=1, T=T, H=2, dk=4, dv=3, rng=rng, h0=False)
    h0 = _rand(2, 2, 4, 3, rng=rng)
    cu = [0, 96, 256]
    o, hT = oracle.forward(q, k, v, g, beta, 0.5, h0=h0, cu_seqlens=cu)
    for n in range(2):
        sl = slice(cu[n], cu[n + 1])
        on, hn = oracle.forward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], 0.5,
                                h0=h0[n:n + 1])
        assert np.array_equal(on, o[:, sl])
        assert np.array_equal(hn[0], hT[n])
    o_nocu, _ = oracle.forward(q, k, v, g, beta, 0.5, h0=h0[:1])
    assert not np.allclose(o_nocu[:, 96:], o[:, 96:])
    assert np.array_equal(o_nocu[:, :96], o[:, :96])


def test_empty_and_single_token_documents():
    rng = np.random.default_rng(3)
    cu = [0, 1, 1, 5, 6]
    q, k, v, g, beta, _ = _case(B=1, T=6, H=1, dk=3, dv=2, rng=rng, h0=False)
    h0 = _rand(4, 1, 3, 2, rng=rng)
    o, hT = oracle.forward(q, k, v, g, beta, 1.0, h0=h0, cu_seqlens=cu)
    assert np.array_equal(hT[1], h0[1])  # empty document: hT = h0
    # a one-token document is one step from its own h0
    o1, h1 = oracle.step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], 1.0, h0[0:1])
    assert np.array_equal(o1, o[:, 0])
    assert np.array_equal(h1, hT[0:1])


def test_steps_equal_forward():
    q, k, v, g, beta, h0 = _case(B=3, T=11, H=2, dk=4, dv=5)
    o, hT = oracle.forward(q, k, v, g, beta, 0.6, h0=h0)
    h = h0.copy()
    for t in range(11):
        ot, h = oracle.step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], 0.6, h)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(h, hT)


# ---------------------------------------------------------------- backward pins
def _loss(inputs, scale, d_o, dhT, cu=None):
    q, k, v, g, beta, h0 = inputs
    o, hT = oracle.forward(q, k, v, g, beta, scale, h0=h0, cu_seqlens=cu)
    return float(np.sum(o * d_o) + np.sum(hT * dhT))


@pytest.mark.parametrize("shape,cu", [((1, 7, 2, 3, 4), None), ((2, 5, 1, 2, 3), None),
                                      ((1, 12, 2, 4, 2), [0, 3, 3, 4, 12])])
def test_backward_matches_finite_differences(shape, cu):
    B, T, H, dk, dv = shape
    rng = np.random.default_rng(sum(shape))
    q, k, v, g, beta, _ = _case(B, T, H, dk, dv, rng=rng, h0=False)
    N = B if cu is None else len(cu) - 1
    h0 = _rand(N, H, dk, dv, rng=rng, std=0.5)
    d_o = _rand(B, T, H, dv, rng=rng)
    dhT = _rand(N, H, dk, dv, rng=rng)
    scale = 0.45
    gr = oracle.backward(q, k, v, g, beta, scale, d_o, h0=h0, dhT=dhT, cu_seqlens=cu)
    inputs = [q, k, v, g, beta, h0]
    names = ["dq", "dk", "dv", "dg", "dbeta", "dh0"]
    eps = 1e-6
    for i, nm in enumerate(names):
        x = inputs[i]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + eps
            lp = _loss(inputs, scale, d_o, dhT, cu)
            x[idx] = orig - eps
            lm = _loss(inputs, scale, d_o, dhT, cu)
            x[idx] = orig
            fd[idx] = (lp - lm) / (2 * eps)
        assert relerr(gr[nm], fd) < 1e-7, (nm, relerr(gr[nm], fd))


def test_backward_directional_across_checkpoints():
    """T = 150 crosses the backward's recompute checkpoints (every 64 tokens)."""
    rng = np.random.default_rng(99)
    B, T, H, dk, dv = 1, 150, 1, 3, 2
    q, k, v, g, beta, h0 = _case(B, T, H, dk, dv, rng=rng, weak=True)
    g = g * 0.05
    d_o = _rand(B, T, H, dv, rng=rng)
    dhT = _rand(B, H, dk, dv, rng=rng)
    gr = oracle.backward(q, k, v, g, beta, 0.5, d_o, h0=h0, dhT=dhT)
    inputs = [q, k, v, g, beta, h0]
    names = ["dq", "dk", "dv", "dg", "dbeta", "dh0"]
    eps = 1e-6
    for i, nm in enumerate(names):
        d = rng.standard_normal(inputs[i].shape)
        base = inputs[i].copy()
        inputs[i] = base + eps * d
        lp = _loss(inputs, 0.5, d_o, dhT)
        inputs[i] = base - eps * d
        lm = _loss(inputs, 0.5, d_o, dhT)
        inputs[i] = base
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(gr[nm] * d))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (nm, fd, an)


def test_beta_zero_closed_form_gradients():
    """beta = 0: dh0 = sum_t scale Diag(G_t) q_t do_t^T + Diag(G_T) dhT; dq_t = scale Diag(G_t) h0 do_t."""
    q, k, v, g, beta, h0 = _case(B=1, T=9, H=2, dk=3, dv=4)
    beta = np.zeros_like(beta)
    d_o = _rand(1, 9, 2, 4)
    dhT = _rand(1, 2, 3, 4)
    gr = oracle.backward(q, k, v, g, beta, 0.8, d_o, h0=h0, dhT=dhT)
    Gm = np.exp(np.cumsum(g, axis=1))
    ref = 0.8 * np.einsum("bthc,bthj->bhcj", Gm * q, d_o) + Gm[:, -1][..., None] * dhT
    assert relerr(gr["dh0"], ref) < 1e-13
    dq = 0.8 * np.einsum("bthc,bhcj,bthj->bthc", Gm, h0, d_o)
    assert relerr(gr["dq"], dq) < 1e-13
    assert np.all(gr["dk"] == 0) and np.all(gr["dv"] == 0)


# ---------------------------------------------------------------- preparation pins
def test_softplus_and_sigmoid_match_library_routines():
    x = np.concatenate([np.linspace(-40, 40, 2001), [19.999, 20.0, 20.001]])
    A_log = np.zeros(1)
    dt = np.zeros((1, 1))
    g = oracle.gate(x.reshape(-1, 1, 1), A_log, dt).ravel()
    sp = torch.nn.functional.softplus(torch.tensor(x, dtype=torch.float64)).numpy()
    np.testing.assert_allclose(-g, sp, rtol=1e-14, atol=1e-300)
    from scipy.special import expit
    np.testing.assert_allclose(oracle.sigmoid(x), expit(x), rtol=1e-14)


def test_gate_closed_form_points():
    # f + dt_bias = 0 -> softplus = log 2 ; A_log = log 3 -> g = -3 log 2
    f = np.array([[[0.25, -1.0]]])
    dt = np.array([[-0.25, 1.0]])
    g = oracle.gate(f, np.array([math.log(3.0)]), dt)
    np.testing.assert_allclose(g.ravel(), [-3 * math.log(2.0)] * 2, rtol=1e-15)


def test_l2norm_unit_length_and_direction():
    x = RNG.standard_normal((50, 7)) * 3
    y = oracle.l2norm(x, eps=0.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-13)
    y2 = oracle.l2norm(x)  # with eps the norm is just below 1
    assert np.all(np.linalg.norm(y2, axis=-1) < 1.0)


def test_l2norm_epsilon_inside_the_root_closed_form():
    """x = (3, 4): |x|^2 = 25, so x^ = x / sqrt(25 + eps) with eps inside the root.
    An eps outside it, x / (|x| + eps) = x / 5.000001, differs by about 1.8e-7
    relative (sqrt(25 + 1e-6) = 5.0000001), far above the rtol used here; so does a
    missing eps (x / 5, 2e-8 relative)."""
    x = np.array([[3.0, 4.0]])
    for eps in (1e-6, 0.5):
        y = oracle.l2norm(x, eps=eps)
        np.testing.assert_allclose(y, x / math.sqrt(25.0 + eps), rtol=1e-15, atol=0)
        assert abs(y[0, 0] - 3.0 / (5.0 + eps)) > 1e-9
    # the default is eps = 1e-6 (reading 5 of the pages' silence)
    np.testing.assert_allclose(oracle.l2norm(x), x / math.sqrt(25.0 + 1e-6), rtol=1e-15, atol=0)


def test_prep_backward_finite_differences():
    rng = np.random.default_rng(5)
    T, H, dk = 4, 2, 3
    qr, kr, f = (rng.standard_normal((1, T, H, dk)) for _ in range(3))
    A_log = np.log(rng.uniform(1, 16, H))
    dt = rng.standard_normal((H, dk)) * 0.1
    b = rng.standard_normal((1, T, H))
    ups = [rng.standard_normal((1, T, H, dk)) for _ in range(3)] + [rng.standard_normal((1, T, H))]

    def loss(qr, kr, f, A_log, dt, b):
        outs = oracle.prep_forward(qr, kr, f, A_log, dt, b)
        return float(sum(np.sum(o * u) for o, u in zip(outs, ups)))

    gr = oracle.prep_backward(qr, kr, f, A_log, dt, b, *ups)
    args = [qr, kr, f, A_log, dt, b]
    names = ["dq", "dk", "df", "dA_log", "ddt_bias", "db"]
    eps = 1e-6
    for i, nm in enumerate(names):
        x = args[i]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            o0 = x[idx]
            x[idx] = o0 + eps
            lp = loss(*args)
            x[idx] = o0 - eps
            lm = loss(*args)
            x[idx] = o0
            fd[idx] = (lp - lm) / (2 * eps)
        assert relerr(gr[nm], fd) < 1e-7, nm


# ---------------------------------------------------------------- metadata pins
def test_varlen_metadata_golden():
    fx = json.load(open(os.path.join(GOLD, "varlen_metadata.json")))
    for case in fx["cases"]:
        idx, off = oracle.plan_varlen(case["cu_seqlens"], case["chunk"])
        assert off.tolist() == case["chunk_offsets"]
        assert idx.tolist() == case["chunk_indices"]


def test_varlen_metadata_brute_force():
    """Enumerate tokens one by one: a new chunk starts at every document start and
    every C tokens after it."""
    rng = np.random.default_rng(17)
    for _ in range(50):
        N = int(rng.integers(1, 12))
        lens = rng.integers(0, 200, size=N)
        lens[rng.random(N) < 0.2] = 1
        cu = np.concatenate([[0], np.cumsum(lens)])
        C = int(rng.choice([1, 16, 64]))
        idx, off = oracle.plan_varlen(cu, C)
        starts = []
        for n in range(N):
            for t in range(int(lens[n])):
                if t % C == 0:
                    starts.append((n, t // C))
        assert [tuple(r) for r in idx.tolist()] == starts
        assert off[-1] == len(starts)
        assert len(starts) <= oracle.max_chunks(int(cu[-1]), N, C)
