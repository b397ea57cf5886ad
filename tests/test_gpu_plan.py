"""Varlen chunk metadata on the device: bit-exact against the oracle's enumeration."""
import json
import os

import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunk_amd as kda
import oracle

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _check(cu):
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    T = int(cu[-1])
    N = len(cu) - 1
    idx, off = kda.plan_varlen(cu_t, T)
    ridx, roff = oracle.plan_varlen(cu, 64)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), roff)
    M = kda.max_chunks(T, N)
    got = idx.cpu().numpy()
    assert got.shape == (M, 2)
    n = len(ridx)
    assert np.array_equal(got[:n], ridx)
    assert np.all(got[n:] == -1)


def test_plan_golden():
    fx = json.load(open(os.path.join(GOLD, "varlen_metadata.json")))
    for case in fx["cases"]:
        _check(case["cu_seqlens"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_plan_random(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 3000))
    lens = rng.integers(0, 300, size=N)
    lens[rng.random(N) < 0.1] = 1
    lens[rng.random(N) < 0.05] = 0
    _check(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))


def test_plan_packed_config_row():
    """The 65,536-token packed row with geometric document lengths (mean 512)."""
    cu = kda_inputs.geometric_cu_seqlens(3).numpy()
    assert cu[-1] == 65536 and np.any(np.diff(cu) == 1)
    _check(cu)
    kda.check_cu_seqlens(torch.tensor(cu, device="cuda"), 65536)


def test_check_cu_seqlens_rejects_bad_offsets():
    with pytest.raises(kda.KdaError):
        kda.check_cu_seqlens(torch.tensor([0, 5, 3, 9], dtype=torch.int32, device="cuda"), 9)
    with pytest.raises(kda.KdaError):
        kda.check_cu_seqlens(torch.tensor([0, 5, 8], dtype=torch.int32, device="cuda"), 9)
