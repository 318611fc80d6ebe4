"""Inputs that force the candidate buffers of the fused kernel to fill and be
compacted many times: with strictly increasing scores every key beats the
current threshold. Scores are exact in fp32, so selections must match the
oracle exactly, including the lower-index rule on plateaus of equal scores."""
import numpy as np
import pytest
import torch

from parity import assert_ok, check_dense, check_pivot

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def increasing(L, plateau=1, H=4, d=32, batch=1):
    # one head, one dimension: score(t, s) = x_s, the s-th positive bf16 value
    # above 1.0 (every bf16 step is exact), repeated `plateau` times
    bits = (0x3F80 + np.arange(L) // plateau).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    Q = torch.zeros((batch, L, H, d), dtype=torch.bfloat16, device=DEV)
    Q[:, :, 0, 0] = 1.0
    K = torch.zeros((batch, L, d), dtype=torch.bfloat16, device=DEV)
    K[:, :, 0] = x
    W = torch.zeros((batch, L, H), dtype=torch.float32, device=DEV)
    W[:, :, 0] = 1.0
    return Q, W, K


@pytest.mark.parametrize("plateau", [1, 8])
@pytest.mark.parametrize("k", [64, 700])
def test_dense_compaction(plateau, k):
    Q, W, K = increasing(6000, plateau)
    res, idx, _ = check_dense(Q, W, K, k)
    assert_ok(res)
    assert res.exact == res.rows
    if plateau == 1:
        for r in (k - 1, 3000, 5999):
            assert idx[0, r].tolist() == list(range(r - k + 1, r + 1))


@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_pivot_compaction(variant):
    Q, W, K = increasing(5000, 4)
    rc, rr, _, _, _ = check_pivot(Q, W, K, 4, 200, 64, variant)
    assert_ok(rc, rr)
    assert rc.exact == rc.rows and rr.exact == rr.rows


def test_dense_compaction_h64():
    Q, W, K = increasing(5000, 3, H=64, d=128)
    rows = [(0, r) for r in (0, 100, 2047, 2048, 4095, 4999)]
    res, _, _ = check_dense(Q, W, K, 2048, rows=rows)
    assert_ok(res)
    assert res.exact == res.rows
