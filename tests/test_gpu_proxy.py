"""Proxy aggregation strategies of PIVOT (endpoint queries, mean over a window
of members) through the *_varlen entry points, against the oracle computing
the same proxy; both kernel families; groups of 4 and of 16 (window 4)."""
import pytest
import torch

import sparse_attention_indexer_dense_amd as dsa
from parity import assert_ok, check_varlen
from test_gpu_varlen import SCAN, SPLIT, packed

pytestmark = pytest.mark.gpu

STRATEGIES = [("first", 0), ("last", 0), ("mean", 2), ("mean", 3), ("mean", 0)]


@pytest.mark.parametrize("shape", [SCAN, SPLIT], ids=["scan", "split"])
@pytest.mark.parametrize("kind,window", STRATEGIES)
@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_proxy_strategies(shape, kind, window, variant):
    L, q = shape
    Q, W, K = packed(L, q, seed=31)
    g, c, k = 4, 128, 64
    if variant == "reuse":
        out = dsa.pivot_reuse_varlen(Q, W, K, L, q, g, k, c=c, proxy=kind, window=window, cand=True)
    else:
        out = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, proxy=kind, window=window, cand=True)
    rd, rc, rr = check_varlen(variant, Q, W, K, L, q, g, c, k, 0, out, kind=kind, window=window)
    assert_ok(rd, rc, rr)
    assert rr.rows == sum(q)


@pytest.mark.parametrize("window", [4, 0])
def test_window4_at_g16(window):
    L, q = [4096, 2500], [4096, 2500]
    Q, W, K = packed(L, q, H=64, d=128, seed=37)
    g, c, k = 16, 1024, 256
    out = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, proxy="mean", window=window, cand=True)
    rd, rc, rr = check_varlen("refine", Q, W, K, L, q, g, c, k, 0, out, max_groups=12,
                              kind="mean", window=window)
    assert_ok(rd, rc, rr)


def test_window_wider_than_group_is_group_mean():
    L, q = SCAN
    Q, W, K = packed(L, q, seed=41)
    a = dsa.pivot_refine_varlen(Q, W, K, L, q, 4, 128, 64, proxy="mean", window=0, cand=True)
    b = dsa.pivot_refine_varlen(Q, W, K, L, q, 4, 128, 64, proxy="mean", window=9, cand=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
