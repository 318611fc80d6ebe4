"""Parity at the full workload sizes, through the same entry points and launch
configuration the benchmark times, checked by the oracle on sampled rows and
groups (first, last and seeded-random ones). The oracle work runs in a pool of
CPU-only worker processes (oracle_pool), which makes samples of the sizes the
plan calls for affordable: 256 stratified rows at 16K, 64 groups (plus the
first and last) at 128K and 1M, every request of the decode step.

Workloads: dense prefill at L=16384; dense/Reuse/Refine at L=131072 (g=4,
c=4096, k=2048); a decode step of 32 requests x 65536 keys (2 rows each,
Refine, c=4096); and dense/Reuse/Refine at L=1048576 (g=16, c=8192).
"""
import gc

import numpy as np
import pytest
import torch

import sparse_attention_indexer_dense_amd as dsa
import synth
from oracle_pool import OraclePool
from parity import HostView, assert_ok, check_dense_rows, check_pivot_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


class Rows:
    """Host copies of selected rows of a [B, R, n] GPU tensor, indexed [b, r]."""

    def __init__(self, t, keys):
        self.d = {}
        if t is None:
            return
        keys = sorted(set(keys))
        bs = torch.tensor([b for b, _ in keys], device=t.device)
        rs = torch.tensor([r for _, r in keys], device=t.device)
        sub = t[bs, rs].cpu().numpy()
        for i, key in enumerate(keys):
            self.d[key] = sub[i]

    def __getitem__(self, key):
        return self.d[key]


def sample(n, head, tail, rand, seed):
    rng = np.random.default_rng(seed)
    s = set(range(min(head, n))) | set(range(max(0, n - tail), n))
    s |= set(rng.integers(0, n, rand).tolist())
    return sorted(s)


def run_dense(Q, W, K, k, rows, pool):
    idx, sc = dsa.dense(Q, W, K, k)
    torch.cuda.synchronize()
    B, q_len = Q.shape[:2]
    L = K.shape[1]
    res = check_dense_rows(Rows(idx, rows), Rows(sc, rows), HostView(Q, W, K), L, q_len, k, rows,
                           pool=pool)
    del idx, sc
    return res


def run_pivot(Q, W, K, g, c, k, variant, groups, pool):
    if variant == "reuse":
        idx, sc, cand = dsa.pivot_reuse(Q, W, K, g, k, c=c, cand=True)
    else:
        idx, sc, cand = dsa.pivot_refine(Q, W, K, g, c, k, cand=True)
    torch.cuda.synchronize()
    B, q_len = Q.shape[:2]
    L = K.shape[1]
    rows = [(b, r) for b, m in groups for r in range(m * g, min(m * g + g, q_len))]
    rc, rr = check_pivot_rows(variant, Rows(idx, rows), Rows(sc, rows), Rows(cand, groups),
                              HostView(Q, W, K), L, q_len, g, c, k, groups, pool=pool)
    del idx, sc, cand
    return rc, rr


def test_dense16k():
    w = synth.WORKLOADS["dense16k"]
    Q, W, K = synth.make(w, device=DEV)
    # stratified: the first 64 rows, the last 64 and 128 seeded-random ones
    rows = [(0, r) for r in sample(w.L, 64, 64, 128, 1)]
    with OraclePool(synth.to_u16(K)) as pool:
        res = run_dense(Q, W, K, w.k, rows, pool)
    assert_ok(res)
    print(res.summary())


@pytest.fixture(scope="module")
def pivot128k():
    w = synth.WORKLOADS["pivot128k"]
    Q, W, K = synth.make(w, device=DEV)
    with OraclePool(synth.to_u16(K)) as pool:
        yield w, Q, W, K, pool
    del Q, W, K
    gc.collect()
    torch.cuda.empty_cache()


def test_pivot128k_dense(pivot128k):
    w, Q, W, K, pool = pivot128k
    rows = [(0, r) for r in sample(w.L, 8, 8, 48, 2)]
    res = run_dense(Q, W, K, w.k, rows, pool)
    assert_ok(res)
    print(res.summary())


@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_pivot128k(pivot128k, variant):
    w, Q, W, K, pool = pivot128k
    G = w.L // w.g
    groups = [(0, m) for m in sample(G, 1, 1, 64, 3)]
    rc, rr = run_pivot(Q, W, K, w.g, w.c, w.k, variant, groups, pool)
    assert_ok(rc, rr)
    print(variant, rc.summary(), rr.summary())


def test_decode64k():
    w = synth.WORKLOADS["decode64k"]
    Q, W, K = synth.make(w, device=DEV)
    reqs = range(w.batch)  # every request
    with OraclePool(synth.to_u16(K)) as pool:
        res = run_dense(Q, W, K, w.k, [(b, r) for b in reqs for r in range(w.g)], pool)
        assert_ok(res)
        rc, rr = run_pivot(Q, W, K, w.g, w.c, w.k, "refine", [(b, 0) for b in reqs], pool)
    assert_ok(rc, rr)
    print(res.summary(), rc.summary(), rr.summary())


@pytest.fixture(scope="module")
def pivot1m():
    w = synth.WORKLOADS["pivot1m"]
    Q, W, K = synth.make(w, device=DEV)
    with OraclePool(synth.to_u16(K)) as pool:
        yield w, Q, W, K, pool
    del Q, W, K
    gc.collect()
    torch.cuda.empty_cache()


def test_pivot1m_dense(pivot1m):
    w, Q, W, K, pool = pivot1m
    rows = [(0, r) for r in sample(w.L, 1, 1, 14, 4)]
    res = run_dense(Q, W, K, w.k, rows, pool)
    assert_ok(res)
    print(res.summary())


@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_pivot1m(pivot1m, variant):
    w, Q, W, K, pool = pivot1m
    G = w.L // w.g
    groups = [(0, m) for m in sample(G, 1, 1, 62, 5)]
    rc, rr = run_pivot(Q, W, K, w.g, w.c, w.k, variant, groups, pool)
    assert_ok(rc, rr)
    print(variant, rc.summary(), rr.summary())
