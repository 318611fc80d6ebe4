"""Batches of requests of different lengths, through the *_varlen entry points:
every request's rows against the oracle run on that request alone; groups
never reach into a neighbouring request; the guard scores short groups as
dense rows. Covers the scan (many rows) and split-key (few rows) paths, short
last groups, q_len < L, a request shorter than k, requests without queries
(with or without keys), and the guard's limits."""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_dense_amd as dsa
import synth
from parity import assert_ok, check_varlen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed(L, q_len, H=4, d=32, seed=0):
    """Packed Q, W, K of requests whose queries are their last q_len positions."""
    Qs, Ws, Ks = [], [], []
    for i, (Lb, qb) in enumerate(zip(L, q_len)):
        if qb == Lb:
            Q, W, K = synth.prefill(Lb, H, d, 0.9, 2, seed + i, DEV)
        else:
            Q, W, K = synth.decode(1, Lb, qb, H, d, 0.9, 2, seed + i, DEV)
        Qs.append(Q[0])
        Ws.append(W[0])
        Ks.append(K[0])
    return torch.cat(Qs).contiguous(), torch.cat(Ws).contiguous(), torch.cat(Ks).contiguous()


# many rows per request (scan kernels) and few rows (split-key kernels)
SCAN = ([1000, 3001, 257, 700], [1000, 120, 257, 65])
SPLIT = ([5000, 1200, 300, 9000, 77], [2, 3, 1, 2, 3])


@pytest.mark.parametrize("shape", [SCAN, SPLIT], ids=["scan", "split"])
def test_dense_varlen(shape):
    L, q = shape
    Q, W, K = packed(L, q)
    idx, sc = dsa.dense_varlen(Q, W, K, L, q, 64)
    res, _, _ = check_varlen("dense", Q, W, K, L, q, 1, 0, 64, 0, (idx, sc, None))
    assert_ok(res)
    assert res.rows == sum(q)


@pytest.mark.parametrize("shape", [SCAN, SPLIT], ids=["scan", "split"])
@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_pivot_varlen(shape, variant):
    L, q = shape
    Q, W, K = packed(L, q, seed=3)
    g, c, k = 4, 128, 64
    if variant == "reuse":
        out = dsa.pivot_reuse_varlen(Q, W, K, L, q, g, k, c=c, cand=True)
    else:
        out = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, cand=True)
    rd, rc, rr = check_varlen(variant, Q, W, K, L, q, g, c, k, 0, out)
    assert_ok(rd, rc, rr)
    assert rd.rows == 0 and rr.rows == sum(q)


@pytest.mark.parametrize("g", [2, 3, 6])
def test_refine_split_rows_per_wave(g):
    # few rows per request (split-key kernels): with an even g a wave scores
    # two member rows of a group on each gathered tile, with an odd g one;
    # counts of 1, 3 and 5 rows leave a pair's second row missing or a short
    # last group
    L, q = [3000, 9000, 700, 5000], [3, 5, 1, 6]
    Q, W, K = packed(L, q, seed=11)
    c, k = 256, 64
    out = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, cand=True)
    rd, rc, rr = check_varlen("refine", Q, W, K, L, q, g, c, k, 0, out)
    assert_ok(rd, rc, rr)
    assert rr.rows == sum(q)


def test_reuse_varlen_without_candidates():
    L, q = SCAN
    Q, W, K = packed(L, q, seed=5)
    out = dsa.pivot_reuse_varlen(Q, W, K, L, q, 4, 64)
    rd, rc, rr = check_varlen("reuse", Q, W, K, L, q, 4, 0, 64, 0, out)
    assert_ok(rd, rc, rr)


@pytest.mark.parametrize("guard", [64, 600, 3001])
@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_guard(variant, guard):
    L, q = SCAN
    Q, W, K = packed(L, q, seed=7)
    g, c, k = 4, 128, 64
    f = dsa.pivot_reuse_varlen if variant == "reuse" else dsa.pivot_refine_varlen
    out = (f(Q, W, K, L, q, g, k, c=c, guard=guard, cand=True) if variant == "reuse"
           else f(Q, W, K, L, q, g, c, k, guard=guard, cand=True))
    rd, rc, rr = check_varlen(variant, Q, W, K, L, q, g, c, k, guard, out)
    assert_ok(rd, rc, rr)
    assert rd.rows > 0
    if guard >= max(L):
        assert rr.rows == 0  # everything dense


@pytest.mark.parametrize("shape", [SCAN, SPLIT], ids=["scan", "split"])
def test_refine_guard_up_to_c_changes_nothing(shape):
    L, q = shape
    Q, W, K = packed(L, q, seed=11)
    g, c, k = 4, 512, 64
    i0, s0, _ = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k)
    i1, s1, _ = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, guard=c)
    assert torch.equal(i0, i1)
    assert torch.equal(s0, s1)


@pytest.mark.parametrize("variant", ["dense", "reuse", "refine"])
def test_equal_lengths_match_uniform_batch(variant):
    B, L, q = 3, 2000, 300
    Qs, Ws, Ks = [], [], []
    for b in range(B):
        Q, W, K = synth.decode(1, L, q, 4, 32, 0.9, 2, 20 + b, DEV)
        Qs.append(Q)
        Ws.append(W)
        Ks.append(K)
    Qu, Wu, Ku = torch.cat(Qs), torch.cat(Ws), torch.cat(Ks)
    Qv, Wv, Kv = Qu.reshape(B * q, 4, 32), Wu.reshape(B * q, 4), Ku.reshape(B * L, 32)
    g, c, k = 4, 256, 64
    if variant == "dense":
        iu, su = dsa.dense(Qu, Wu, Ku, k)
        iv, sv = dsa.dense_varlen(Qv, Wv, Kv, [L] * B, [q] * B, k)
    elif variant == "reuse":
        iu, su, _ = dsa.pivot_reuse(Qu, Wu, Ku, g, k)
        iv, sv, _ = dsa.pivot_reuse_varlen(Qv, Wv, Kv, [L] * B, [q] * B, g, k)
    else:
        iu, su, _ = dsa.pivot_refine(Qu, Wu, Ku, g, c, k)
        iv, sv, _ = dsa.pivot_refine_varlen(Qv, Wv, Kv, [L] * B, [q] * B, g, c, k)
    assert torch.equal(iu.reshape(B * q, k), iv)
    assert torch.equal(su.reshape(B * q, k), sv)


def test_h64_d128_mixed():
    L, q = [2500, 700, 4096], [2500, 5, 33]
    Q, W, K = packed(L, q, H=64, d=128, seed=13)
    g, c, k = 4, 512, 256
    out = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, guard=800, cand=True)
    rd, rc, rr = check_varlen("refine", Q, W, K, L, q, g, c, k, 800, out, max_groups=24)
    assert_ok(rd, rc, rr)


def test_decode_batch_of_lengths():
    # a decode step of requests with different cache lengths, 2 new rows each
    L = [40000, 7000, 65536, 12289, 3000, 20000]
    q = [2] * len(L)
    Q, W, K = packed(L, q, H=64, d=128, seed=17)
    g, c, k = 2, 4096, 2048
    out = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, cand=True)
    rd, rc, rr = check_varlen("refine", Q, W, K, L, q, g, c, k, 0, out)
    assert_ok(rd, rc, rr)
    d_idx, d_sc = dsa.dense_varlen(Q, W, K, L, q, k)
    res, _, _ = check_varlen("dense", Q, W, K, L, q, 1, 0, k, 0, (d_idx, d_sc, None))
    assert_ok(res)


def packed_with_empty(L, q_len, H=4, d=32, seed=0):
    """As packed(), where a request with q_len = 0 brings only its keys (none
    if L = 0)."""
    Qs, Ws, Ks = [], [], []
    for i, (Lb, qb) in enumerate(zip(L, q_len)):
        if qb > 0:
            Q, W, K = packed([Lb], [qb], H, d, seed + i)
        else:
            Q = torch.empty((0, H, d), dtype=torch.bfloat16, device=DEV)
            W = torch.empty((0, H), dtype=torch.float32, device=DEV)
            K = (synth.decode(1, Lb, 1, H, d, 0.9, 2, seed + i, DEV)[2][0] if Lb > 0
                 else torch.empty((0, d), dtype=torch.bfloat16, device=DEV))
        Qs.append(Q)
        Ws.append(W)
        Ks.append(K)
    return torch.cat(Qs).contiguous(), torch.cat(Ws).contiguous(), torch.cat(Ks).contiguous()


# requests without queries (with and without keys) among ordinary ones, on
# the scan path (up to 120 rows per request) and the split-key path
EMPTY_SCAN = ([0, 3001, 500, 0, 700, 9000], [0, 120, 0, 0, 65, 2])
EMPTY_SPLIT = ([0, 5000, 300, 9000], [0, 2, 0, 3])


@pytest.mark.parametrize("shape", [EMPTY_SCAN, EMPTY_SPLIT], ids=["scan", "split"])
@pytest.mark.parametrize("variant", ["dense", "reuse", "refine"])
def test_empty_requests(shape, variant):
    L, q = shape
    Q, W, K = packed_with_empty(L, q, seed=11)
    g, c, k = 4, 128, 64
    if variant == "dense":
        idx, sc = dsa.dense_varlen(Q, W, K, L, q, k)
        out = (idx, sc, None)
    elif variant == "reuse":
        out = dsa.pivot_reuse_varlen(Q, W, K, L, q, g, k, c=c, cand=True)
    else:
        out = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, cand=True)
    rd, rc, rr = check_varlen(variant, Q, W, K, L, q, g, c, k, 0, out)
    assert_ok(rd, rc, rr)
    assert out[0].shape[0] == sum(q)
    assert rd.rows + rr.rows == sum(q)


def test_all_requests_empty():
    # no request has queries: the calls return empty outputs and touch nothing
    L, q = [0, 300, 0], [0, 0, 0]
    Q = torch.empty((0, 4, 32), dtype=torch.bfloat16, device=DEV)
    W = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    K = synth.decode(1, 300, 1, 4, 32, 0.9, 2, 0, DEV)[2][0].contiguous()
    idx, sc = dsa.dense_varlen(Q, W, K, L, q, 64)
    assert tuple(idx.shape) == (0, 64)
    idx, sc, cand = dsa.pivot_refine_varlen(Q, W, K, L, q, 4, 128, 64, cand=True)
    assert tuple(idx.shape) == (0, 64) and tuple(cand.shape) == (0, 128)
    idx, sc, cand = dsa.pivot_reuse_varlen(Q, W, K, L, q, 4, 64, c=128, cand=True)
    assert tuple(idx.shape) == (0, 64) and tuple(cand.shape) == (0, 128)
    torch.cuda.synchronize()
