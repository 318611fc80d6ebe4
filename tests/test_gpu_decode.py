"""The decode form of PIVOT (one group of at most two rows per request, the
MTP drafts of one step: PIVOT Method) through the few-row kernels: both
shapes, Reuse with and without candidates, every proxy strategy, requests of
one and two rows, guarded requests, prefixes shorter than k and c, signed and
exact-integer inputs, a row of equal scores (whose sample threshold admits the
whole row, so the exact path over the row runs), g = 1, and one long request
spread over many workgroups."""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_dense_amd as dsa
import synth
from parity import assert_ok, check_pivot, check_varlen
from test_gpu_varlen import packed

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("shape", [(4, 32), (64, 128)])
@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_decode_uniform(shape, variant):
    H, d = shape
    Q, W, K = synth.decode(5, 9001, 2, H, d, 0.95, 4, seed=3, device=DEV)
    rc, rr, idx, sc, cand = check_pivot(Q, W, K, 2, 1000, 300, variant)
    assert_ok(rc, rr)
    assert rr.rows == 10


@pytest.mark.parametrize("kind,window", [("first", 0), ("last", 0), ("mean", 1), ("mean", 0), ("mean", 5)])
@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_decode_proxy_strategies_mixed_rows(kind, window, variant):
    # requests of two rows and of one row (then the proxy is that row)
    L = [3000, 777, 12345, 64, 5000]
    q = [2, 1, 2, 1, 2]
    Q, W, K = packed(L, q, seed=51)
    g, c, k = 2, 256, 100
    if variant == "reuse":
        out = dsa.pivot_reuse_varlen(Q, W, K, L, q, g, k, c=c, proxy=kind, window=window, cand=True)
    else:
        out = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, proxy=kind, window=window, cand=True)
    rd, rc, rr = check_varlen(variant, Q, W, K, L, q, g, c, k, 0, out, kind=kind, window=window)
    assert_ok(rd, rc, rr)
    assert rr.rows == sum(q)


@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_decode_guard_and_short_prefixes(variant):
    # short requests are guarded (dense rows); others have prefixes shorter
    # than k or c (padding), or long ones
    L = [50, 3000, 180, 700, 20000, 2]
    q = [2, 2, 1, 2, 2, 2]
    Q, W, K = packed(L, q, H=64, d=128, seed=53)
    g, c, k, guard = 2, 512, 128, 100
    if variant == "reuse":
        out = dsa.pivot_reuse_varlen(Q, W, K, L, q, g, k, c=c, guard=guard, cand=True)
    else:
        out = dsa.pivot_refine_varlen(Q, W, K, L, q, g, c, k, guard=guard, cand=True)
    rd, rc, rr = check_varlen(variant, Q, W, K, L, q, g, c, k, guard, out)
    assert_ok(rd, rc, rr)
    assert rd.rows == 4  # the requests of 50 and 2 keys


def test_decode_reuse_without_candidates_equals_with():
    Q, W, K = synth.decode(4, 6000, 2, 64, 128, 0.95, 4, seed=5, device=DEV)
    a_idx, a_sc, _ = dsa.pivot_reuse(Q, W, K, 2, 256)
    b_idx, b_sc, cand = dsa.pivot_reuse(Q, W, K, 2, 256, c=1024, cand=True)
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)
    rc, rr, _, _, _ = check_pivot(Q, W, K, 2, 1024, 256, "reuse")
    assert_ok(rc, rr)


@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_decode_signed_weights(variant):
    Q, _, K = synth.decode(3, 7000, 2, 64, 128, 0.95, 4, seed=7, device=DEV)
    W = synth.signed_weights(6, 64, 7, DEV).view(3, 2, 64).contiguous()
    rc, rr, _, sc, _ = check_pivot(Q, W, K, 2, 700, 200, variant)
    assert_ok(rc, rr)
    # whole rows (k = c = L): every score, negative ones included, is compared
    Q, _, K = synth.decode(2, 3000, 2, 64, 128, 0.95, 4, seed=8, device=DEV)
    W = synth.signed_weights(4, 64, 8, DEV).view(2, 2, 64).contiguous()
    rc, rr, _, sc, _ = check_pivot(Q, W, K, 2, 3000, 3000, variant)
    assert_ok(rc, rr)
    assert (sc[np.isfinite(sc)] < 0).any()


def test_decode_exact_integers():
    # exact scores: every selection equal to the oracle's, ties to the lower index
    gen = torch.Generator(device=DEV)
    gen.manual_seed(21)
    B, L, H, d = 3, 4000, 4, 32
    Q = torch.randint(-2, 3, (B, 2, H, d), generator=gen, device=DEV).to(torch.bfloat16)
    K = torch.randint(-2, 3, (B, L, d), generator=gen, device=DEV).to(torch.bfloat16)
    W = (2.0 ** -torch.randint(0, 4, (B, 2, H), generator=gen, device=DEV)).float()
    for variant in ("reuse", "refine"):
        rc, rr, _, _, _ = check_pivot(Q, W, K, 2, 600, 150, variant)
        assert_ok(rc, rr)
        assert rc.exact == rc.rows and rr.exact == rr.rows and rr.max_rel == 0.0


def test_decode_one_bin_holds_the_row():
    # all-zero queries: every score is 0, the threshold admits the whole row
    # (more than the selection stages in LDS), so the exact path over the row
    # runs; the selections are the lowest indices
    Q, W, K = synth.decode(2, 20000, 2, 64, 128, 0.95, 4, seed=9, device=DEV)
    Q.zero_()
    c, k = 4096, 2048
    idx, sc, cand = dsa.pivot_refine(Q, W, K, 2, c, k, cand=True)
    torch.cuda.synchronize()
    assert torch.equal(cand.cpu(), torch.arange(c, dtype=torch.int32).expand(2, 1, c))
    assert torch.equal(idx.cpu(), torch.arange(k, dtype=torch.int32).expand(2, 2, k))
    assert bool((sc == 0).all())
    u_idx, _, u_cand = dsa.pivot_reuse(Q, W, K, 2, k, c=c, cand=True)
    assert torch.equal(u_idx, idx) and torch.equal(u_cand, cand)


@pytest.mark.parametrize("q_len,g", [(1, 1), (1, 2)])
def test_decode_single_row(q_len, g):
    # one row per request: the proxy is the row, Refine and Reuse are its
    # dense top-k whenever k <= c
    Q, W, K = synth.decode(4, 5000, q_len, 64, 128, 0.95, 4, seed=11, device=DEV)
    d_idx, d_sc = dsa.dense(Q, W, K, 256)
    f_idx, f_sc, _ = dsa.pivot_refine(Q, W, K, g, 512, 256)
    u_idx, u_sc, _ = dsa.pivot_reuse(Q, W, K, g, 256)
    assert torch.equal(d_idx, f_idx) and torch.equal(d_sc, f_sc)
    assert torch.equal(d_idx, u_idx) and torch.equal(d_sc, u_sc)
    rc, rr, _, _, _ = check_pivot(Q, W, K, g, 512, 256, "refine")
    assert_ok(rc, rr)


def test_decode_one_long_request():
    # one request of 131072 keys: many workgroups per row
    Q, W, K = synth.decode(1, 131072, 2, 64, 128, 0.95, 4, seed=13, device=DEV)
    rc, rr, _, _, _ = check_pivot(Q, W, K, 2, 4096, 2048, "refine")
    assert_ok(rc, rr)
