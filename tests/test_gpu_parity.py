"""GPU parity at sizes the oracle checks in seconds: every row, several tiles,
ragged tails, batches, both kernel families (many-row fused scan, few-row split
scan), ties, exact-integer inputs and the PIVOT reductions (g = 1, c >= L)."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_ok, check_dense, check_pivot

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def tiny(seed=0, L=2048, H=4, d=32, rho=0.9, rank=2, batch=1):
    Qs, Ws, Ks = [], [], []
    for b in range(batch):
        Q, W, K = synth.prefill(L, H, d, rho, rank, seed + 97 * b, DEV)
        Qs.append(Q)
        Ws.append(W)
        Ks.append(K)
    return torch.cat(Qs), torch.cat(Ws), torch.cat(Ks)


def test_dense_tiny_full_rows():
    # k = L: the selection of every row is its whole causal prefix, so every
    # score of the lower triangle is compared with the oracle
    Q, W, K = tiny()
    res, idx, _ = check_dense(Q, W, K, 2048)
    assert_ok(res)
    assert res.exact == res.rows == 2048


def test_dense_tiny_k64():
    Q, W, K = tiny()
    res, _, _ = check_dense(Q, W, K, 64)
    assert_ok(res)
    print(res.summary())


def test_dense_ragged_batch():
    Q, W, K = tiny(seed=5, L=1000, batch=2)
    res, _, _ = check_dense(Q, W, K, 37)
    assert_ok(res)


def test_dense_few_rows_split_path():
    # q_len <= 64 rows: the split-key kernels; k > L pads with -1
    Q, W, K = synth.decode(3, 777, 5, 4, 32, 0.95, 2, seed=3, device=DEV)
    for k in (50, 1000):
        res, idx, _ = check_dense(Q, W, K, k)
        assert_ok(res)


def test_dense_all_zero_queries_tie_to_lowest_index():
    Q, W, K = tiny(seed=1, L=700)
    Q.zero_()
    res, idx, sc = check_dense(Q, W, K, 64)
    assert_ok(res)
    for r in range(700):
        n = min(64, r + 1)
        assert idx[0, r, :n].tolist() == list(range(n))
        assert np.all(sc[0, r, :n] == 0)


def test_dense_exact_integer_inputs():
    # small integers and power-of-two weights: every score is exact in fp32,
    # so scores must match bit for bit and sets exactly (many equal scores)
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    L, H, d = 1500, 4, 32
    Q = torch.randint(-2, 3, (1, L, H, d), generator=g, device=DEV).to(torch.bfloat16)
    K = torch.randint(-2, 3, (1, L, d), generator=g, device=DEV).to(torch.bfloat16)
    W = (2.0 ** -torch.randint(0, 4, (1, L, H), generator=g, device=DEV)).float()
    res, idx, sc = check_dense(Q, W, K, 100)
    assert_ok(res)
    assert res.exact == res.rows and res.max_rel == 0.0


@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_pivot_tiny(variant):
    Q, W, K = tiny()
    rc, rr, _, _, _ = check_pivot(Q, W, K, 4, 128, 64, variant)
    assert_ok(rc, rr)
    print(variant, rc.summary(), rr.summary())


def test_reuse_without_candidates():
    Q, W, K = tiny(seed=2)
    rc, rr, _, _, cand = check_pivot(Q, W, K, 4, 128, 64, "reuse", with_cand=False)
    assert cand is None
    assert_ok(rr)


@pytest.mark.parametrize("g", [3, 16])
@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_pivot_ragged_groups(variant, g):
    # q_len not a multiple of g: the last group is short
    Q, W, K = tiny(seed=4, L=1001, batch=2)
    rc, rr, _, _, _ = check_pivot(Q, W, K, g, 100, 30, variant)
    assert_ok(rc, rr)


@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_pivot_decode_shape(variant):
    # decode: q_len = g new rows per request, one group each (split kernels)
    Q, W, K = synth.decode(4, 3000, 2, 4, 32, 0.95, 2, seed=9, device=DEV)
    rc, rr, _, _, _ = check_pivot(Q, W, K, 2, 256, 64, variant)
    assert_ok(rc, rr)


def test_g1_reuse_and_refine_equal_dense():
    import sparse_attention_indexer_dense_amd as dsa
    Q, W, K = tiny(seed=6, L=900)
    d_idx, d_sc = dsa.dense(Q, W, K, 40)
    u_idx, u_sc, _ = dsa.pivot_reuse(Q, W, K, 1, 40)
    f_idx, f_sc, _ = dsa.pivot_refine(Q, W, K, 1, 80, 40)
    assert torch.equal(d_idx, u_idx) and torch.equal(d_sc, u_sc)
    assert torch.equal(d_idx, f_idx) and torch.equal(d_sc, f_sc)


def test_refine_with_c_ge_L_equals_dense():
    import sparse_attention_indexer_dense_amd as dsa
    Q, W, K = tiny(seed=8, L=900)
    d_idx, d_sc = dsa.dense(Q, W, K, 40)
    f_idx, f_sc, _ = dsa.pivot_refine(Q, W, K, 4, 900, 40)
    assert torch.equal(d_idx, f_idx) and torch.equal(d_sc, f_sc)


def test_dense_h64_d128_rows():
    Q, W, K = synth.prefill(3000, 64, 128, 0.95, 4, seed=11, device=DEV)
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 1, 2, 63, 64, 255, 256, 2047, 2048, 2999] + rng.integers(0, 3000, 40).tolist()))
    res, _, _ = check_dense(Q, W, K, 256, rows=[(0, r) for r in rows])
    assert_ok(res)
    print(res.summary())


@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_pivot_h64_d128(variant):
    Q, W, K = synth.prefill(3000, 64, 128, 0.95, 4, seed=12, device=DEV)
    rng = np.random.default_rng(1)
    groups = sorted(set([0, 1, 749] + rng.integers(0, 750, 12).tolist()))
    rc, rr, _, _, _ = check_pivot(Q, W, K, 4, 512, 256, variant, groups=[(0, m) for m in groups])
    assert_ok(rc, rr)
    print(variant, rc.summary(), rr.summary())


def test_decode_h64_d128():
    Q, W, K = synth.decode(3, 5000, 2, 64, 128, 0.95, 4, seed=13, device=DEV)
    res, _, _ = check_dense(Q, W, K, 512)
    assert_ok(res)
    rc, rr, _, _, _ = check_pivot(Q, W, K, 2, 1024, 512, "refine")
    assert_ok(rc, rr)


def test_deterministic_repeat():
    import sparse_attention_indexer_dense_amd as dsa
    Q, W, K = tiny(seed=10)
    a = dsa.pivot_refine(Q, W, K, 4, 128, 64, cand=True)
    b = dsa.pivot_refine(Q, W, K, 4, 128, 64, cand=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_binding_rejects_mismatched_outputs():
    # caller-provided outputs are checked before any launch: wrong shape,
    # dtype or device never reach the kernels
    import sparse_attention_indexer_dense_amd as dsa
    Q, W, K = tiny(L=256)
    k = 16
    good = torch.empty((1, 256, k), dtype=torch.int32, device=DEV)
    score = torch.empty((1, 256, k), dtype=torch.float32, device=DEV)
    bad = [
        (torch.empty((1, 256, k - 1), dtype=torch.int32, device=DEV), score),
        (torch.empty((1, 256, k), dtype=torch.int64, device=DEV), score),
        (torch.empty((1, 256, k), dtype=torch.int32), score),
        (good, torch.empty((1, 255, k), dtype=torch.float32, device=DEV)),
        (torch.empty((1, k, 256), dtype=torch.int32, device=DEV).transpose(1, 2), score),
    ]
    for out in bad:
        with pytest.raises(ValueError):
            dsa.dense(Q, W, K, k, out=out)
    with pytest.raises(ValueError):
        dsa.pivot_refine(Q, W, K, 4, 32, k, out=(good, score, torch.empty((1, 63, 32), dtype=torch.int32,
                                                                             device=DEV)))
    i, s = dsa.dense(Q, W, K, k, out=(good, score))
    assert i.data_ptr() == good.data_ptr()
