"""The few-row path (at most 64 score rows per batch item): scores go to memory
and one workgroup selects each row. Covers rows short enough to be held whole
in LDS, rows of up to 65536 scores held in registers, longer rows, each
reduced through a threshold taken from a sample, and inputs on which that
threshold passes too few or too many scores, where the exact selection over
the whole row takes over. Scores built from exact bf16 values
must match the oracle exactly, ties going to the lower index."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_ok, check_dense, check_pivot

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def keyed(bits, q_len, H=4, d=32):
    """score(t, s) = the bf16 value with bit pattern bits[s], for every row."""
    L = len(bits)
    x = torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)
    Q = torch.zeros((1, q_len, H, d), dtype=torch.bfloat16, device=DEV)
    Q[:, :, 0, 0] = 1.0
    K = torch.zeros((1, L, d), dtype=torch.bfloat16, device=DEV)
    K[0, :, 0] = x
    W = torch.zeros((1, q_len, H), dtype=torch.float32, device=DEV)
    W[:, :, 0] = 1.0
    return Q, W, K


def keyed2(xbits, ybits, q_len, H=4, d=32):
    """score(t, s) = relu(x[s]) - relu(y[s]) for every row (two heads, weights
    +1 and -1), so that scores can be positive, zero or negative."""
    Q, W, K = keyed(xbits, q_len, H, d)
    y = torch.from_numpy(np.asarray(ybits, np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)
    Q[:, :, 1, 1] = 1.0
    K[0, :, 1] = y
    W[:, :, 1] = -1.0
    return Q, W, K


def reg_sample_positions(n, waves=16, every=8, steps=64):
    """Positions the register-held selection samples in a row of n scores:
    wave w holds a contiguous segment of S positions (S a multiple of 64) in
    steps of 64, and every `every`-th step is sampled."""
    S = -(-n // (waves * 64)) * 64
    out = []
    for w in range(waves):
        b0 = w * S
        ln = max(0, min(S, n - b0))
        for q in range(0, steps, every):
            out.extend(range(b0 + q * 64, b0 + min(ln, q * 64 + 64)))
    return np.asarray(out, np.int64)


def random_inputs(L, q_len, seed, B=1, H=4, d=32):
    # the last q_len positions of B sequences of L keys
    return synth.decode(B, L, q_len, H, d, 0.9, 2, seed, DEV)


@pytest.mark.parametrize("L,q_len,k", [(40001, 5, 2048), (65536, 2, 4096), (20000, 3, 1), (16390, 4, 300),
                                        (65600, 2, 2048), (100003, 3, 4096)])
def test_long_rows_random(L, q_len, k):
    Q, W, K = random_inputs(L, q_len, seed=L + k, B=2)
    res, _, _ = check_dense(Q, W, K, k)
    assert_ok(res)
    assert res.rows == 2 * q_len


def test_rows_near_k():
    # k above the shorter rows (padding) and close to the longer ones
    Q, W, K = random_inputs(40001, 5, seed=9)
    res, idx, _ = check_dense(Q, W, K, 39998)
    assert_ok(res)
    assert (idx[0, 0, 39997:] == -1).all()


@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_pivot_long_rows(variant):
    Q, W, K = random_inputs(30001, 8, seed=5)
    rc, rr, _, _, _ = check_pivot(Q, W, K, 4, 4096, 512, variant)
    assert_ok(rc, rr)


def test_all_equal_scores():
    # every score ties: the threshold passes the whole row, which does not fit
    # in LDS; the exact path must return the lowest indices
    Q, W, K = keyed(np.full(30000, 0x3F80), 2)
    res, idx, _ = check_dense(Q, W, K, 1000)
    assert_ok(res)
    assert res.exact == res.rows
    assert idx[0, 1].tolist() == list(range(1000))


def test_sample_overestimates():
    # odd positions score high and fall with the position, even ones low: a
    # sample of odd positions puts the threshold above the k-th score
    L = 20000
    bits = np.full(L, 0x3C00, np.int64)
    bits[1::2] = 0x4700 - np.arange(L // 2)
    Q, W, K = keyed(bits, 1)
    res, idx, _ = check_dense(Q, W, K, 2048)
    assert_ok(res)
    assert res.exact == res.rows
    assert idx[0, 0].tolist() == list(range(1, 2 * 2048, 2))


@pytest.mark.parametrize("L", [20000, 70000])
def test_sample_chunks_overestimate(L):
    # the sampled positions score high and fall with the position, all others
    # low: the sample puts the threshold above the k-th score of the row.
    # Rows of up to 65536 scores sample every eighth 64-position step of each
    # wave's segment; longer rows 128 chunks of 64 spread evenly.
    k = 2048
    if L <= 65536:
        hot = reg_sample_positions(L)
    else:
        ns = min(L // 2, 8192) // 64 * 64
        nch = ns // 64
        hot = np.concatenate([np.arange(c * L // nch, c * L // nch + 64) for c in range(nch)])
    assert len(hot) >= k
    bits = np.full(L, 0x3C00, np.int64)
    bits[hot] = 0x4700 - np.arange(len(hot))
    Q, W, K = keyed(bits, 1)
    res, idx, _ = check_dense(Q, W, K, k)
    assert_ok(res)
    assert res.exact == res.rows
    assert idx[0, 0].tolist() == sorted(hot[:k].tolist())


def test_threshold_at_zero():
    # positive, exactly zero and negative scores: the sampled threshold is +0,
    # which passes the zeros (not the negatives), and those fit in LDS; the
    # top-k is every positive score and then the lowest-index zeros
    L, k = 20000, 2048
    rng = np.random.default_rng(3)
    kind = rng.permutation(np.repeat([1, 0, -1], [300, 8000, L - 8300]))
    x = np.where(kind > 0, 0x3F80 + rng.integers(0, 64, L), 0)
    y = np.where(kind < 0, 0x3F80 + rng.integers(0, 64, L), 0)
    Q, W, K = keyed2(x, y, 1)
    res, idx, _ = check_dense(Q, W, K, k)
    assert_ok(res)
    assert res.exact == res.rows
    pos = np.flatnonzero(kind > 0)
    zero = np.flatnonzero(kind == 0)[: k - len(pos)]
    assert idx[0, 0].tolist() == sorted(np.concatenate([pos, zero]).tolist())


@pytest.mark.parametrize("plateau", [1, 8, 300])
def test_plateaus_long_row(plateau):
    L = 30000
    bits = 0x0400 + np.arange(L) // plateau  # finite, positive, normal
    Q, W, K = keyed(bits, 3)
    res, _, _ = check_dense(Q, W, K, 2000)
    assert_ok(res)
    assert res.exact == res.rows
