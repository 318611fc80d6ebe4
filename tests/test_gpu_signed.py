"""Head weights of either sign through the many-row fused scan kernel.

Nothing in the index score (PIVOT, observation-O3 paragraph: a per-head ReLU
of q.k, then a weighted sum over the heads) makes the weights non-negative, and
the C ABI accepts any fp32 W. With signed weights scores can be negative, zero
by cancellation between heads, and the admission threshold and radix bins run
through the negative half of the key order. Every request here has more than
64 query rows, so the dense pass, the proxy scan (Reuse with candidates) and
Refine all run on the fused scan kernel, for both supported shapes; one case
forces the candidate buffer's compaction with negative scores only."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_ok, check_dense, check_pivot

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def signed(L, H, d, rho, rank, seed):
    Q, _, K = synth.prefill(L, H, d, rho, rank, seed, DEV)
    W = synth.signed_weights(L, H, seed, DEV)[None]
    return Q, W, K


def spread_rows(L, n, seed):
    """First and last n rows and n seeded-random ones in between."""
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(n, L - n), size=n, replace=False)
    return [(0, int(r)) for r in sorted(set(range(n)) | set(range(L - n, L)) | set(mid.tolist()))]


@pytest.mark.parametrize("shape", [(4, 32), (64, 128)])
def test_signed_dense(shape):
    H, d = shape
    L = 2048 if H == 4 else 1200
    Q, W, K = signed(L, H, d, 0.9, 2, 41)
    rows = None if H == 4 else spread_rows(L, 48, 1)
    res, idx, sc = check_dense(Q, W, K, 64 if H == 4 else 256, rows=rows)
    assert_ok(res)
    assert (sc[np.isfinite(sc)] < 0).any(), "no negative score was selected"
    print(res.summary())


@pytest.mark.parametrize("shape", [(4, 32), (64, 128)])
@pytest.mark.parametrize("variant", ["reuse", "refine"])
def test_signed_pivot(shape, variant):
    H, d = shape
    L = 2048 if H == 4 else 1200
    g, c, k = (4, 128, 64) if H == 4 else (4, 512, 256)
    Q, W, K = signed(L, H, d, 0.9, 2, 43)
    rc, rr, idx, sc, cand = check_pivot(Q, W, K, g, c, k, variant)
    assert_ok(rc, rr)
    print(rc.summary(), rr.summary())


def integer_inputs(L, H, d, seed):
    """Small-integer queries and keys, weights +-2^-j: every score is exact in
    fp32 (negative, zero and positive), so scores must match bit for bit and
    the many ties fall to the lower index."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    Q = torch.randint(-2, 3, (1, L, H, d), generator=gen, device=DEV).to(torch.bfloat16)
    K = torch.randint(-2, 3, (1, L, d), generator=gen, device=DEV).to(torch.bfloat16)
    sign = torch.randint(0, 2, (1, L, H), generator=gen, device=DEV).float() * 2 - 1
    W = sign * (2.0 ** -torch.randint(0, 4, (1, L, H), generator=gen, device=DEV)).float()
    # rows whose heads cancel: two heads with equal queries and opposite weights
    Q[:, ::3, 1] = Q[:, ::3, 0]
    W[:, ::3, 1] = -W[:, ::3, 0]
    W[:, ::3, 2:] = 0.0
    return Q, W, K


@pytest.mark.parametrize("shape", [(4, 32), (64, 128)])
def test_signed_exact_integers(shape):
    H, d = shape
    L = 1500 if H == 4 else 700
    Q, W, K = integer_inputs(L, H, d, 9)
    res, idx, sc = check_dense(Q, W, K, 100)
    assert_ok(res)
    assert res.exact == res.rows and res.max_rel == 0.0
    zero = sc == 0
    assert zero.any() and (sc < 0).any()
    # a zero score is written as +0 (the kernel folds -0 into +0)
    assert not np.signbit(sc[zero]).any()
    for variant in ("reuse", "refine"):
        rc, rr, _, _, _ = check_pivot(Q, W, K, 4, 160, 100, variant)
        assert_ok(rc, rr)
        assert rc.exact == rc.rows and rr.exact == rr.rows


def rising_negative(L, plateau, H, d):
    """score(t, s) = -x_s with x_s > 0 falling in s: every new key outranks the
    keys before it, so the candidate buffers fill and are compacted, with
    negative scores only (exact in fp32)."""
    bits = (0x4780 - np.arange(L) // plateau).astype(np.uint16)  # 65536 and down
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    Q = torch.zeros((1, L, H, d), dtype=torch.bfloat16, device=DEV)
    Q[:, :, 0, 0] = 1.0
    Q[:, :, 1, 0] = -1.0  # second head: always ReLU'd away
    K = torch.zeros((1, L, d), dtype=torch.bfloat16, device=DEV)
    K[:, :, 0] = x
    W = torch.zeros((1, L, H), dtype=torch.float32, device=DEV)
    W[:, :, 0] = -1.0
    W[:, :, 1] = 0.5
    return Q, W, K


@pytest.mark.parametrize("shape", [(4, 32), (64, 128)])
def test_signed_compaction(shape):
    H, d = shape
    L = 5000
    Q, W, K = rising_negative(L, 2, H, d)
    rows = None if H == 4 else [(0, r) for r in (0, 63, 64, 1000, 1001, 2047, 2048, 4999)]
    res, idx, sc = check_dense(Q, W, K, 64, rows=rows)
    assert_ok(res)
    assert res.exact == res.rows
    assert (sc[np.isfinite(sc)] < 0).all()
    for r in (63, 1001, 4999):
        # whole pairs of equal scores: the most recent 64 keys
        assert idx[0, r].tolist() == list(range(r - 63, r + 1)), r
    # r = 1000 ends on half a pair: keys 936 and 937 tie at the cut and the
    # lower index is kept
    assert idx[0, 1000].tolist() == [936] + list(range(938, 1001))
    if H == 4:
        for variant in ("reuse", "refine"):
            rc, rr, _, _, _ = check_pivot(Q, W, K, 4, 200, 64, variant)
            assert_ok(rc, rr)
            assert rc.exact == rc.rows and rr.exact == rr.rows
