"""PIVOT-Refine on the on-chip re-score kernel (groups of at most four members
and at most 4608 candidates, each member's scores and top-k kept in LDS) at
its limits, against the oracle re-scoring the GPU's own candidates (PIVOT,
Method: member i keeps its own top-k among the candidates causal for it).

Covered: both list capacities it is built for (c = 4096 and c = 4097 .. 4608)
at their edges, beside the first list it does not take (c = 4609, the scan
kernel's Refine); k above 2048 (output slots past the
first half of a row) and above a short group's list (padding); exact-integer
inputs whose rows hold long runs of equal scores (the partial take of equal
keys at the cut); all-zero queries (every score equal: the first k candidates
in index order); three-member groups with a short last group and a stage
count that is odd before padding, on the small shape; and a mix of g, c, k,
lengths and batch sizes on sampled groups."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_ok, check_pivot

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def sample_groups(G, n, seed):
    """First and last n groups and n seeded-random ones in between."""
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(n, G - n), size=n, replace=False)
    return [(0, int(m)) for m in sorted(set(range(n)) | set(range(G - n, G)) | set(mid.tolist()))]


@pytest.mark.parametrize("c", [4096, 4097, 4608, 4609])
def test_refine_list_limit(c):
    L, g, k = 6000, 4, 2048
    Q, W, K = synth.prefill(L, 64, 128, 0.95, 4, seed=71, device=DEV)
    rc, rr, _, _, cand = check_pivot(Q, W, K, g, c, k, "refine", groups=sample_groups(L // g, 6, 2))
    assert_ok(rc, rr)
    # late groups hold a full list of c keys
    assert (cand[0, -1] >= 0).sum() == c
    print(c, rc.summary(), rr.summary())


def test_refine_k_above_half_row():
    L, g, c, k = 5000, 2, 4096, 3000
    Q, W, K = synth.prefill(L, 64, 128, 0.95, 4, seed=72, device=DEV)
    rc, rr, idx, sc, _ = check_pivot(Q, W, K, g, c, k, "refine", groups=sample_groups(L // g, 5, 3))
    assert_ok(rc, rr)
    # early rows keep every causal candidate and pad the rest with -1 / -inf
    assert (idx[0, 0, 1:] == -1).all() and np.isneginf(sc[0, 0, 1:]).all()
    assert (idx[0, -1] >= 0).all()


def test_refine_exact_integer_ties():
    g_ = torch.Generator(device=DEV)
    g_.manual_seed(73)
    L, H, d = 5000, 64, 128
    Q = torch.randint(-1, 2, (1, L, H, d), generator=g_, device=DEV).to(torch.bfloat16)
    K = torch.randint(-1, 2, (1, L, d), generator=g_, device=DEV).to(torch.bfloat16)
    W = (2.0 ** -torch.randint(0, 3, (1, L, H), generator=g_, device=DEV)).float()
    rc, rr, _, _, _ = check_pivot(Q, W, K, 4, 4096, 1000, "refine", groups=sample_groups(L // 4, 4, 4))
    assert_ok(rc, rr)
    assert rr.max_rel == 0.0


def test_refine_all_zero_queries():
    import sparse_attention_indexer_dense_amd as dsa
    L, g, c, k = 4500, 4, 4096, 2048
    Q, W, K = synth.prefill(L, 64, 128, 0.95, 4, seed=74, device=DEV)
    Q.zero_()
    idx, sc, cand = dsa.pivot_refine(Q, W, K, g, c, k, cand=True)
    idx, sc, cand = idx.cpu().numpy(), sc.cpu().numpy(), cand.cpu().numpy()
    assert np.all(sc[np.isfinite(sc)] == 0)
    for r in (0, 1, 2047, 2048, 3333, L - 1):
        m = r // g
        cm = cand[0, m]
        causal = cm[(cm >= 0) & (cm <= r)]
        n = min(k, causal.size)
        assert idx[0, r, :n].tolist() == causal[:n].tolist(), r
        assert (idx[0, r, n:] == -1).all()


def test_refine_three_members_small_shape():
    L, g, c, k = 5001, 3, 300, 100
    Q, W, K = synth.prefill(L, 4, 32, 0.9, 2, seed=75, device=DEV)
    rc, rr, _, _, _ = check_pivot(Q, W, K, g, c, k, "refine", groups=sample_groups((L + g - 1) // g, 8, 5))
    assert_ok(rc, rr)


# (seed, B, L, shape, g, c, k): list lengths below, at and between the two
# capacities, every g the kernel takes, k from small to c, one and two requests
MIX = [
    (81, 1, 777, (4, 32), 1, 130, 17),
    (82, 2, 1300, (4, 32), 2, 257, 256),
    (83, 1, 2049, (4, 32), 3, 2048, 1000),
    (84, 2, 5000, (4, 32), 4, 4500, 4500),
    (85, 1, 4700, (4, 32), 2, 4608, 123),
    (86, 1, 3000, (64, 128), 3, 1000, 999),
]


@pytest.mark.parametrize("case", MIX, ids=[f"mix{i}" for i in range(len(MIX))])
def test_refine_parameter_mix(case):
    seed, B, L, (H, d), g, c, k = case
    Qs, Ws, Ks = [], [], []
    for b in range(B):
        Q, W, K = synth.prefill(L, H, d, 0.9, 2, seed + 13 * b, DEV)
        Qs.append(Q)
        Ws.append(W)
        Ks.append(K)
    Q, W, K = torch.cat(Qs), torch.cat(Ws), torch.cat(Ks)
    G = -(-L // g)
    groups = [(b, m) for b in range(B) for _, m in sample_groups(G, 4, seed)]
    rc, rr, _, _, _ = check_pivot(Q, W, K, g, c, k, "refine", groups=groups)
    assert_ok(rc, rr)
