"""indexer_sort_rows: rows reordered into ranking order (score descending,
equal scores by ascending index, -1 padding last). Checked against a lexsort
of the same rows (exact), against the oracle's ranking order of the dense
indexer (up to scores within the parity tolerance of each other), on ties,
padding, the largest k and more rows than one grid dimension holds."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_dense_amd as dsa
import synth
from checker import MTOL, RTOL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def ranking(idx, sc):
    """Reference order of one row: lexsort on (-score, index), padding last."""
    pad = idx < 0
    order = np.lexsort((idx, -sc.astype(np.float64)))
    order = np.concatenate([order[~pad[order]], order[pad[order]]])
    return idx[order], sc[order]


def check_rows(i0, s0, i1, s1):
    for r in range(i0.shape[0]):
        wi, ws = ranking(i0[r], s0[r])
        assert np.array_equal(i1[r], wi), r
        assert np.array_equal(s1[r].view(np.uint32), ws.astype(np.float32).view(np.uint32)), r


def test_sort_dense_rows_tiny():
    Q, W, K = synth.prefill(2048, 4, 32, 0.9, 2, 3, DEV)
    idx, sc = dsa.dense(Q, W, K, 64)
    i0, s0 = idx.cpu().numpy()[0], sc.cpu().numpy()[0]
    dsa.sort_rows(idx, sc)
    torch.cuda.synchronize()
    i1, s1 = idx.cpu().numpy()[0], sc.cpu().numpy()[0]
    check_rows(i0, s0, i1, s1)
    # against the oracle's order: oracle scores never rise by more than the
    # tolerance along a sorted row, and the first rows (short prefixes) pad last
    Qh, Wh, Kh = synth.to_u16(Q[0]), W[0].cpu().numpy(), synth.to_u16(K[0])
    for r in (0, 5, 63, 64, 1000, 2047):
        ref, mass = oracle.scores(Qh[r], Wh[r], Kh, n=r + 1)
        row = i1[r][i1[r] >= 0]
        assert row.size == min(64, r + 1)
        tol = RTOL * np.abs(ref) + MTOL * mass
        v = ref[row]
        assert np.all(v[1:] <= v[:-1] + tol[row][1:] + tol[row][:-1]), r
        if r < 64:  # the whole prefix is selected
            assert sorted(row.tolist()) == list(range(r + 1))


def test_sort_ties_and_padding():
    k, rows = 100, 7
    sc = torch.zeros((rows, k), dtype=torch.float32, device=DEV)
    idx = torch.arange(k, dtype=torch.int32, device=DEV).flip(0).repeat(rows, 1).contiguous()
    sc[:, 90:] = -float("inf")
    idx[:, 90:] = -1
    sc[3, :5] = -0.0
    i0, s0 = idx.cpu().numpy(), sc.cpu().numpy()
    dsa.sort_rows(idx, sc)
    torch.cuda.synchronize()
    i1 = idx.cpu().numpy()
    for r in range(rows):
        assert i1[r][:90].tolist() == sorted(i0[r][:90].tolist())  # equal scores: ascending index
        assert np.all(i1[r][90:] == -1)
    assert np.all(sc.cpu().numpy()[:, :90] == 0.0)


@pytest.mark.parametrize("rows,k", [(3, 8192), (70000, 16), (513, 1000)])
def test_sort_random_rows(rows, k):
    g = torch.Generator(device=DEV).manual_seed(rows + k)
    sc = torch.randn((rows, k), generator=g, device=DEV).to(torch.bfloat16).float()  # many exact ties
    idx = torch.randperm(k * 4, generator=g, device=DEV)[:k].int().repeat(rows, 1).contiguous()
    i0, s0 = idx.cpu().numpy(), sc.cpu().numpy()
    dsa.sort_rows(idx, sc)
    torch.cuda.synchronize()
    i1, s1 = idx.cpu().numpy(), sc.cpu().numpy()
    pick = sorted(set([0, rows - 1, rows // 2]) | set(np.random.default_rng(k).integers(0, rows, 20).tolist()))
    check_rows(i0[pick], s0[pick], i1[pick], s1[pick])
