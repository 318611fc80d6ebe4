"""The guard on the key-chunk path (PIVOT, results, the guardrail paragraph:
short groups fall back to the dense indexer): the rows of every group whose
causal prefix holds at most `guard` keys are the dense indexer's rows (checked
against the oracle), their selected-chunk and candidate rows are -1, and every
other group's chunks, list and rows are those of the unguarded call, bit for
bit. Both kernel families, the on-chip Refine, every group guarded, and the
variable-length form."""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_dense_amd as dsa
import synth
from parity import HostView, assert_ok, check_dense_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(Q, W, K, block, g, nsel, k, guard):
    B, L = K.shape[:2]
    cend = dsa.chunks_fixed(B, L, block, DEV)
    Kbar = dsa.chunk_means(K, cend)
    o = dsa.chunk_refine(Q, W, K, Kbar, cend, g, nsel, block, k, chunks=True, cand=True, guard=guard)
    torch.cuda.synchronize()
    return o


def check_guard(Q, W, K, block, g, nsel, k, guard, dense_rows_checked=None):
    B, q_len = Q.shape[:2]
    L = K.shape[1]
    G = -(-q_len // g)
    o0 = run(Q, W, K, block, g, nsel, k, 0)
    og = run(Q, W, K, block, g, nsel, k, guard)
    # guarded groups: t_last + 1 <= guard, a prefix of the groups
    t_last = [L - q_len + min(m * g + g, q_len) - 1 for m in range(G)]
    m0 = sum(1 for t in t_last if t + 1 <= guard)
    rg = min(m0 * g, q_len)
    idx, sc = og[0].cpu().numpy(), og[1].cpu().numpy()
    rows = list(range(rg)) if dense_rows_checked is None else [r for r in dense_rows_checked if r < rg]
    res = check_dense_rows(idx, sc, HostView(Q, W, K), L, q_len, k, [(b, r) for b in range(B) for r in rows])
    assert_ok(res)
    assert bool((og[2][:, :m0] == -1).all()) and bool((og[3][:, :m0] == -1).all())
    for a, b_ in ((og[0], o0[0]), (og[1], o0[1])):
        assert torch.equal(a[:, rg:], b_[:, rg:])
    for a, b_ in ((og[2], o0[2]), (og[3], o0[3])):
        assert torch.equal(a[:, m0:], b_[:, m0:])
    return m0, G


@pytest.mark.parametrize("guard", [600, 2048])
def test_chunk_guard_scan_kernels(guard):
    Q, W, K = synth.prefill(2048, 4, 32, 0.9, 2, 91, DEV)
    m0, G = check_guard(Q, W, K, 64, 4, 6, 64, guard, dense_rows_checked=range(0, 2048, 7))
    assert (m0 == G) == (guard >= 2048) and m0 > 0


def test_chunk_guard_split_kernels():
    # few rows per request: group 0 guarded, group 1 on the chunk path
    Q, W, K = synth.decode(2, 5000, 8, 4, 32, 0.95, 2, seed=92, device=DEV)
    m0, G = check_guard(Q, W, K, 64, 4, 8, 64, 4997)
    assert (m0, G) == (1, 2)


def test_chunk_guard_onchip_refine():
    Q, W, K = synth.prefill(3000, 64, 128, 0.95, 4, 93, DEV)
    m0, G = check_guard(Q, W, K, 64, 4, 16, 256, 1000, dense_rows_checked=range(0, 1000, 37))
    assert m0 == 250


def test_chunk_guard_varlen_equals_per_request():
    L, q_len, g, block, nsel, k, guard = [2048, 1000, 900], [2048, 3, 900], 4, 64, 6, 64, 700
    reqs = []
    for r, (Lr, qr) in enumerate(zip(L, q_len)):
        Q, W, K = synth.prefill(Lr, 4, 32, 0.9, 2, 94 + r, DEV)
        reqs.append((Q[0, Lr - qr:].contiguous(), W[0, Lr - qr:].contiguous(), K[0].contiguous()))
    Q = torch.cat([x[0] for x in reqs])
    W = torch.cat([x[1] for x in reqs])
    K = torch.cat([x[2] for x in reqs])
    cend, nc = dsa.chunks_fixed_varlen(L, block, DEV)
    Kbar = dsa.chunk_means_varlen(K, L, cend, nc)
    out = dsa.chunk_refine_varlen(Q, W, K, Kbar, cend, L, q_len, nc, g, nsel, block, k, chunks=True, cand=True,
                                  guard=guard)
    torch.cuda.synchronize()
    qo = np.concatenate([[0], np.cumsum(q_len)])
    G = [-(-q // g) for q in q_len]
    go = np.concatenate([[0], np.cumsum(G)])
    for r, (Qr, Wr, Kr) in enumerate(reqs):
        ref = run(Qr[None], Wr[None], Kr[None], block, g, nsel, k, guard)
        got = (out[0][qo[r]:qo[r + 1]], out[1][qo[r]:qo[r + 1]], out[2][go[r]:go[r + 1]], out[3][go[r]:go[r + 1]])
        for name, a, b in zip(("idx", "score", "chunks", "cand"), got, ref):
            assert torch.equal(a, b[0]), f"request {r}: {name}"
