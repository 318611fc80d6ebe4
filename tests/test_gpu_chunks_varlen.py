"""The key-chunk path over variable-length batches (the *_varlen entry
points): every request's chunk ends, summaries, selected chunks, candidate
lists and Refine rows equal, bit for bit, those of the uniform calls on that
request alone (whose parity with the oracle the key-chunk tests check), and
sampled groups of the packed outputs are checked against the oracle too.
Batches mix a prefill request (scan kernels), short query runs over long
caches (split-key kernels), a request shorter than one chunk (its rows wider
than it needs), a request without queries (offsets only), both partitions,
g = 1 and g > 1, and both head shapes."""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_dense_amd as dsa
import synth
from parity import assert_ok
from test_gpu_chunks import check_chunk_refine, uneven_keys

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def requests(L, q_len, H, d, block, seed, uneven=False):
    """Per request: Q [q, H, d], W [q, H] (the last q positions of a prefill
    sequence of L keys), K [L, d]."""
    out = []
    for r, (Lr, qr) in enumerate(zip(L, q_len)):
        Q, W, K = synth.prefill(Lr, H, d, 0.9, 2, seed + 17 * r, DEV)
        if uneven:
            K = uneven_keys(1, Lr, d, block, seed + 31 * r)
        out.append((Q[0, Lr - qr:].contiguous(), W[0, Lr - qr:].contiguous(), K[0].contiguous()))
    return out


def offsets(xs):
    return np.concatenate([[0], np.cumsum(xs)]).astype(np.int64)


# (L, q_len, H, d, block, adaptive, g, nsel, k)
CASES = [
    ([2048, 1000, 5000, 40, 700], [2048, 3, 5000, 40, 0], 4, 32, 64, False, 1, 6, 64),
    ([2048, 1000, 5000, 40, 700], [2048, 3, 5000, 40, 0], 4, 32, 64, False, 4, 6, 64),
    ([3000, 129, 2500, 600], [3000, 2, 17, 600], 4, 32, 32, True, 2, 8, 64),
    ([4096, 300, 2000], [4096, 2, 0], 64, 128, 64, False, 4, 16, 256),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_chunk_path_varlen_equals_per_request(case):
    L, q_len, H, d, block, adaptive, g, nsel, k = case
    reqs = requests(L, q_len, H, d, block, seed=500 + sum(L), uneven=adaptive)
    Q = torch.cat([q for q, _, _ in reqs])
    W = torch.cat([w for _, w, _ in reqs])
    K = torch.cat([kk for _, _, kk in reqs])
    if adaptive:
        cend, nc = dsa.chunks_adaptive_varlen(K, L, block)
    else:
        cend, nc = dsa.chunks_fixed_varlen(L, block, DEV)
    Kbar = dsa.chunk_means_varlen(K, L, cend, nc)
    max_chunk = 2 * block if adaptive else block
    out = dsa.chunk_refine_varlen(Q, W, K, Kbar, cend, L, q_len, nc, g, nsel, max_chunk, k, chunks=True,
                                  cand=True)
    torch.cuda.synchronize()
    co, qo = offsets(nc), offsets(q_len)
    G = [-(-q // g) for q in q_len]
    go = offsets(G)
    checked = 0
    for r, (Qr, Wr, Kr) in enumerate(reqs):
        ce_r = dsa.chunks_adaptive(Kr[None], block) if adaptive else dsa.chunks_fixed(1, L[r], block, DEV)
        assert torch.equal(cend[co[r]:co[r + 1]], ce_r[0]), f"request {r}: chunk ends"
        kb_r = dsa.chunk_means(Kr[None], ce_r)
        assert torch.equal(Kbar[co[r]:co[r + 1]], kb_r[0]), f"request {r}: summaries"
        if q_len[r] == 0:
            continue
        ref = dsa.chunk_refine(Qr[None], Wr[None], Kr[None], kb_r, ce_r, g, nsel, max_chunk, k, chunks=True,
                               cand=True)
        got = (out[0][qo[r]:qo[r + 1]], out[1][qo[r]:qo[r + 1]], out[2][go[r]:go[r + 1]],
               out[3][go[r]:go[r + 1]])
        for name, a, b in zip(("idx", "score", "chunks", "cand"), got, ref):
            assert torch.equal(a, b[0]), f"request {r}: {name}"
        # the oracle on a few groups of this request, from the packed outputs
        groups = sorted({0, G[r] // 2, G[r] - 1})
        res = check_chunk_refine(Qr[None], Wr[None], Kr[None], Kbar[co[r]:co[r + 1]][None],
                                 cend[co[r]:co[r + 1]][None], g, nsel, max_chunk, k,
                                 tuple(x[None] for x in got), groups=[(0, m) for m in groups])
        assert_ok(*res)
        checked += 1
    assert checked >= 2
