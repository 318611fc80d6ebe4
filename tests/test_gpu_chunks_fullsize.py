"""The key-chunk path at the benchmark's size and launch configuration
(L = 131072, H_I = 64, d_I = 128, k = 2048, 64-key blocks, 64 chunks kept,
g = 1 and g = 4, fixed and adaptive partitions, keys with local structure),
checked by the oracle on sampled groups: the first ones (no or few complete
chunks), the last ones and seeded-random ones. Partitions and summaries are
compared whole."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_dense_amd as dsa
import synth
from checker import Result, check_row
from parity import assert_ok

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
L, H, D, K_SEL, BLOCK, NSEL = 131072, 64, 128, 2048, 64, 64


@pytest.fixture(scope="module")
def inputs():
    w = synth.WORKLOADS["pivot128k"]
    Q, W, _ = synth.make(w, device=DEV)
    K = synth.keys_local(w.L, w.d, w.rank, w.seed, DEV)[None]
    yield Q, W, K
    del Q, W, K
    torch.cuda.empty_cache()


def rows_of(t, idx):
    return t[0, torch.tensor(idx, device=t.device)].cpu().numpy()


@pytest.mark.parametrize("partition", ["fixed", "adaptive"])
@pytest.mark.parametrize("g", [1, 4])
def test_chunk_refine_fullsize(inputs, partition, g):
    Q, W, K = inputs
    if partition == "adaptive":
        cend = dsa.chunks_adaptive(K, BLOCK)
        mc = 2 * BLOCK
    else:
        cend = dsa.chunks_fixed(1, L, BLOCK, DEV)
        mc = BLOCK
    Kbar = dsa.chunk_means(K, cend)
    idx, sc, ch, cand = dsa.chunk_refine(Q, W, K, Kbar, cend, g, NSEL, mc, K_SEL, chunks=True, cand=True)
    torch.cuda.synchronize()
    K_h = synth.to_u16(K[0])
    ce = cend[0].cpu().numpy()
    want_ce = oracle.adaptive_chunks(K_h, BLOCK) if partition == "adaptive" else oracle.fixed_chunks(L, BLOCK)
    assert np.array_equal(ce, want_ce)
    kbar_h = synth.to_u16(Kbar[0])
    assert np.array_equal(kbar_h, oracle.chunk_means(K_h, ce))

    G = L // g
    rng = np.random.default_rng(7 + g)
    groups = sorted(set(range(3)) | {G - 1, G - 2} | set(rng.integers(0, G, 64).tolist()))
    chs, cands = rows_of(ch, groups), rows_of(cand, groups)
    members = [m * g + i for m in groups for i in range(g)]
    ids, scs = rows_of(idx, members), rows_of(sc, members)
    starts = np.concatenate([[0], ce[:-1]])
    cw = (NSEL + 1) * mc
    rs, rc, rr = Result(), Result(), Result()
    for gi, m in enumerate(groups):
        r0 = m * g
        t_last = r0 + g - 1
        ncomp = int(np.sum(ce <= t_last + 1))
        Qm, Wm = synth.to_u16(Q[0, r0:r0 + g]), W[0, r0:r0 + g].cpu().numpy()
        qb, wb = oracle.proxy(Qm, Wm, g, 0)
        if ncomp:
            ref, mass = oracle.scores(qb, wb, kbar_h, n=ncomp)
            check_row(chs[gi], None, np.arange(ncomp), ref, mass, NSEL, rs, f"chunks m{m}")
        sel = chs[gi][chs[gi] >= 0]
        want = [s for c in sel for s in range(starts[c], ce[c])]
        want += list(range(int(ce[ncomp - 1]) if ncomp else 0, t_last + 1))
        want = np.array(want + [-1] * (cw - len(want)), np.int64)
        rc.add(bool(np.array_equal(cands[gi], want)), True, 0.0, f"cand m{m}")
        for i in range(g):
            pos = r0 + i
            cp = cands[gi][(cands[gi] >= 0) & (cands[gi] <= pos)]
            ref_i, mass_i = oracle.scores(Qm[i], Wm[i], np.ascontiguousarray(K_h[cp]))
            j = gi * g + i
            check_row(ids[j], scs[j], cp, ref_i, mass_i, K_SEL, rr, f"refine r{pos}")
    assert_ok(rs, rc, rr)
    assert rr.rows == len(members)
    del idx, sc, ch, cand


def test_adaptive_partition_1m():
    # the adaptive partition at L = 1048576 (16384 blocks of 64 keys, sorted
    # in the workspace rather than in LDS) and its summaries, bit for bit;
    # then the chunk path for the last 64 query rows (4 groups of 16)
    w = synth.WORKLOADS["pivot1m"]
    L1 = w.L
    K = synth.keys_local(L1, w.d, w.rank, w.seed, DEV)[None]
    cend = dsa.chunks_adaptive(K, BLOCK)
    Kbar = dsa.chunk_means(K, cend)
    torch.cuda.synchronize()
    K_h = synth.to_u16(K[0])
    ce = cend[0].cpu().numpy()
    want = oracle.adaptive_chunks(K_h, BLOCK)
    assert ce.size == L1 // BLOCK
    assert np.array_equal(ce, want), np.nonzero(ce != want)[0][:5]
    assert int(np.sum(np.diff(np.concatenate([[0], ce])) != BLOCK)) > 0
    kbar_h = synth.to_u16(Kbar[0])
    assert np.array_equal(kbar_h, oracle.chunk_means(K_h, ce))

    g, q_len = 16, 64
    Q = synth.queries(q_len, H, D, w.rho, w.seed, DEV)[None]
    W = synth.weights(q_len, H, w.seed, DEV)[None]
    mc = 2 * BLOCK
    idx, sc, ch, cand = dsa.chunk_refine(Q, W, K, Kbar, cend, g, NSEL, mc, K_SEL, chunks=True, cand=True)
    torch.cuda.synchronize()
    idx, sc, ch, cand = [x[0].cpu().numpy() for x in (idx, sc, ch, cand)]
    starts = np.concatenate([[0], ce[:-1]])
    cw = (NSEL + 1) * mc
    rs, rc, rr = Result(), Result(), Result()
    off = L1 - q_len
    for m in range(q_len // g):
        r0 = m * g
        t_last = off + r0 + g - 1
        ncomp = int(np.sum(ce <= t_last + 1))
        Qm, Wm = synth.to_u16(Q[0, r0:r0 + g]), W[0, r0:r0 + g].cpu().numpy()
        qb, wb = oracle.proxy(Qm, Wm, g, 0)
        ref, mass = oracle.scores(qb, wb, kbar_h, n=ncomp)
        check_row(ch[m], None, np.arange(ncomp), ref, mass, NSEL, rs, f"chunks m{m}")
        sel = ch[m][ch[m] >= 0]
        keys = [s for c in sel for s in range(starts[c], ce[c])]
        keys += list(range(int(ce[ncomp - 1]), t_last + 1))
        keys = np.array(keys + [-1] * (cw - len(keys)), np.int64)
        rc.add(bool(np.array_equal(cand[m], keys)), True, 0.0, f"cand m{m}")
        for i in range(g):
            pos = off + r0 + i
            cp = cand[m][(cand[m] >= 0) & (cand[m] <= pos)]
            ref_i, mass_i = oracle.scores(Qm[i], Wm[i], np.ascontiguousarray(K_h[cp]))
            check_row(idx[r0 + i], sc[r0 + i], cp, ref_i, mass_i, K_SEL, rr, f"refine r{pos}")
    assert_ok(rs, rc, rr)
    assert rr.rows == q_len
    del K, Kbar, cend
    torch.cuda.empty_cache()

