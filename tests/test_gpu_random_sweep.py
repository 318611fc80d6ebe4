"""A seeded random sweep over the public entry points against the oracle:
dense, Reuse and Refine (uniform and variable-length batches, with and
without the guard), and the key-chunk path (fixed and adaptive partitions,
variable-length, guard), over random lengths (prefill-like and decode-like
query runs, requests without queries), group sizes, k and c (lists across the
on-chip Refine kernel's capacities), both head shapes and signed weights.
Sampled rows and groups of every case go through the parity rule of
``checker``. Every input is valid; a failure names its case."""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_dense_amd as dsa
import synth
from checker import Result
from parity import HostView, check_dense_rows, check_varlen, merge
from test_gpu_chunks import check_chunk_refine

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CASES_PER_TEST = 25


def run_case(i, rng, wide):
    big = rng.random() < 0.15
    H, d = (64, 128) if big else (4, 32)
    kind = rng.choice(["pivot", "pivot", "pivot", "chunk"])
    uniform = rng.random() < 0.4
    B = int(rng.integers(1, 4))
    decode_like = rng.random() < 0.4
    Lmax = (5000 if big else 12000) if wide else (2500 if big else 6000)
    if uniform:
        L1 = int(rng.integers(1, Lmax))
        if decode_like:
            q1 = int(rng.integers(1, min(L1, 12) + 1))
        else:
            q1 = L1 if rng.random() < 0.6 else int(rng.integers(1, L1 + 1))
        Ls, qs = [L1] * B, [q1] * B
    else:
        Ls, qs = [], []
        for b in range(B):
            L = int(rng.integers(1, Lmax))
            if rng.random() < 0.1:
                q = 0
            elif decode_like:
                q = int(rng.integers(1, min(L, 12) + 1))
            else:
                q = L if rng.random() < 0.5 else int(rng.integers(1, L + 1))
            Ls.append(L)
            qs.append(q)
        if sum(qs) == 0:
            qs[0] = 1
    g = int(rng.choice([1, 2, 3, 4, 5, 8]))
    k = int(rng.integers(1, 2100 if wide else 300))
    signed = rng.random() < 0.3
    seed = int(rng.integers(0, 1 << 30))
    reqs = []
    for r, (L, q) in enumerate(zip(Ls, qs)):
        Q, W, K = synth.prefill(L, H, d, 0.9, 2, seed + r, DEV)
        if signed:
            W = synth.signed_weights(L, H, seed + 7 * r, DEV)[None]
        reqs.append((Q[0, L - q:].contiguous(), W[0, L - q:].contiguous(), K[0].contiguous()))
    Qp = torch.cat([x[0] for x in reqs])
    Wp = torch.cat([x[1] for x in reqs])
    Kp = torch.cat([x[2] for x in reqs])
    if kind == "pivot":
        variant = str(rng.choice(["dense", "reuse", "refine"]))
        c = int(rng.integers(k, max(k + 1, 5000 if wide else 1500)))
        guard = int(rng.choice([0, 0, 0, int(rng.integers(1, 5000))]))
        desc = (f"case {i}: pivot {variant} uniform={uniform} B={B} L={Ls} q={qs} H={H} d={d} g={g} c={c} k={k} "
                f"guard={guard} signed={signed} seed={seed}")
        if uniform and (variant == "dense" or guard == 0):
            Q4, W4, K4 = Qp.view(B, qs[0], H, d), Wp.view(B, qs[0], H), Kp.view(B, Ls[0], d)
            if variant == "dense":
                idx, sc = dsa.dense(Q4, W4, K4, k)
                out = (idx.view(-1, k), sc.view(-1, k), None)
            elif variant == "reuse":
                idx, sc, cand = dsa.pivot_reuse(Q4, W4, K4, g, k, c=c, cand=True)
                out = (idx.view(-1, k), sc.view(-1, k), cand.view(-1, c))
            else:
                idx, sc, cand = dsa.pivot_refine(Q4, W4, K4, g, c, k, cand=True)
                out = (idx.view(-1, k), sc.view(-1, k), cand.view(-1, c))
        elif variant == "dense":
            out = (*dsa.dense_varlen(Qp, Wp, Kp, Ls, qs, k), None)
        elif variant == "reuse":
            out = dsa.pivot_reuse_varlen(Qp, Wp, Kp, Ls, qs, g, k, c=c, guard=guard, cand=True)
        else:
            out = dsa.pivot_refine_varlen(Qp, Wp, Kp, Ls, qs, g, c, k, guard=guard, cand=True)
        torch.cuda.synchronize()
        if variant == "dense":
            idx, sc = out[0].cpu().numpy(), out[1].cpu().numpy()
            res = Result()
            qo = np.concatenate([[0], np.cumsum(qs)])
            for r, (Qr, Wr, Kr) in enumerate(reqs):
                if qs[r] == 0:
                    continue
                rows = sorted(set(rng.choice(qs[r], size=min(qs[r], 24), replace=False).tolist()) | {0, qs[r] - 1})
                hv = HostView(Qr[None], Wr[None], Kr[None])
                check_dense_rows(idx[qo[r]:qo[r + 1]][None], sc[qo[r]:qo[r + 1]][None], hv, Ls[r], qs[r], k,
                                 [(0, x) for x in rows], res)
            results = (res,)
        else:
            results = check_varlen(variant, Qp, Wp, Kp, Ls, qs, g, c, k, guard, out, max_groups=4, seed=i)
    else:
        block = int(rng.choice([16, 32, 64]))
        adaptive = rng.random() < 0.4
        nsel = int(rng.integers(1, 24))
        max_chunk = 2 * block if adaptive else block
        if (nsel + 1) * max_chunk < k:
            nsel = -(-k // max_chunk)
        guard = int(rng.choice([0, 0, int(rng.integers(1, 5000))]))
        desc = (f"case {i}: chunk adaptive={adaptive} B={B} L={Ls} q={qs} H={H} d={d} g={g} block={block} "
                f"nsel={nsel} k={k} guard={guard} signed={signed} seed={seed}")
        if adaptive:
            cend, nc = dsa.chunks_adaptive_varlen(Kp, Ls, block)
        else:
            cend, nc = dsa.chunks_fixed_varlen(Ls, block, DEV)
        Kbar = dsa.chunk_means_varlen(Kp, Ls, cend, nc)
        out = dsa.chunk_refine_varlen(Qp, Wp, Kp, Kbar, cend, Ls, qs, nc, g, nsel, max_chunk, k, chunks=True,
                                      cand=True, guard=guard)
        torch.cuda.synchronize()
        co = np.concatenate([[0], np.cumsum(nc)])
        qo = np.concatenate([[0], np.cumsum(qs)])
        G = [-(-q // g) for q in qs]
        go = np.concatenate([[0], np.cumsum(G)])
        rs, rc, rr, rd = Result(), Result(), Result(), Result()
        for r, (Qr, Wr, Kr) in enumerate(reqs):
            if qs[r] == 0:
                continue
            L, q = Ls[r], qs[r]
            t_last = [L - q + min(m * g + g, q) - 1 for m in range(G[r])]
            m0 = sum(1 for t in t_last if t + 1 <= guard) if guard > 0 else 0
            spans = [(qo[r], qo[r + 1])] * 2 + [(go[r], go[r + 1])] * 2
            got = tuple(x[a:b_][None] for x, (a, b_) in zip(out, spans))
            # guarded rows: dense
            hv = HostView(Qr[None], Wr[None], Kr[None])
            rows = list(range(min(m0 * g, q)))
            if rows:
                rows = sorted(set(rng.choice(rows, size=min(len(rows), 12), replace=False).tolist()))
                check_dense_rows(got[0].cpu().numpy(), got[1].cpu().numpy(), hv, L, q, k,
                                 [(0, x) for x in rows], rd)
            groups = list(range(m0, G[r]))
            if len(groups) > 4:
                pick = set(rng.choice(groups, size=4, replace=False).tolist())
                groups = sorted(pick | {groups[0], groups[-1]})
            if groups:
                a, b_, c_ = check_chunk_refine(Qr[None], Wr[None], Kr[None], Kbar[co[r]:co[r + 1]][None],
                                               cend[co[r]:co[r + 1]][None], g, nsel, max_chunk, k, got,
                                               groups=[(0, m) for m in groups])
                merge(rs, a)
                merge(rc, b_)
                merge(rr, c_)
        results = (rd, rs, rc, rr)
    return desc, results


@pytest.mark.parametrize("block", range(6))
def test_random_sweep(block):
    rng = np.random.default_rng(1000 + block)
    wide = block % 2 == 1
    bad = []
    for i in range(CASES_PER_TEST):
        desc, results = run_case(block * CASES_PER_TEST + i, rng, wide)
        fails = [f for r in results for f in r.failures]
        if fails:
            bad.append(desc + "\n    " + "\n    ".join(fails[:5]))
    assert not bad, "\n".join(bad)
