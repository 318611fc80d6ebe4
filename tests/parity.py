"""GPU-vs-oracle parity drivers shared by the GPU test files and the smoke check.

Every function runs the HIP library through the C ABI (via the Python binding),
copies the very input tensors it used to the host, recomputes the selected rows
with the fp64 oracle and applies the parity rule of ``checker``.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_attention_indexer_dense_amd as dsa
import synth
from checker import Result, check_row


def host(Q, W, K):
    return synth.to_u16(Q), W.detach().cpu().numpy(), synth.to_u16(K)


def _rows_all(B, q_len):
    return [(b, r) for b in range(B) for r in range(q_len)]


def check_dense(Q, W, K, k, rows=None, out=None):
    """Dense indexer: GPU rows vs oracle. rows: list of (b, r); default all."""
    idx, sc = dsa.dense(Q, W, K, k)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    Qh, Wh, Kh = host(Q, W, K)
    B, q_len = Qh.shape[:2]
    L = Kh.shape[1]
    res = Result() if out is None else out
    for b, r in (rows or _rows_all(B, q_len)):
        pos = L - q_len + r
        ref, mass = oracle.scores(Qh[b, r], Wh[b, r], Kh[b], n=pos + 1)
        check_row(idx[b, r], sc[b, r], np.arange(pos + 1), ref, mass, k, res, f"dense b{b} r{r}")
    return res, idx, sc


def groups_all(B, G):
    return [(b, m) for b in range(B) for m in range(G)]


def check_pivot(Q, W, K, g, c, k, variant, groups=None, with_cand=True):
    """PIVOT Reuse or Refine: candidates vs the oracle's proxy scan, Reuse rows
    vs the proxy top-k (identical within a group), Refine rows vs the oracle
    re-scoring the GPU's own candidates (checked first)."""
    if variant == "reuse":
        idx, sc, cand = dsa.pivot_reuse(Q, W, K, g, k, c=c, cand=with_cand)
    else:
        idx, sc, cand = dsa.pivot_refine(Q, W, K, g, c, k, cand=True)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    cand = cand.cpu().numpy() if cand is not None else None
    Qh, Wh, Kh = host(Q, W, K)
    B, q_len = Qh.shape[:2]
    L = Kh.shape[1]
    G = (q_len + g - 1) // g
    res_c, res_r = Result(), Result()
    for b, m in (groups or groups_all(B, G)):
        r0, r1 = m * g, min(m * g + g, q_len)
        t_last = L - q_len + r1 - 1
        qb, wb = oracle.proxy(Qh[b], Wh[b], g, m)
        ref, mass = oracle.scores(qb, wb, Kh[b], n=t_last + 1)
        univ = np.arange(t_last + 1)
        if cand is not None:
            check_row(cand[b, m], None, univ, ref, mass, c, res_c, f"cand b{b} m{m}")
        for r in range(r0, r1):
            if variant == "reuse":
                check_row(idx[b, r], sc[b, r], univ, ref, mass, k, res_r, f"reuse b{b} r{r}")
                if not (np.array_equal(idx[b, r], idx[b, r0]) and np.array_equal(sc[b, r], sc[b, r0])):
                    res_r.add(False, False, 0.0, f"reuse b{b} r{r}: differs from the group's first row")
            else:
                pos = L - q_len + r
                cm = cand[b, m]
                cp = cm[(cm >= 0) & (cm <= pos)]
                ref_i, mass_i = oracle.scores(Qh[b, r], Wh[b, r], np.ascontiguousarray(Kh[b][cp]))
                check_row(idx[b, r], sc[b, r], cp, ref_i, mass_i, k, res_r, f"refine b{b} r{r}")
    return res_c, res_r, idx, sc, cand


def assert_ok(*results):
    for r in results:
        assert not r.failures, r.summary() + "\n" + "\n".join(r.failures[:10])
