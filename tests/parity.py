"""GPU-vs-oracle parity drivers shared by the GPU test files and the smoke check.

Every function runs the HIP library through the C ABI (via the Python binding),
copies to the host the very input rows it needs, recomputes the selected rows
with the fp64 oracle and applies the parity rule of ``checker``.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import oracle_pool
import sparse_attention_indexer_dense_amd as dsa
import synth
from checker import Result, check_row


def _rows_all(B, q_len):
    return [(b, r) for b in range(B) for r in range(q_len)]


def groups_all(B, G):
    return [(b, m) for b in range(B) for m in range(G)]


class HostView:
    """Host copies of K per batch item (on demand) and of individual Q/W rows."""

    def __init__(self, Q, W, K):
        self.Q, self.W, self.K = Q, W, K
        self._k = {}

    def keys(self, b):
        if b not in self._k:
            self._k[b] = synth.to_u16(self.K[b])
        return self._k[b]

    def rows(self, b, r0, r1):
        return synth.to_u16(self.Q[b, r0:r1]), self.W[b, r0:r1].detach().cpu().numpy()


def check_dense_rows(idx, sc, hv, L, q_len, k, rows, res=None, pool=None):
    """Check GPU dense output rows (host arrays idx/sc [B, q_len, k]) for `rows`
    (in the worker processes of an oracle_pool.OraclePool when one is given)."""
    res = Result() if res is None else res
    if pool is not None:
        jobs = []
        for b, r in rows:
            q, w = hv.rows(b, r, r + 1)
            jobs.append((b, r, q[0], w[0], L - q_len + r + 1, np.asarray(idx[b, r]), np.asarray(sc[b, r]), k))
        for part in pool.map(oracle_pool._dense_job, jobs):
            merge(res, part)
        return res
    for b, r in rows:
        pos = L - q_len + r
        q, w = hv.rows(b, r, r + 1)
        ref, mass = oracle.scores(q[0], w[0], hv.keys(b), n=pos + 1)
        check_row(idx[b, r], sc[b, r], np.arange(pos + 1), ref, mass, k, res, f"dense b{b} r{r}")
    return res


def check_dense(Q, W, K, k, rows=None, out=None):
    """Dense indexer: GPU rows vs oracle. rows: list of (b, r); default all."""
    idx, sc = dsa.dense(Q, W, K, k)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    B, q_len = Q.shape[:2]
    L = K.shape[1]
    hv = HostView(Q, W, K)
    res = check_dense_rows(idx, sc, hv, L, q_len, k, rows or _rows_all(B, q_len), out)
    return res, idx, sc


def check_pivot_rows(variant, idx, sc, cand, hv, L, q_len, g, c, k, groups, kind="mean", window=0,
                     pool=None):
    """Check PIVOT outputs (host arrays) for `groups` [(b, m)]: candidates vs the
    oracle's proxy scan, Reuse rows vs the proxy top-k (identical within a
    group), Refine rows vs the oracle re-scoring the GPU's own candidates. With
    an oracle_pool.OraclePool the proxy scans run in its worker processes."""
    res_c, res_r = Result(), Result()
    scan = cand is not None or variant == "reuse"
    if pool is not None and scan:
        jobs = []
        for b, m in groups:
            r0, r1 = m * g, min(m * g + g, q_len)
            Qm, Wm = hv.rows(b, r0, r1)
            qb, wb = oracle.proxy(Qm, Wm, g, 0, kind=kind, window=window)
            reuse = ([(r, np.asarray(idx[b, r]), np.asarray(sc[b, r])) for r in range(r0, r1)]
                     if variant == "reuse" else [])
            jobs.append((b, m, qb, wb, L - q_len + r1, None if cand is None else np.asarray(cand[b, m]), c,
                         reuse, k))
        for rc_, rr_ in pool.map(oracle_pool._proxy_job, jobs):
            merge(res_c, rc_)
            merge(res_r, rr_)
        scan = False  # done
    refine_jobs = []
    for b, m in groups:
        r0, r1 = m * g, min(m * g + g, q_len)
        t_last = L - q_len + r1 - 1
        Qm, Wm = hv.rows(b, r0, r1)
        univ = None
        if scan:
            qb, wb = oracle.proxy(Qm, Wm, g, 0, kind=kind, window=window)
            ref, mass = oracle.scores(qb, wb, hv.keys(b), n=t_last + 1)
            univ = np.arange(t_last + 1)
            if cand is not None:
                check_row(cand[b, m], None, univ, ref, mass, c, res_c, f"cand b{b} m{m}")
        for r in range(r0, r1):
            if variant == "reuse":
                if scan:
                    check_row(idx[b, r], sc[b, r], univ, ref, mass, k, res_r, f"reuse b{b} r{r}")
                if not (np.array_equal(idx[b, r], idx[b, r0]) and np.array_equal(sc[b, r], sc[b, r0])):
                    res_r.add(False, False, 0.0, f"reuse b{b} r{r}: differs from the group's first row")
            else:
                pos = L - q_len + r
                cm = cand[b, m]
                cp = cm[(cm >= 0) & (cm <= pos)]
                if pool is not None:
                    refine_jobs.append((b, r, Qm[r - r0], Wm[r - r0], np.ascontiguousarray(cp),
                                        np.asarray(idx[b, r]), np.asarray(sc[b, r]), k))
                    continue
                kc = np.ascontiguousarray(hv.keys(b)[cp])
                ref_i, mass_i = oracle.scores(Qm[r - r0], Wm[r - r0], kc)
                check_row(idx[b, r], sc[b, r], cp, ref_i, mass_i, k, res_r, f"refine b{b} r{r}")
    for part in (pool.map(oracle_pool._refine_job, refine_jobs) if refine_jobs else []):
        merge(res_r, part)
    return res_c, res_r


def check_pivot(Q, W, K, g, c, k, variant, groups=None, with_cand=True):
    if variant == "reuse":
        idx, sc, cand = dsa.pivot_reuse(Q, W, K, g, k, c=c, cand=with_cand)
    else:
        idx, sc, cand = dsa.pivot_refine(Q, W, K, g, c, k, cand=True)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    cand = cand.cpu().numpy() if cand is not None else None
    B, q_len = Q.shape[:2]
    L = K.shape[1]
    G = (q_len + g - 1) // g
    hv = HostView(Q, W, K)
    res_c, res_r = check_pivot_rows(variant, idx, sc, cand, hv, L, q_len, g, c, k,
                                    groups or groups_all(B, G))
    return res_c, res_r, idx, sc, cand


def assert_ok(*results):
    for r in results:
        assert not r.failures, r.summary() + "\n" + "\n".join(r.failures[:10])


def merge(dst, src):
    dst.rows += src.rows
    dst.exact += src.exact
    dst.band += src.band
    dst.max_rel = max(dst.max_rel, src.max_rel)
    dst.failures += src.failures
    return dst


def check_varlen(variant, Q, W, K, L, q_len, g, c, k, guard, out, max_groups=None, seed=0,
                 kind="mean", window=0):
    """Check the outputs of a packed batch of requests (variant dense, reuse or
    refine). out = (idx [sum q_len, k], score, cand [sum G, c] or None) on the
    GPU. Rows of guarded groups must hold their dense selection and their
    candidate rows -1; the other groups are checked as PIVOT groups. With
    max_groups, that many seeded-random groups per request (plus the first
    and last unguarded ones) are checked. Returns (dense rows, cand, PIVOT
    rows) results."""
    idx, sc, cand = out
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    cand = cand.cpu().numpy() if cand is not None else None
    key_off, q_off, g_off = oracle.request_offsets(L, q_len, g)
    rng = np.random.default_rng(seed)
    res_d, res_c, res_r = Result(), Result(), Result()
    for b, (Lb, qb) in enumerate(zip(L, q_len)):
        hv = HostView(Q[q_off[b]:q_off[b] + qb][None], W[q_off[b]:q_off[b] + qb][None],
                      K[key_off[b]:key_off[b] + Lb][None])
        ib = idx[q_off[b]:q_off[b] + qb][None]
        sb = sc[q_off[b]:q_off[b] + qb][None]
        if variant == "dense":
            check_dense_rows(ib, sb, hv, Lb, qb, k, [(0, r) for r in range(qb)], res_d)
            continue
        G = -(-qb // g)
        m0 = oracle.guarded_groups(Lb, qb, g, guard)
        check_dense_rows(ib, sb, hv, Lb, qb, k, [(0, r) for r in range(min(m0 * g, qb))], res_d)
        cb = None if cand is None else cand[g_off[b]:g_off[b] + G][None]
        if cb is not None:
            for m in range(m0):
                ok = bool((cb[0, m] == -1).all())
                res_c.add(ok, ok, 0.0, None if ok else f"cand b{b} m{m}: guarded group not -1")
        groups = list(range(m0, G))
        if max_groups is not None and len(groups) > max_groups:
            pick = set(rng.choice(groups, max_groups, replace=False).tolist()) | {groups[0], groups[-1]}
            groups = sorted(pick)
        rc, rr = check_pivot_rows(variant, ib, sb, cb, hv, Lb, qb, g, c, k, [(0, m) for m in groups],
                                  kind=kind, window=window)
        merge(res_c, rc)
        merge(res_r, rr)
    return res_d, res_c, res_r
