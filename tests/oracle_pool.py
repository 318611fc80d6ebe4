"""Oracle checks of many full-length rows in worker processes.

The fp64 oracle needs about a second per full 128K-key row, so the full-size
parity tests hand their oracle work to a pool of spawned worker processes.
The workers import only numpy, the oracle and the checker (no torch, no GPU
library): they never touch the GPU. K travels once, through shared memory;
each job carries its query row, its GPU output row and its bounds, and returns
the checker's small Result, not the score row.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import shared_memory

import numpy as np

import oracle
from checker import Result, check_row

_K = None  # worker: the shared keys [B][L][d] (uint16)
_SHM = None


def _attach(name, shape):
    global _K, _SHM
    _SHM = shared_memory.SharedMemory(name=name)
    _K = np.ndarray(shape, dtype=np.uint16, buffer=_SHM.buf)
    oracle.load()


def _dense_job(job):
    """A dense row: the oracle's scores of keys 0..n-1 against the GPU row."""
    b, r, q, w, n, idx_row, sc_row, k = job
    res = Result()
    ref, mass = oracle.scores(q, w, _K[b], n=n)
    check_row(idx_row, sc_row, np.arange(n), ref, mass, k, res, f"dense b{b} r{r}")
    return res


def _proxy_job(job):
    """A group's proxy scan: its candidate row (top-c) and, for Reuse, the
    member rows (top-k of the same scores), against one oracle score row."""
    b, m, qb, wb, n, cand_row, c, reuse_rows, k = job
    res_c, res_r = Result(), Result()
    ref, mass = oracle.scores(qb, wb, _K[b], n=n)
    univ = np.arange(n)
    if cand_row is not None:
        check_row(cand_row, None, univ, ref, mass, c, res_c, f"cand b{b} m{m}")
    for r, idx_row, sc_row in reuse_rows:
        check_row(idx_row, sc_row, univ, ref, mass, k, res_r, f"reuse b{b} r{r}")
    return res_c, res_r


def _refine_job(job):
    """A Refine member row: the oracle re-scores the GPU's own causal
    candidates cp with the member's query and weights."""
    b, r, q, w, cp, idx_row, sc_row, k = job
    res = Result()
    kc = np.ascontiguousarray(_K[b][cp])
    ref, mass = oracle.scores(q, w, kc)
    check_row(idx_row, sc_row, cp, ref, mass, k, res, f"refine b{b} r{r}")
    return res


class OraclePool:
    """Process pool for oracle checks over the keys K (a [B][L][d] uint16 host
    array), with at most `workers` processes."""

    def __init__(self, K, workers=16):
        K = np.ascontiguousarray(K, dtype=np.uint16)
        self.shm = shared_memory.SharedMemory(create=True, size=max(1, K.nbytes))
        np.ndarray(K.shape, dtype=np.uint16, buffer=self.shm.buf)[:] = K
        n = max(1, min(workers, os.cpu_count() or 1))
        self.ex = ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                                      initializer=_attach, initargs=(self.shm.name, K.shape))

    def map(self, fn, jobs):
        return list(self.ex.map(fn, jobs))

    def close(self):
        self.ex.shutdown()
        self.shm.close()
        self.shm.unlink()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
