"""CPU oracle for the DSA token indexer and PIVOT Reuse/Refine (fp64, one thread).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only users. The GPU library never imports or links this
package, and this package imports nothing from the library.

The arithmetic lives in ``oracle.c`` (plain C, compiled with gcc into
``liboracle.so`` next to it); this module only marshals numpy arrays through
ctypes. bf16 tensors travel as their raw ``uint16`` bit patterns so that the
oracle widens exactly the values the GPU reads.

Paper: "PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention"
(arXiv 2607.24593); see ``oracle.c`` for which section each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Plain build: no fast-math, no FMA contraction, so every double operation is
# the IEEE operation written in the source.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc. Returns the path of the shared library."""
    tmp = f"{out}.{os.getpid()}.tmp"  # parallel builders never share a file
    cmd = ["gcc", *CFLAGS, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    lib.orc_scores.argtypes = [P, P, P, i32, i32, i64, P, P]
    lib.orc_select.argtypes = [P, P, i64, i64, P, P]
    lib.orc_dense_rows.argtypes = [P, P, P, i64, i64, i32, i32, i64, P, i64, P, P]
    lib.orc_proxy.argtypes = [P, P, i64, i32, i32, i64, i64, P, P]
    lib.orc_pivot_groups.argtypes = [P, P, P, i64, i64, i32, i32, i64, i64, i64,
                                     P, i64, P, P, P, P, P, P, P]
    lib.orc_proxy_ex.argtypes = [P, P, i64, i32, i32, i64, i64, i32, i64, P, P]
    lib.orc_pivot_groups_ex.argtypes = [P, P, P, i64, i64, i32, i32, i64, i64, i64, i32, i64,
                                        P, i64, P, P, P, P, P, P, P]
    lib.orc_chunk_means.argtypes = [P, i64, i32, P, i64, P]
    lib.orc_chunk_adaptive.argtypes = [P, i64, i32, i64, P]
    lib.orc_chunk_groups.argtypes = [P, P, P, i64, i64, i32, i32, i64, i32, i64, P, i64, i64, i64, i64,
                                     P, i64, P, P, P, P, P]
    for f in (lib.orc_scores, lib.orc_select, lib.orc_dense_rows, lib.orc_proxy,
              lib.orc_pivot_groups, lib.orc_proxy_ex, lib.orc_pivot_groups_ex,
              lib.orc_chunk_means, lib.orc_chunk_adaptive, lib.orc_chunk_groups):
        f.restype = ctypes.c_int
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 arrays are passed as uint16 bit patterns")
    return a


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def scores(q, w, K, n=None, lib=None):
    """Index scores of one query row against keys 0..n-1.

    q: uint16 [H, d]; w: float32 [H]; K: uint16 [>=n, d].
    Returns (score, mass), float64 [n] each; mass bounds every partial sum.
    """
    lib = lib or load()
    q, K, w = _u16(q), _u16(K), _f32(w)
    H, d = q.shape
    n = K.shape[0] if n is None else int(n)
    sc = np.empty(n, np.float64)
    ms = np.empty(n, np.float64)
    _check(lib.orc_scores(_p(q), _p(w), _p(K), H, d, n, _p(sc), _p(ms)), "scores")
    return sc, ms


def select(score, k, idx=None, lib=None):
    """Top-k under (score desc, index asc). Returns (idx int64 [k], score [k])."""
    lib = lib or load()
    score = np.ascontiguousarray(score, dtype=np.float64)
    n = score.shape[0]
    ix = None if idx is None else np.ascontiguousarray(idx, dtype=np.int64)
    oi = np.empty(k, np.int64)
    os_ = np.empty(k, np.float64)
    _check(lib.orc_select(_p(score), _p(ix), n, k, _p(oi), _p(os_)), "select")
    return oi, os_


PROXY = {"mean": 0, "first": 1, "last": 2}


def proxy(Q, W, g, m, kind="mean", window=0, lib=None):
    """Proxy (bf16 bits [H, d], fp32 [H]) of query group m of Q [q_len, H, d]:
    the mean of the group (or of its last ``window`` members), or its first
    or last member (``kind``)."""
    lib = lib or load()
    Q, W = _u16(Q), _f32(W)
    q_len, H, d = Q.shape
    qb = np.empty((H, d), np.uint16)
    wb = np.empty(H, np.float32)
    _check(lib.orc_proxy_ex(_p(Q), _p(W), q_len, H, d, g, m, PROXY[kind], window, _p(qb), _p(wb)),
           "proxy")
    return qb, wb


def dense_rows(Q, W, K, k, rows, lib=None):
    """Dense top-k for query rows ``rows`` of one sequence.

    Q: uint16 [q_len, H, d] (the last q_len positions of the sequence);
    W: float32 [q_len, H]; K: uint16 [L, d]. Returns (idx [nrows, k], score).
    """
    lib = lib or load()
    Q, K, W = _u16(Q), _u16(K), _f32(W)
    q_len, H, d = Q.shape
    L = K.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    oi = np.empty((rows.size, k), np.int64)
    os_ = np.empty((rows.size, k), np.float64)
    _check(lib.orc_dense_rows(_p(Q), _p(W), _p(K), L, q_len, H, d, k, _p(rows),
                              rows.size, _p(oi), _p(os_)), "dense_rows")
    return oi, os_


def pivot_groups(Q, W, K, g, c, k, groups, cand_in=None, kind="mean", window=0, lib=None):
    """PIVOT proxy scan, candidates, Reuse and Refine for groups ``groups``.

    Returns a dict with cand/cand_score [ng, c], reuse/reuse_score [ng, k] and
    refine/refine_score [ng, g, k]. ``cand_in`` ([ng, c], -1 padded) replaces the
    candidate list Refine uses.
    """
    lib = lib or load()
    Q, K, W = _u16(Q), _u16(K), _f32(W)
    q_len, H, d = Q.shape
    L = K.shape[0]
    groups = np.ascontiguousarray(groups, dtype=np.int64)
    ng = groups.size
    ci = None if cand_in is None else np.ascontiguousarray(cand_in, dtype=np.int64)
    out = dict(
        cand=np.empty((ng, c), np.int64), cand_score=np.empty((ng, c), np.float64),
        reuse=np.empty((ng, k), np.int64), reuse_score=np.empty((ng, k), np.float64),
        refine=np.empty((ng, g, k), np.int64),
        refine_score=np.empty((ng, g, k), np.float64),
    )
    _check(lib.orc_pivot_groups_ex(
        _p(Q), _p(W), _p(K), L, q_len, H, d, g, c, k, PROXY[kind], window, _p(groups), ng, _p(ci),
        _p(out["cand"]), _p(out["cand_score"]), _p(out["reuse"]),
        _p(out["reuse_score"]), _p(out["refine"]), _p(out["refine_score"])),
        "pivot_groups")
    return out


# ------------------------------------------------- key chunks (coarse stage)
def fixed_chunks(L, block):
    """Chunk ends of fixed blocks of ``block`` keys (the last one short when
    ``block`` does not divide L): the fixed-block hierarchical baseline of the
    SCALE paper's abstract (HISA-64 at block = 64)."""
    return np.minimum(np.arange(1, -(-L // block) + 1, dtype=np.int64) * block, L).astype(np.int32)


def adaptive_chunks(K, block, lib=None):
    """Score-adaptive chunk ends (the reading of SCALE's split/merge rule that
    ``oracle.c`` states) for keys K [L, d]: ceil(L / block) chunks."""
    lib = lib or load()
    K = _u16(K)
    L, d = K.shape
    out = np.empty(-(-L // block), np.int32)
    _check(lib.orc_chunk_adaptive(_p(K), L, d, block, _p(out)), "chunk_adaptive")
    return out


def chunk_means(K, cend, lib=None):
    """Mean key (bf16 bits [nc, d]) of every chunk of K [L, d]."""
    lib = lib or load()
    K = _u16(K)
    L, d = K.shape
    cend = np.ascontiguousarray(cend, dtype=np.int32)
    out = np.empty((cend.size, d), np.uint16)
    _check(lib.orc_chunk_means(_p(K), L, d, _p(cend), cend.size, _p(out)), "chunk_means")
    return out


def chunk_groups(Q, W, K, g, cend, nsel, cw, k, groups, kind="mean", window=0, lib=None):
    """Coarse chunk scan, candidate expansion and token-level Refine for groups
    ``groups``. Returns a dict with chunks/chunk_score [ng, nsel] (selected
    chunks ascending), cand [ng, cw] (ascending keys, -1 padded) and
    refine/refine_score [ng, g, k]."""
    lib = lib or load()
    Q, K, W = _u16(Q), _u16(K), _f32(W)
    q_len, H, d = Q.shape
    L = K.shape[0]
    cend = np.ascontiguousarray(cend, dtype=np.int32)
    groups = np.ascontiguousarray(groups, dtype=np.int64)
    ng = groups.size
    out = dict(
        chunks=np.empty((ng, nsel), np.int64), chunk_score=np.empty((ng, nsel), np.float64),
        cand=np.empty((ng, cw), np.int64),
        refine=np.empty((ng, g, k), np.int64), refine_score=np.empty((ng, g, k), np.float64),
    )
    _check(lib.orc_chunk_groups(
        _p(Q), _p(W), _p(K), L, q_len, H, d, g, PROXY[kind], window, _p(cend), cend.size, nsel, cw, k,
        _p(groups), ng, _p(out["chunks"]), _p(out["chunk_score"]), _p(out["cand"]),
        _p(out["refine"]), _p(out["refine_score"])), "chunk_groups")
    return out


# ------------------------------------------------- batches of requests
def request_offsets(L, q_len, g=1):
    """Per request of a packed batch: (first key row, first query row, first
    group), requests in order and without padding; a group never spans two
    requests (PIVOT paper, Method: the last group of a request may be
    smaller)."""
    key_off, q_off, g_off = [], [], []
    kk = qq = gg = 0
    for Lb, qb in zip(L, q_len):
        key_off.append(kk)
        q_off.append(qq)
        g_off.append(gg)
        kk += int(Lb)
        qq += int(qb)
        gg += -(-int(qb) // g)
    return key_off, q_off, g_off


def guarded_groups(L, q_len, g, guard):
    """Leading groups of one request that the guard scores densely.

    PIVOT paper, Results (the guardrail: PIVOT falls back to a dense scan for
    short groups). Reading taken: group m, whose last position is
    t_last = L - q_len + min((m + 1) g, q_len) - 1, is guarded when its whole
    causal prefix, t_last + 1 keys, is at most ``guard``; guard = 0 guards
    nothing. t_last grows with m, so the guarded groups are a prefix.
    """
    off = L - q_len
    n = 0
    for m in range(-(-q_len // g)):
        if off + min((m + 1) * g, q_len) <= guard:
            n += 1
        else:
            break
    return n
