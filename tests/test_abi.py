"""The C-ABI library loads, exports every function include/dsaidx.h declares,
and rejects invalid arguments before touching the GPU (no kernel runs here)."""
import ctypes
import os
import re

import pytest

import sparse_attention_indexer_dense_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsaidx.h")
OK, EINVAL, EUNSUPPORTED, EWORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(indexer_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return dsa.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(dsa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version(lib):
    assert dsa.indexer_version().startswith("dsaidx")


def ws(mode, B=1, L=4096, q_len=4096, H=64, d=128, g=4, c=512, k=256):
    return dsa.indexer_workspace_bytes(mode, B, L, q_len, H, d, g, c, k)


def test_workspace_sizes():
    assert ws(dsa.DENSE) > 0
    assert ws(dsa.REUSE) > 0 and ws(dsa.REFINE) > 0
    # row buffers grow with the selection size (up to one row's keys)
    assert ws(dsa.DENSE, L=131072, q_len=131072, k=2048) > ws(dsa.DENSE, L=131072, q_len=131072, k=256)
    assert ws(dsa.DENSE, k=2048) == ws(dsa.DENSE, k=4000)  # capped by L
    # decode shape: per-row score vectors
    assert ws(dsa.DENSE, B=32, L=65536, q_len=2, k=2048) >= 32 * 2 * 65536 * 4
    assert ws(dsa.DENSE, B=0) == 0
    assert ws(dsa.DENSE, H=8, d=64) == 0
    assert ws(dsa.REFINE, c=100, k=200) == 0
    for bad in (3, -1, 99):  # not a dsaidx_mode
        assert ws(bad) == 0
        assert "unknown mode" in dsa.indexer_last_error()


P = ctypes.c_void_p


def fake(addr=0x100000):
    return P(addr)


def call_dense(B=1, L=1024, q_len=1024, H=64, d=128, k=64, Q=None, W=None, K=None,
               out=None, ws_ptr=None, ws_bytes=1 << 40):
    Q = fake() if Q is None else Q
    W = fake() if W is None else W
    K = fake() if K is None else K
    out = fake() if out is None else out
    ws_ptr = fake() if ws_ptr is None else ws_ptr
    return dsa.indexer_dense(Q, W, K, B, L, q_len, H, d, k, out, None, ws_ptr, ws_bytes, None)


def test_dense_rejects_bad_sizes():
    assert call_dense(B=0) == EINVAL
    assert call_dense(q_len=2000) == EINVAL
    assert call_dense(q_len=-1) == EINVAL
    assert call_dense(L=-1, q_len=0) == EINVAL
    assert call_dense(k=0) == EINVAL
    assert call_dense(H=8, d=64) == EUNSUPPORTED
    assert "no kernel" in dsa.indexer_last_error()


def test_dense_rejects_bad_pointers():
    assert call_dense(Q=P(0)) == EINVAL
    assert call_dense(out=P(0)) == EINVAL
    assert call_dense(Q=fake(0x100008)) == EINVAL  # not 16-byte aligned
    assert "aligned" in dsa.indexer_last_error()
    assert call_dense(ws_bytes=16) == EWORKSPACE
    assert "workspace" in dsa.indexer_last_error()


def call_pivot(fn, g=4, c=512, k=256, cand=None, ws_bytes=1 << 40, L=1024):
    return fn(fake(), fake(), fake(), 1, L, L, 64, 128, g, c, k, fake(), None, cand,
              fake(), ws_bytes, None)


@pytest.mark.parametrize("fn", [dsa.indexer_pivot_reuse, dsa.indexer_pivot_refine])
def test_pivot_rejects_bad_arguments(fn):
    assert call_pivot(fn, g=0) == EINVAL
    assert call_pivot(fn, c=100, k=256, cand=fake()) == EINVAL  # c < k with candidates
    assert call_pivot(fn, ws_bytes=1) == EWORKSPACE


def test_refine_requires_c_ge_k():
    assert call_pivot(dsa.indexer_pivot_refine, c=100, k=256) == EINVAL
    assert "c=" in dsa.indexer_last_error()


def varlen_ws(mode, L, q, g=4, c=512, k=256, guard=0, H=64, d=128, proxy=0, window=0):
    arr = ctypes.c_int64 * len(L)
    opts = ctypes.byref(dsa.PivotOpts(guard, proxy, window))
    return dsa.indexer_varlen_workspace_bytes(mode, len(L), arr(*L), arr(*q), H, d, g, c, k, opts)


def test_varlen_workspace_sizes():
    assert varlen_ws(dsa.DENSE, [100, 5000], [100, 2]) > 0
    assert varlen_ws(dsa.REFINE, [100, 5000], [100, 2]) > 0
    assert varlen_ws(dsa.REUSE, [100, 5000], [100, 2], guard=50) > 0
    for bad in (3, -1):
        assert varlen_ws(bad, [100, 5000], [100, 2]) == 0
        assert "unknown mode" in dsa.indexer_last_error()
    # the guard removes the PIVOT stages when every group is guarded
    assert varlen_ws(dsa.REFINE, [4096], [4096], guard=4096) < varlen_ws(dsa.REFINE, [4096], [4096])
    assert varlen_ws(dsa.DENSE, [100, 50], [100, 60]) == 0   # q_len > L
    assert varlen_ws(dsa.DENSE, [0], [1]) == 0   # q_len > L
    assert varlen_ws(dsa.DENSE, [5], [-1]) == 0
    assert varlen_ws(dsa.REFINE, [100], [100], guard=-1) == 0
    assert varlen_ws(dsa.REFINE, [100], [100], proxy=3) == 0
    assert varlen_ws(dsa.REFINE, [100], [100], window=-2) == 0
    assert varlen_ws(dsa.REFINE, [100], [100], proxy=2, window=4) > 0


def test_varlen_rejects_bad_arguments():
    arr = ctypes.c_int64 * 2
    L, q = arr(1000, 50), arr(1000, 60)
    rc = dsa.indexer_dense_varlen(fake(), fake(), fake(), 2, L, q, 64, 128, 64, fake(), None, fake(),
                                  1 << 40, None)
    assert rc == EINVAL and "q_len" in dsa.indexer_last_error()
    rc = dsa.indexer_pivot_refine_varlen(fake(), fake(), fake(), 2, None, q, 64, 128, 4, 128, 64, None,
                                         fake(), None, None, fake(), 1 << 40, None)
    assert rc == EINVAL
    L, q = arr(1000, 50), arr(1000, 50)
    rc = dsa.indexer_pivot_reuse_varlen(fake(), fake(), fake(), 2, L, q, 64, 128, 0, 128, 64, None,
                                        fake(), None, None, fake(), 1 << 40, None)
    assert rc == EINVAL
    rc = dsa.indexer_pivot_refine_varlen(fake(), fake(), fake(), 2, L, q, 64, 128, 4, 32, 64, None,
                                         fake(), None, None, fake(), 1 << 40, None)
    assert rc == EINVAL  # c < k
    bad = ctypes.byref(dsa.PivotOpts(0, 7, 0))
    rc = dsa.indexer_pivot_refine_varlen(fake(), fake(), fake(), 2, L, q, 64, 128, 4, 128, 64, bad,
                                         fake(), None, None, fake(), 1 << 40, None)
    assert rc == EINVAL and "proxy" in dsa.indexer_last_error()


def test_empty_batches_do_nothing():
    # no query rows: parameters are still checked, nothing is touched, and the
    # pointers may be NULL
    N = None
    assert dsa.indexer_dense(N, N, N, 2, 1024, 0, 64, 128, 64, N, N, N, 0, None) == OK
    assert dsa.indexer_dense(N, N, N, 2, 0, 0, 64, 128, 64, N, N, N, 0, None) == OK
    assert dsa.indexer_dense(N, N, N, 2, 1024, 0, 64, 128, 0, N, N, N, 0, None) == EINVAL  # k = 0
    for fn in (dsa.indexer_pivot_reuse, dsa.indexer_pivot_refine):
        assert fn(N, N, N, 1, 1024, 0, 64, 128, 4, 512, 256, N, N, N, N, 0, None) == OK
        assert fn(N, N, N, 1, 1024, 0, 64, 128, 0, 512, 256, N, N, N, N, 0, None) == EINVAL  # g = 0
    assert dsa.indexer_pivot_refine(N, N, N, 1, 1024, 0, 64, 128, 4, 100, 256, N, N, N, N, 0,
                                    None) == EINVAL  # c < k
    arr = ctypes.c_int64 * 3
    L, q = arr(0, 500, 70), arr(0, 0, 0)
    assert dsa.indexer_dense_varlen(N, N, N, 3, L, q, 64, 128, 64, N, N, N, 0, None) == OK
    for fn in (dsa.indexer_pivot_reuse_varlen, dsa.indexer_pivot_refine_varlen):
        assert fn(N, N, N, 3, L, q, 64, 128, 4, 512, 256, None, N, N, N, N, 0, None) == OK
    assert varlen_ws(dsa.REFINE, [0, 500, 70], [0, 0, 0]) > 0
    # a batch with some queries still needs its pointers
    q = arr(0, 10, 0)
    assert dsa.indexer_dense_varlen(N, N, N, 3, L, q, 64, 128, 64, N, N, N, 0, None) == EINVAL
    # the key-chunk path keeps L, q_len >= 1
    assert chunk_ws(q_len=0) == 0


def chunk_ws(B=1, L=8192, q_len=8192, H=64, d=128, g=1, nc=128, nsel=16, max_chunk=64, k=256):
    return dsa.indexer_chunk_refine_workspace_bytes(B, L, q_len, H, d, g, nc, nsel, max_chunk, k, None)


def test_chunk_workspace_sizes():
    assert chunk_ws() > 0
    assert chunk_ws(g=4) > 0 and chunk_ws(q_len=2, g=2) > 0
    assert chunk_ws(nsel=3, max_chunk=32, k=256) == 0    # (nsel + 1) * max_chunk < k
    assert chunk_ws(nc=0) == 0 and chunk_ws(nc=8193) == 0
    assert chunk_ws(g=0) == 0 and chunk_ws(max_chunk=0) == 0
    assert chunk_ws(H=8, d=128) == 0
    assert dsa.indexer_chunks_adaptive_workspace_bytes(2, 8192, 64) >= 2 * 128 * 8
    assert dsa.indexer_chunks_adaptive_workspace_bytes(0, 8192, 64) == 0


def test_chunk_entry_points_reject_bad_arguments():
    assert dsa.indexer_chunks_fixed(0, 100, 8, fake(), None) == EINVAL
    assert dsa.indexer_chunks_fixed(1, 100, 0, fake(), None) == EINVAL
    assert dsa.indexer_chunks_fixed(1, 100, 8, None, None) == EINVAL
    big = 1 << 40
    # adaptive: odd block, too many blocks, unsupported d
    assert dsa.indexer_chunks_adaptive(fake(), 1, 1000, 128, 7, fake(), fake(), big, None) == EINVAL
    rc = dsa.indexer_chunks_adaptive(fake(), 1, (262144 + 1) * 64, 128, 64, fake(), fake(), big, None)
    assert rc == EUNSUPPORTED and "262144" in dsa.indexer_last_error()
    assert dsa.indexer_chunks_adaptive(fake(), 1, 1000, 64, 8, fake(), fake(), big, None) == EUNSUPPORTED
    assert dsa.indexer_chunks_adaptive(fake(), 1, 1000, 128, 8, fake(), fake(), 8, None) == EWORKSPACE
    # summaries
    assert dsa.indexer_chunk_means(fake(), 1, 100, 128, fake(), 0, 0, fake(), None) == EINVAL
    assert dsa.indexer_chunk_means(fake(), 1, 100, 128, fake(), 10, 11, fake(), None) == EINVAL
    assert dsa.indexer_chunk_means(fake(), 1, 100, 128, fake(), 10, 10, fake(), None) == OK  # nothing to do
    # refine
    def refine(opts=None, nc=128, nsel=16, max_chunk=64, k=256, Kbar=fake(), ws_bytes=big):
        return dsa.indexer_chunk_refine(fake(), fake(), fake(), Kbar, fake(), nc, 1, 8192, 8192, 64, 128, 1,
                                        nsel, max_chunk, k, opts, fake(), None, None, None, fake(), ws_bytes,
                                        None)
    assert refine(opts=ctypes.byref(dsa.PivotOpts(-1, 0, 0))) == EINVAL
    assert "guard" in dsa.indexer_last_error()
    assert refine(opts=ctypes.byref(dsa.PivotOpts(0, 5, 0))) == EINVAL
    assert refine(nsel=2, max_chunk=32) == EINVAL and ">= k" in dsa.indexer_last_error()
    assert refine(nc=9000) == EINVAL
    assert refine(Kbar=None) == EINVAL
    assert refine(ws_bytes=64) == EWORKSPACE


def test_sort_rows_rejects_bad_arguments():
    assert dsa.indexer_sort_rows(fake(), fake(), 10, 0, None) == EINVAL
    assert dsa.indexer_sort_rows(fake(), fake(), 10, 8193, None) == EINVAL
    assert dsa.indexer_sort_rows(None, fake(), 10, 64, None) == EINVAL
    assert dsa.indexer_sort_rows(fake(), None, 10, 64, None) == EINVAL
    assert dsa.indexer_sort_rows(fake(), fake(), -1, 64, None) == EINVAL
    assert dsa.indexer_sort_rows(fake(), fake(), 0, 64, None) == OK  # nothing to do


def arr(*xs):
    return (ctypes.c_int64 * len(xs))(*xs)


def test_chunk_varlen_entry_points_reject_bad_arguments():
    big = 1 << 40
    L, q, nc = arr(3000, 64, 500), arr(3000, 10, 0), arr(47, 1, 8)
    # sizes: every request is checked before anything is enqueued
    assert dsa.indexer_chunks_fixed_varlen(3, arr(3000, 0, 500), 64, fake(), None) == EINVAL
    assert "request 1" in dsa.indexer_last_error()
    assert dsa.indexer_chunks_fixed_varlen(3, L, 0, fake(), None) == EINVAL
    assert dsa.indexer_chunks_fixed_varlen(3, L, 64, None, None) == EINVAL
    assert dsa.indexer_chunks_fixed_varlen(0, L, 64, fake(), None) == EINVAL
    assert dsa.indexer_chunks_adaptive_varlen_workspace_bytes(3, L, 64) > 0
    assert dsa.indexer_chunks_adaptive_varlen(fake(), 3, L, 128, 7, fake(), fake(), big, None) == EINVAL
    assert dsa.indexer_chunks_adaptive_varlen(fake(), 3, L, 128, 64, fake(), fake(), 8, None) == EWORKSPACE
    assert dsa.indexer_chunk_means_varlen(fake(), 3, L, 128, fake(), None, fake(), None) == EINVAL
    assert dsa.indexer_chunk_means_varlen(fake(), 3, L, 128, fake(), arr(47, 65, 8), fake(), None) == EINVAL
    assert "request 1" in dsa.indexer_last_error()

    def ws(q_len=q, nc_=nc, nsel=8, max_chunk=64, k=128):
        return dsa.indexer_chunk_refine_varlen_workspace_bytes(3, L, q_len, 64, 128, 4, nc_, nsel, max_chunk, k,
                                                               None)
    assert ws() > 0
    assert ws(q_len=arr(0, 0, 0)) > 0                # nothing to run is still a valid call
    assert ws(q_len=arr(3000, 65, 0)) == 0           # q_len > L
    assert ws(nc_=arr(47, 1, 0)) == 0                # nc < 1
    assert ws(nsel=1, max_chunk=32, k=128) == 0      # (nsel + 1) * max_chunk < k
    assert ws(q_len=None) == 0 and ws(nc_=None) == 0
    # a request shorter than the largest chunk is valid (its rows are only wider)
    assert dsa.indexer_chunk_refine_varlen_workspace_bytes(2, arr(3000, 40), arr(8, 8), 64, 128, 4,
                                                         arr(47, 1), 8, 64, 128, None) > 0

    def refine(q_len=q, nc_=nc, Kbar=fake(), ws_bytes=big, opts=None):
        return dsa.indexer_chunk_refine_varlen(fake(), fake(), fake(), Kbar, fake(), nc_, 3, L, q_len, 64, 128,
                                               4, 8, 64, 128, opts, fake(), None, None, None, fake(), ws_bytes,
                                               None)
    assert refine(q_len=arr(3000, 65, 0)) == EINVAL and "request 1" in dsa.indexer_last_error()
    assert refine(nc_=None) == EINVAL
    assert refine(Kbar=None) == EINVAL
    assert refine(ws_bytes=64) == EWORKSPACE
    assert refine(opts=ctypes.byref(dsa.PivotOpts(-1, 0, 0))) == EINVAL and "guard" in dsa.indexer_last_error()
    assert refine(q_len=arr(0, 0, 0)) == OK          # no request has rows: nothing to do
