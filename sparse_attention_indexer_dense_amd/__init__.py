"""Python binding of the dsaidx C ABI (include/dsaidx.h): the DSA token indexer
and PIVOT Reuse/Refine on AMD MI355X (gfx950).

This module only marshals arguments: the functions named like the C entry
points (``indexer_dense``, ``indexer_pivot_reuse``, ``indexer_pivot_refine``,
their ``*_varlen`` forms for batches of requests of different lengths,
``indexer_workspace_bytes``, ``indexer_varlen_workspace_bytes``,
the key-chunk coarse stage ``indexer_chunks_fixed``, ``indexer_chunks_adaptive``,
``indexer_chunk_means``, ``indexer_chunk_refine`` with their workspace queries,
``indexer_sort_rows``,
``indexer_last_error``, ``indexer_version``) take raw device pointers and
sizes, exactly as the C functions do. ``dense``, ``pivot_reuse``,
``pivot_refine``, their ``*_varlen`` forms, ``chunks_fixed``,
``chunks_adaptive``, ``chunk_means`` and ``chunk_refine`` take torch tensors on the GPU,
allocate the outputs and the workspace with torch (device memory and the
current stream are the only things torch provides) and call the same entry
points. Every step of the computation runs in the library's HIP kernels;
there is no other path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsaidx.so")

DENSE, REUSE, REFINE = 0, 1, 2
STATUS = {0: "OK", 1: "EINVAL", 2: "EUNSUPPORTED", 3: "EWORKSPACE", 4: "EHIP"}
EXPORTS = ("indexer_workspace_bytes", "indexer_dense", "indexer_pivot_reuse",
           "indexer_pivot_refine", "indexer_varlen_workspace_bytes", "indexer_dense_varlen",
           "indexer_pivot_reuse_varlen", "indexer_pivot_refine_varlen", "indexer_chunks_fixed",
           "indexer_chunks_adaptive_workspace_bytes", "indexer_chunks_adaptive", "indexer_chunk_means",
           "indexer_chunk_refine_workspace_bytes", "indexer_chunk_refine", "indexer_sort_rows",
           "indexer_last_error", "indexer_version", "indexer_pivot_refine_noalloc",
           "indexer_chunks_fixed_varlen", "indexer_chunks_adaptive_varlen_workspace_bytes",
           "indexer_chunks_adaptive_varlen", "indexer_chunk_means_varlen",
           "indexer_chunk_refine_varlen_workspace_bytes", "indexer_chunk_refine_varlen")


class IndexerError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libdsaidx.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m sparse_attention_indexer_dense_amd.build`")
    lib = ctypes.CDLL(path)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.indexer_workspace_bytes.argtypes = [i32, i32, i64, i64, i32, i32, i32, i32, i32]
    lib.indexer_workspace_bytes.restype = sz
    lib.indexer_dense.argtypes = [P, P, P, i32, i64, i64, i32, i32, i32, P, P, P, sz, P]
    lib.indexer_dense.restype = i32
    for f in (lib.indexer_pivot_reuse, lib.indexer_pivot_refine):
        f.argtypes = [P, P, P, i32, i64, i64, i32, i32, i32, i32, i32, P, P, P, P, sz, P]
        f.restype = i32
    lib.indexer_pivot_refine_noalloc.argtypes = [P, P, P, i32, i64, i64, i32, i32, i32, i32, i32, P, P, P, P]
    lib.indexer_pivot_refine_noalloc.restype = i32
    lib.indexer_varlen_workspace_bytes.argtypes = [i32, i32, P, P, i32, i32, i32, i32, i32, P]
    lib.indexer_varlen_workspace_bytes.restype = sz
    lib.indexer_dense_varlen.argtypes = [P, P, P, i32, P, P, i32, i32, i32, P, P, P, sz, P]
    lib.indexer_dense_varlen.restype = i32
    for f in (lib.indexer_pivot_reuse_varlen, lib.indexer_pivot_refine_varlen):
        f.argtypes = [P, P, P, i32, P, P, i32, i32, i32, i32, i32, P, P, P, P, P, sz, P]
        f.restype = i32
    lib.indexer_chunks_fixed.argtypes = [i32, i64, i32, P, P]
    lib.indexer_chunks_fixed.restype = i32
    lib.indexer_chunks_adaptive_workspace_bytes.argtypes = [i32, i64, i32]
    lib.indexer_chunks_adaptive_workspace_bytes.restype = sz
    lib.indexer_chunks_adaptive.argtypes = [P, i32, i64, i32, i32, P, P, sz, P]
    lib.indexer_chunks_adaptive.restype = i32
    lib.indexer_chunk_means.argtypes = [P, i32, i64, i32, P, i64, i64, P, P]
    lib.indexer_chunk_means.restype = i32
    lib.indexer_chunk_refine_workspace_bytes.argtypes = [i32, i64, i64, i32, i32, i32, i64, i32, i32, i32, P]
    lib.indexer_chunk_refine_workspace_bytes.restype = sz
    lib.indexer_chunk_refine.argtypes = [P, P, P, P, P, i64, i32, i64, i64, i32, i32, i32, i32, i32, i32, P,
                                         P, P, P, P, P, sz, P]
    lib.indexer_chunk_refine.restype = i32
    lib.indexer_chunks_fixed_varlen.argtypes = [i32, P, i32, P, P]
    lib.indexer_chunks_fixed_varlen.restype = i32
    lib.indexer_chunks_adaptive_varlen_workspace_bytes.argtypes = [i32, P, i32]
    lib.indexer_chunks_adaptive_varlen_workspace_bytes.restype = sz
    lib.indexer_chunks_adaptive_varlen.argtypes = [P, i32, P, i32, i32, P, P, sz, P]
    lib.indexer_chunks_adaptive_varlen.restype = i32
    lib.indexer_chunk_means_varlen.argtypes = [P, i32, P, i32, P, P, P, P]
    lib.indexer_chunk_means_varlen.restype = i32
    lib.indexer_chunk_refine_varlen_workspace_bytes.argtypes = [i32, P, P, i32, i32, i32, P, i32, i32, i32, P]
    lib.indexer_chunk_refine_varlen_workspace_bytes.restype = sz
    lib.indexer_chunk_refine_varlen.argtypes = [P, P, P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, P,
                                                P, P, P, P, P, sz, P]
    lib.indexer_chunk_refine_varlen.restype = i32
    lib.indexer_sort_rows.argtypes = [P, P, i64, i32, P]
    lib.indexer_sort_rows.restype = i32
    lib.indexer_last_error.argtypes = []
    lib.indexer_last_error.restype = ctypes.c_char_p
    lib.indexer_version.argtypes = []
    lib.indexer_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---------------------------------------------------------------- raw C ABI
def indexer_workspace_bytes(mode, B, L, q_len, H_I, d_I, g, c, k):
    return load().indexer_workspace_bytes(mode, B, L, q_len, H_I, d_I, g, c, k)


def indexer_dense(Q, W, K, B, L, q_len, H_I, d_I, k, out_idx, out_score, ws, ws_bytes, stream):
    return load().indexer_dense(Q, W, K, B, L, q_len, H_I, d_I, k, out_idx, out_score, ws,
                                ws_bytes, stream)


def indexer_pivot_reuse(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, out_idx, out_score, out_cand,
                        ws, ws_bytes, stream):
    return load().indexer_pivot_reuse(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, out_idx, out_score,
                                      out_cand, ws, ws_bytes, stream)


def indexer_pivot_refine(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, out_idx, out_score, out_cand,
                         ws, ws_bytes, stream):
    return load().indexer_pivot_refine(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, out_idx, out_score,
                                       out_cand, ws, ws_bytes, stream)


def indexer_pivot_refine_noalloc(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, out_idx, out_score, out_cand,
                                 stream):
    return load().indexer_pivot_refine_noalloc(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, out_idx,
                                               out_score, out_cand, stream)


class PivotOpts(ctypes.Structure):
    """dsaidx_pivot_opts: guard, proxy strategy, proxy window."""
    _fields_ = [("guard", ctypes.c_int64), ("proxy", ctypes.c_int32), ("window", ctypes.c_int32)]


PROXY = {"mean": 0, "first": 1, "last": 2}


def indexer_varlen_workspace_bytes(mode, B, L, q_len, H_I, d_I, g, c, k, opts):
    return load().indexer_varlen_workspace_bytes(mode, B, L, q_len, H_I, d_I, g, c, k, opts)


def indexer_dense_varlen(Q, W, K, B, L, q_len, H_I, d_I, k, out_idx, out_score, ws, ws_bytes, stream):
    return load().indexer_dense_varlen(Q, W, K, B, L, q_len, H_I, d_I, k, out_idx, out_score, ws,
                                       ws_bytes, stream)


def indexer_pivot_reuse_varlen(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, opts, out_idx, out_score,
                               out_cand, ws, ws_bytes, stream):
    return load().indexer_pivot_reuse_varlen(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, opts, out_idx,
                                             out_score, out_cand, ws, ws_bytes, stream)


def indexer_pivot_refine_varlen(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, opts, out_idx, out_score,
                                out_cand, ws, ws_bytes, stream):
    return load().indexer_pivot_refine_varlen(Q, W, K, B, L, q_len, H_I, d_I, g, c, k, opts, out_idx,
                                              out_score, out_cand, ws, ws_bytes, stream)


def indexer_chunks_fixed(B, L, block, cend, stream):
    return load().indexer_chunks_fixed(B, L, block, cend, stream)


def indexer_chunks_adaptive_workspace_bytes(B, L, block):
    return load().indexer_chunks_adaptive_workspace_bytes(B, L, block)


def indexer_chunks_adaptive(K, B, L, d_I, block, cend, ws, ws_bytes, stream):
    return load().indexer_chunks_adaptive(K, B, L, d_I, block, cend, ws, ws_bytes, stream)


def indexer_chunk_means(K, B, L, d_I, cend, nc, first, Kbar, stream):
    return load().indexer_chunk_means(K, B, L, d_I, cend, nc, first, Kbar, stream)


def indexer_chunk_refine_workspace_bytes(B, L, q_len, H_I, d_I, g, nc, nsel, max_chunk, k, opts=None):
    return load().indexer_chunk_refine_workspace_bytes(B, L, q_len, H_I, d_I, g, nc, nsel, max_chunk, k, opts)


def indexer_chunk_refine(Q, W, K, Kbar, cend, nc, B, L, q_len, H_I, d_I, g, nsel, max_chunk, k, opts,
                         out_idx, out_score, out_chunks, out_cand, ws, ws_bytes, stream):
    return load().indexer_chunk_refine(Q, W, K, Kbar, cend, nc, B, L, q_len, H_I, d_I, g, nsel, max_chunk,
                                       k, opts, out_idx, out_score, out_chunks, out_cand, ws, ws_bytes,
                                       stream)


def indexer_chunks_fixed_varlen(B, L, block, cend, stream):
    return load().indexer_chunks_fixed_varlen(B, L, block, cend, stream)


def indexer_chunks_adaptive_varlen_workspace_bytes(B, L, block):
    return load().indexer_chunks_adaptive_varlen_workspace_bytes(B, L, block)


def indexer_chunks_adaptive_varlen(K, B, L, d_I, block, cend, ws, ws_bytes, stream):
    return load().indexer_chunks_adaptive_varlen(K, B, L, d_I, block, cend, ws, ws_bytes, stream)


def indexer_chunk_means_varlen(K, B, L, d_I, cend, nc, Kbar, stream):
    return load().indexer_chunk_means_varlen(K, B, L, d_I, cend, nc, Kbar, stream)


def indexer_chunk_refine_varlen_workspace_bytes(B, L, q_len, H_I, d_I, g, nc, nsel, max_chunk, k, opts=None):
    return load().indexer_chunk_refine_varlen_workspace_bytes(B, L, q_len, H_I, d_I, g, nc, nsel, max_chunk,
                                                              k, opts)


def indexer_chunk_refine_varlen(Q, W, K, Kbar, cend, nc, B, L, q_len, H_I, d_I, g, nsel, max_chunk, k, opts,
                                out_idx, out_score, out_chunks, out_cand, ws, ws_bytes, stream):
    return load().indexer_chunk_refine_varlen(Q, W, K, Kbar, cend, nc, B, L, q_len, H_I, d_I, g, nsel,
                                              max_chunk, k, opts, out_idx, out_score, out_chunks, out_cand,
                                              ws, ws_bytes, stream)


def indexer_sort_rows(idx, score, rows, k, stream):
    return load().indexer_sort_rows(idx, score, rows, k, stream)


def indexer_last_error():
    return load().indexer_last_error().decode()


def indexer_version():
    return load().indexer_version().decode()


# ------------------------------------------------------------ torch helpers
def _shapes(Q, W, K):
    import torch
    if Q.dtype != torch.bfloat16 or K.dtype != torch.bfloat16 or W.dtype != torch.float32:
        raise TypeError("Q and K must be bf16, W fp32")
    if not (Q.is_cuda and W.is_cuda and K.is_cuda):
        raise ValueError("Q, W and K must be GPU tensors")
    if Q.dim() != 4 or W.dim() != 3 or K.dim() != 3:
        raise ValueError("expected Q [B,q_len,H,d], W [B,q_len,H], K [B,L,d]")
    B, q_len, H, d = Q.shape
    if tuple(W.shape) != (B, q_len, H) or K.shape[0] != B or K.shape[2] != d:
        raise ValueError("inconsistent Q/W/K shapes")
    for t in (Q, W, K):
        if not t.is_contiguous():
            raise ValueError("Q, W and K must be contiguous")
    return B, K.shape[1], q_len, H, d


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(rc):
    if rc != 0:
        raise IndexerError(rc, indexer_last_error())


class Workspace:
    """Reusable device workspace (grown on demand). Calls that share one
    workspace must not overlap in time: use one per stream."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes, device):
        import torch
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


class _StreamWorkspaces:
    """The default workspace: one per (device, stream), so that calls issued on
    different streams never share scratch memory. (A buffer that grows is
    replaced only for calls on its own stream, where the caching allocator
    may reuse the old one once that stream passes the calls that used it.)"""

    def __init__(self):
        self._ws = {}

    def get(self, nbytes, device):
        import torch
        device = torch.device(device)
        stream = torch.cuda.current_stream(device).cuda_stream
        key = (device.index if device.index is not None else torch.cuda.current_device(), stream)
        ws = self._ws.get(key)
        if ws is None:
            ws = self._ws[key] = Workspace()
        return ws.get(nbytes, device)


_default_ws = _StreamWorkspaces()


def _check_out(t, name, shape, dtype, device):
    """A caller-provided output tensor must match what the kernels write."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")


def _run(mode, Q, W, K, k, g=1, c=0, scores=True, cand=False, ws=None, out=None):
    import torch
    B, L, q_len, H, d = _shapes(Q, W, K)
    dev = Q.device
    # an invalid call sizes to 0 bytes; the entry point then reports the error
    need = indexer_workspace_bytes(mode, B, L, q_len, H, d, g, c, k)
    wsb = (ws or _default_ws).get(need, dev)
    if out is None:
        out_idx = torch.empty((B, q_len, k), dtype=torch.int32, device=dev)
        out_score = torch.empty((B, q_len, k), dtype=torch.float32, device=dev) if scores else None
        G = (q_len + g - 1) // g
        out_cand = torch.empty((B, G, c), dtype=torch.int32, device=dev) if cand else None
    else:
        out_idx, out_score, out_cand = (tuple(out) + (None, None))[:3]
        if out_idx is None:
            raise ValueError("out must hold out_idx")
        G = (q_len + g - 1) // g
        _check_out(out_idx, "out_idx", (B, q_len, k), torch.int32, dev)
        _check_out(out_score, "out_score", (B, q_len, k), torch.float32, dev)
        if mode == DENSE:
            out_cand = None
        else:
            _check_out(out_cand, "out_cand", (B, G, c), torch.int32, dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if mode == DENSE:
        rc = indexer_dense(_ptr(Q), _ptr(W), _ptr(K), B, L, q_len, H, d, k, _ptr(out_idx),
                           _ptr(out_score), _ptr(wsb), wsb.numel(), stream)
    else:
        f = indexer_pivot_reuse if mode == REUSE else indexer_pivot_refine
        rc = f(_ptr(Q), _ptr(W), _ptr(K), B, L, q_len, H, d, g, c, k, _ptr(out_idx),
               _ptr(out_score), _ptr(out_cand), _ptr(wsb), wsb.numel(), stream)
    _check(rc)
    return out_idx, out_score, out_cand


def dense(Q, W, K, k, scores=True, ws=None, out=None):
    """Dense DSA indexer: (idx [B,q_len,k] int32, score fp32 or None)."""
    i, s, _ = _run(DENSE, Q, W, K, k, scores=scores, ws=ws, out=out)
    return i, s


def pivot_reuse(Q, W, K, g, k, c=0, scores=True, cand=False, ws=None, out=None):
    """PIVOT-Reuse: (idx, score or None, cand [B,G,c] or None)."""
    return _run(REUSE, Q, W, K, k, g=g, c=c, scores=scores, cand=cand, ws=ws, out=out)


def pivot_refine(Q, W, K, g, c, k, scores=True, cand=False, ws=None, out=None):
    """PIVOT-Refine: (idx, score or None, cand [B,G,c] or None)."""
    return _run(REFINE, Q, W, K, k, g=g, c=c, scores=scores, cand=cand, ws=ws, out=out)


# ------------------------------------------------------ variable-length batches
def _varlen_shapes(Q, W, K, L, q_len):
    import torch
    if Q.dtype != torch.bfloat16 or K.dtype != torch.bfloat16 or W.dtype != torch.float32:
        raise TypeError("Q and K must be bf16, W fp32")
    if not (Q.is_cuda and W.is_cuda and K.is_cuda):
        raise ValueError("Q, W and K must be GPU tensors")
    if Q.dim() != 3 or W.dim() != 2 or K.dim() != 2:
        raise ValueError("expected packed Q [sum q_len, H, d], W [sum q_len, H], K [sum L, d]")
    for t in (Q, W, K):
        if not t.is_contiguous():
            raise ValueError("Q, W and K must be contiguous")
    L = [int(x) for x in L]
    q_len = [int(x) for x in q_len]
    if len(L) != len(q_len) or not L:
        raise ValueError("L and q_len must list the same, nonzero number of requests")
    nq, H, d = Q.shape
    if nq != sum(q_len) or K.shape[0] != sum(L) or K.shape[1] != d or tuple(W.shape) != (nq, H):
        raise ValueError("packed shapes do not match the request lengths")
    arr = ctypes.c_int64 * len(L)
    return len(L), arr(*L), arr(*q_len), H, d


def _run_varlen(mode, Q, W, K, L, q_len, k, g=1, c=0, guard=0, proxy="mean", window=0, scores=True,
                cand=False, ws=None):
    import torch
    B, La, qa, H, d = _varlen_shapes(Q, W, K, L, q_len)
    dev = Q.device
    if proxy not in PROXY:
        raise ValueError(f"proxy must be one of {sorted(PROXY)}")
    opts = ctypes.byref(PivotOpts(int(guard), PROXY[proxy], int(window)))
    need = indexer_varlen_workspace_bytes(mode, B, La, qa, H, d, g, c, k, opts)
    wsb = (ws or _default_ws).get(need, dev)
    nq = Q.shape[0]
    out_idx = torch.empty((nq, k), dtype=torch.int32, device=dev)
    out_score = torch.empty((nq, k), dtype=torch.float32, device=dev) if scores else None
    ng = sum((int(x) + g - 1) // g for x in q_len)
    out_cand = torch.empty((ng, c), dtype=torch.int32, device=dev) if cand else None
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if mode == DENSE:
        rc = indexer_dense_varlen(_ptr(Q), _ptr(W), _ptr(K), B, La, qa, H, d, k, _ptr(out_idx),
                                  _ptr(out_score), _ptr(wsb), wsb.numel(), stream)
    else:
        f = indexer_pivot_reuse_varlen if mode == REUSE else indexer_pivot_refine_varlen
        rc = f(_ptr(Q), _ptr(W), _ptr(K), B, La, qa, H, d, g, c, k, opts, _ptr(out_idx),
               _ptr(out_score), _ptr(out_cand), _ptr(wsb), wsb.numel(), stream)
    _check(rc)
    return out_idx, out_score, out_cand


def dense_varlen(Q, W, K, L, q_len, k, scores=True, ws=None):
    """Dense indexer over packed requests: (idx [sum q_len, k], score or None)."""
    i, s, _ = _run_varlen(DENSE, Q, W, K, L, q_len, k, scores=scores, ws=ws)
    return i, s


def pivot_reuse_varlen(Q, W, K, L, q_len, g, k, c=0, guard=0, proxy="mean", window=0, scores=True,
                       cand=False, ws=None):
    """PIVOT-Reuse over packed requests: (idx, score or None, cand [sum G, c] or None)."""
    return _run_varlen(REUSE, Q, W, K, L, q_len, k, g=g, c=c, guard=guard, proxy=proxy,
                       window=window, scores=scores, cand=cand, ws=ws)


def pivot_refine_varlen(Q, W, K, L, q_len, g, c, k, guard=0, proxy="mean", window=0, scores=True,
                        cand=False, ws=None):
    """PIVOT-Refine over packed requests: (idx, score or None, cand [sum G, c] or None)."""
    return _run_varlen(REFINE, Q, W, K, L, q_len, k, g=g, c=c, guard=guard, proxy=proxy,
                       window=window, scores=scores, cand=cand, ws=ws)


# ------------------------------------------------- key chunks (coarse stage)
def _stream(dev):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def chunks_fixed(B, L, block, device="cuda"):
    """Chunk ends of fixed blocks: int32 [B, ceil(L / block)]."""
    import torch
    dev = torch.device(device)
    cend = torch.empty((B, -(-L // block)), dtype=torch.int32, device=dev)
    _check(indexer_chunks_fixed(B, L, block, _ptr(cend), _stream(dev)))
    return cend


def chunks_adaptive(K, block, ws=None):
    """Score-adaptive chunk ends of K [B, L, d] (split/merge under the
    fixed-block budget): int32 [B, ceil(L / block)]."""
    import torch
    if K.dtype != torch.bfloat16 or K.dim() != 3 or not K.is_cuda or not K.is_contiguous():
        raise ValueError("K must be a contiguous bf16 GPU tensor [B, L, d]")
    B, L, d = K.shape
    dev = K.device
    need = indexer_chunks_adaptive_workspace_bytes(B, L, block)
    wsb = (ws or _default_ws).get(need, dev)
    cend = torch.empty((B, -(-L // block)), dtype=torch.int32, device=dev)
    _check(indexer_chunks_adaptive(_ptr(K), B, L, d, block, _ptr(cend), _ptr(wsb), wsb.numel(),
                                   _stream(dev)))
    return cend


def chunk_means(K, cend, first=0, out=None):
    """Mean-key summaries bf16 [B, nc, d] of the chunks of K [B, L, d]."""
    import torch
    B, L, d = K.shape
    nc = cend.shape[1]
    if cend.dtype != torch.int32 or tuple(cend.shape) != (B, nc) or not cend.is_contiguous():
        raise ValueError("cend must be contiguous int32 [B, nc]")
    Kbar = out if out is not None else torch.empty((B, nc, d), dtype=torch.bfloat16, device=K.device)
    _check(indexer_chunk_means(_ptr(K), B, L, d, _ptr(cend), nc, first, _ptr(Kbar), _stream(K.device)))
    return Kbar


def chunk_refine(Q, W, K, Kbar, cend, g, nsel, max_chunk, k, proxy="mean", window=0, scores=True,
                 chunks=False, cand=False, ws=None, guard=0):
    """Chunk-level candidates and token-level Refine: (idx [B, q_len, k], score or
    None, selected chunks [B, G, nsel] or None, candidate lists [B, G, cw] or
    None), cw = (nsel + 1) * max_chunk."""
    import torch
    B, L, q_len, H, d = _shapes(Q, W, K)
    nc = cend.shape[1]
    if tuple(Kbar.shape) != (B, nc, d) or Kbar.dtype != torch.bfloat16 or not Kbar.is_contiguous():
        raise ValueError("Kbar must be contiguous bf16 [B, nc, d]")
    if cend.dtype != torch.int32 or tuple(cend.shape) != (B, nc) or not cend.is_contiguous():
        raise ValueError("cend must be contiguous int32 [B, nc]")
    if proxy not in PROXY:
        raise ValueError(f"proxy must be one of {sorted(PROXY)}")
    dev = Q.device
    opts = ctypes.byref(PivotOpts(int(guard), PROXY[proxy], int(window)))
    need = indexer_chunk_refine_workspace_bytes(B, L, q_len, H, d, g, nc, nsel, max_chunk, k, opts)
    wsb = (ws or _default_ws).get(need, dev)
    G = (q_len + g - 1) // g
    cw = (nsel + 1) * max_chunk
    out_idx = torch.empty((B, q_len, k), dtype=torch.int32, device=dev)
    out_score = torch.empty((B, q_len, k), dtype=torch.float32, device=dev) if scores else None
    out_chunks = torch.empty((B, G, nsel), dtype=torch.int32, device=dev) if chunks else None
    out_cand = torch.empty((B, G, cw), dtype=torch.int32, device=dev) if cand else None
    _check(indexer_chunk_refine(_ptr(Q), _ptr(W), _ptr(K), _ptr(Kbar), _ptr(cend), nc, B, L, q_len, H, d,
                                g, nsel, max_chunk, k, opts, _ptr(out_idx), _ptr(out_score),
                                _ptr(out_chunks), _ptr(out_cand), _ptr(wsb), wsb.numel(),
                                _stream(dev)))
    return out_idx, out_score, out_chunks, out_cand


def _i64(xs):
    xs = [int(x) for x in xs]
    return len(xs), (ctypes.c_int64 * len(xs))(*xs), xs


def chunks_fixed_varlen(L, block, device="cuda"):
    """Chunk ends of fixed blocks for requests of L[r] keys, one after the
    other: (cend int32 [sum nc], nc list), nc[r] = ceil(L[r] / block)."""
    import torch
    dev = torch.device(device)
    B, La, Ls = _i64(L)
    nc = [-(-x // block) for x in Ls]
    cend = torch.empty((sum(nc),), dtype=torch.int32, device=dev)
    _check(indexer_chunks_fixed_varlen(B, La, block, _ptr(cend), _stream(dev)))
    return cend, nc


def chunks_adaptive_varlen(K, L, block, ws=None):
    """Score-adaptive chunk ends of packed keys K [sum L, d] per request:
    (cend int32 [sum nc], nc list), nc[r] = ceil(L[r] / block)."""
    import torch
    if K.dtype != torch.bfloat16 or K.dim() != 2 or not K.is_cuda or not K.is_contiguous():
        raise ValueError("K must be a contiguous bf16 GPU tensor [sum L, d]")
    B, La, Ls = _i64(L)
    if K.shape[0] != sum(Ls):
        raise ValueError("K rows do not match the request lengths")
    dev = K.device
    need = indexer_chunks_adaptive_varlen_workspace_bytes(B, La, block)
    wsb = (ws or _default_ws).get(need, dev)
    nc = [-(-x // block) for x in Ls]
    cend = torch.empty((sum(nc),), dtype=torch.int32, device=dev)
    _check(indexer_chunks_adaptive_varlen(_ptr(K), B, La, K.shape[1], block, _ptr(cend), _ptr(wsb), wsb.numel(),
                                          _stream(dev)))
    return cend, nc


def chunk_means_varlen(K, L, cend, nc, out=None):
    """Mean-key summaries bf16 [sum nc, d] of the chunks of packed keys K [sum L, d]."""
    import torch
    B, La, Ls = _i64(L)
    _, nca, ncs = _i64(nc)
    if len(ncs) != B or K.shape[0] != sum(Ls):
        raise ValueError("L, nc and K rows do not match")
    if cend.dtype != torch.int32 or tuple(cend.shape) != (sum(ncs),) or not cend.is_contiguous():
        raise ValueError("cend must be contiguous int32 [sum nc]")
    d = K.shape[1]
    Kbar = out if out is not None else torch.empty((sum(ncs), d), dtype=torch.bfloat16, device=K.device)
    _check(indexer_chunk_means_varlen(_ptr(K), B, La, d, _ptr(cend), nca, _ptr(Kbar), _stream(K.device)))
    return Kbar


def chunk_refine_varlen(Q, W, K, Kbar, cend, L, q_len, nc, g, nsel, max_chunk, k, proxy="mean", window=0,
                        scores=True, chunks=False, cand=False, ws=None, guard=0):
    """The key-chunk path over packed requests: (idx [sum q_len, k], score or
    None, selected chunks [sum G, nsel] or None, candidate lists [sum G, cw]
    or None), G_r = ceil(q_len[r] / g), cw = (nsel + 1) * max_chunk."""
    import torch
    B, La, qa, H, d = _varlen_shapes(Q, W, K, L, q_len)
    _, nca, ncs = _i64(nc)
    if len(ncs) != B:
        raise ValueError("nc must list one chunk count per request")
    if tuple(Kbar.shape) != (sum(ncs), d) or Kbar.dtype != torch.bfloat16 or not Kbar.is_contiguous():
        raise ValueError("Kbar must be contiguous bf16 [sum nc, d]")
    if cend.dtype != torch.int32 or tuple(cend.shape) != (sum(ncs),) or not cend.is_contiguous():
        raise ValueError("cend must be contiguous int32 [sum nc]")
    if proxy not in PROXY:
        raise ValueError(f"proxy must be one of {sorted(PROXY)}")
    dev = Q.device
    opts = ctypes.byref(PivotOpts(int(guard), PROXY[proxy], int(window)))
    need = indexer_chunk_refine_varlen_workspace_bytes(B, La, qa, H, d, g, nca, nsel, max_chunk, k, opts)
    wsb = (ws or _default_ws).get(need, dev)
    nq = Q.shape[0]
    ng = sum((int(x) + g - 1) // g for x in q_len)
    cw = (nsel + 1) * max_chunk
    out_idx = torch.empty((nq, k), dtype=torch.int32, device=dev)
    out_score = torch.empty((nq, k), dtype=torch.float32, device=dev) if scores else None
    out_chunks = torch.empty((ng, nsel), dtype=torch.int32, device=dev) if chunks else None
    out_cand = torch.empty((ng, cw), dtype=torch.int32, device=dev) if cand else None
    _check(indexer_chunk_refine_varlen(_ptr(Q), _ptr(W), _ptr(K), _ptr(Kbar), _ptr(cend), nca, B, La, qa, H, d,
                                       g, nsel, max_chunk, k, opts, _ptr(out_idx), _ptr(out_score),
                                       _ptr(out_chunks), _ptr(out_cand), _ptr(wsb), wsb.numel(), _stream(dev)))
    return out_idx, out_score, out_chunks, out_cand


def sort_rows(idx, score):
    """Reorder output rows (idx int32 [..., k], score fp32 [..., k], both on the
    GPU) in place into ranking order: score descending, ties by ascending index,
    -1 padding last. Returns (idx, score)."""
    import torch
    if idx.dtype != torch.int32 or score.dtype != torch.float32 or idx.shape != score.shape:
        raise ValueError("idx (int32) and score (fp32) of one shape are required")
    if not (idx.is_cuda and score.is_cuda and idx.is_contiguous() and score.is_contiguous()):
        raise ValueError("idx and score must be contiguous GPU tensors")
    k = idx.shape[-1]
    rows = idx.numel() // k if k else 0
    _check(indexer_sort_rows(_ptr(idx), _ptr(score), rows, k, _stream(idx.device)))
    return idx, score
