"""indexer_pivot_refine_noalloc (scratch held by the library, no workspace
argument) against indexer_pivot_refine (caller's workspace), both called
through the C ABI: identical outputs, bit for bit, on two calls in a row, the
second with a smaller input, on both kernel families (few rows per request:
the decode shape; many rows: a prefill sequence). Sizes beyond the scratch are
rejected before anything is enqueued."""
import ctypes

import pytest
import torch

import sparse_attention_indexer_dense_amd as dsa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EWORKSPACE = 3


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)


def outputs(B, q_len, G, c, k, fill):
    return (torch.full((B, q_len, k), fill, dtype=torch.int32, device=DEV),
            torch.full((B, q_len, k), float(fill), dtype=torch.float32, device=DEV),
            torch.full((B, G, c), fill, dtype=torch.int32, device=DEV))


def run_both(Q, W, K, g, c, k):
    B, q_len, H, d = Q.shape
    L = K.shape[1]
    G = (q_len + g - 1) // g
    # the outputs start from different garbage, so equal results are written
    ref = outputs(B, q_len, G, c, k, 7)
    got = outputs(B, q_len, G, c, k, -7)
    need = dsa.indexer_workspace_bytes(dsa.REFINE, B, L, q_len, H, d, g, c, k)
    assert 0 < need <= 64 << 20
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    rc = dsa.indexer_pivot_refine(ptr(Q), ptr(W), ptr(K), B, L, q_len, H, d, g, c, k, ptr(ref[0]),
                                  ptr(ref[1]), ptr(ref[2]), ptr(ws), need, stream())
    assert rc == 0, dsa.indexer_last_error()
    rc = dsa.indexer_pivot_refine_noalloc(ptr(Q), ptr(W), ptr(K), B, L, q_len, H, d, g, c, k, ptr(got[0]),
                                          ptr(got[1]), ptr(got[2]), stream())
    assert rc == 0, dsa.indexer_last_error()
    # without candidates
    got2 = outputs(B, q_len, G, c, k, 5)
    rc = dsa.indexer_pivot_refine_noalloc(ptr(Q), ptr(W), ptr(K), B, L, q_len, H, d, g, c, k, ptr(got2[0]),
                                          ptr(got2[1]), None, stream())
    assert rc == 0, dsa.indexer_last_error()
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    assert torch.equal(ref[0], got2[0]) and torch.equal(ref[1], got2[1])
    assert bool((ref[0] >= -1).all()) and bool((ref[0][..., 0] >= 0).all())


def test_noalloc_decode_shape_twice():
    # few rows per request (split kernels), then a smaller batch
    Q, W, K = synth.decode(6, 20000, 2, 64, 128, 0.95, 4, seed=11, device=DEV)
    run_both(Q, W, K, 2, 1024, 512)
    Q, W, K = synth.decode(3, 5000, 2, 64, 128, 0.95, 4, seed=12, device=DEV)
    run_both(Q, W, K, 2, 512, 256)


def test_noalloc_prefill_shape_twice():
    # many rows (fused scan kernels), then a smaller sequence
    Q, W, K = synth.prefill(1000, 4, 32, 0.9, 2, 13, DEV)
    run_both(Q, W, K, 4, 256, 64)
    Q, W, K = synth.prefill(600, 4, 32, 0.9, 2, 14, DEV)
    run_both(Q, W, K, 4, 128, 32)


def test_noalloc_rejects_sizes_beyond_scratch():
    B, L, q_len, H, d, g, c, k = 64, 1 << 20, 2, 64, 128, 2, 4096, 2048
    need = dsa.indexer_workspace_bytes(dsa.REFINE, B, L, q_len, H, d, g, c, k)
    assert need > 64 << 20
    fake = ctypes.c_void_p(0x100000)
    rc = dsa.indexer_pivot_refine_noalloc(fake, fake, fake, B, L, q_len, H, d, g, c, k, fake, None, None,
                                          stream())
    assert rc == EWORKSPACE
    assert "scratch" in dsa.indexer_last_error()
