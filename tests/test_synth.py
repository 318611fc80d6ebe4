"""The seeded input generator: shapes, determinism and the stated statistics."""
import numpy as np
import torch

import synth


def test_prefill_shapes_and_determinism():
    Q, W, K = synth.prefill(300, 4, 32, 0.9, 2, seed=3)
    assert Q.shape == (1, 300, 4, 32) and Q.dtype == torch.bfloat16
    assert W.shape == (1, 300, 4) and W.dtype == torch.float32
    assert K.shape == (1, 300, 32) and K.dtype == torch.bfloat16
    Q2, W2, K2 = synth.prefill(300, 4, 32, 0.9, 2, seed=3)
    assert torch.equal(Q, Q2) and torch.equal(W, W2) and torch.equal(K, K2)
    Q3, _, _ = synth.prefill(300, 4, 32, 0.9, 2, seed=4)
    assert not torch.equal(Q, Q3)


def test_statistics():
    rho = 0.9
    Q, W, K = synth.prefill(8192, 4, 32, rho, 2, seed=1)
    q = Q[0].float().reshape(8192, -1)[100:]
    # stationary AR(1): lag-1 correlation rho, variance 1 / (1 - rho^2)
    r1 = (q[1:] * q[:-1]).mean() / (q * q).mean()
    assert abs(float(r1) - rho) < 0.01
    assert abs(float(q.var()) - 1 / (1 - rho * rho)) < 0.3
    w = W[0]
    assert float(w.min()) >= 0 and float(w.max()) <= 1 / 4
    # keys: isotropic part of variance 1/d per dim plus the rank-2 component
    k = K[0].float()
    assert 0.5 / 32 < float(k.var(dim=0).mean()) < 10 / 32


def test_chunk_boundary_is_continuous():
    # the AR(1) state carries across generation chunks
    L = synth.QUERY_CHUNK + 64
    Q, _, _ = synth.prefill(L, 1, 16, 0.99, 0, seed=2)
    q = Q[0, :, 0, :].float()
    c = synth.QUERY_CHUNK
    jump = (q[c] - q[c - 1]).abs().mean()
    typical = (q[1:c] - q[:c - 1]).abs().mean()
    assert float(jump) < 3 * float(typical)


def test_decode_shapes():
    Q, W, K = synth.decode(3, 500, 2, 4, 32, 0.95, 2, seed=0)
    assert Q.shape == (3, 2, 4, 32) and W.shape == (3, 2, 4) and K.shape == (3, 500, 32)
    assert not torch.equal(K[0], K[1])


def test_u16_roundtrip():
    t = torch.randn(5, 7).to(torch.bfloat16)
    a = synth.to_u16(t)
    assert a.dtype == np.uint16
    assert torch.equal(synth.from_u16(a), t)
