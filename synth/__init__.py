"""Seeded synthetic inputs for the DSA indexer (queries, weights, keys).

This module holds no indexer arithmetic: it only draws random tensors. It is the
one module that the GPU path's callers and the CPU oracle's callers share.

Recipe (the paper's workloads are long-context benchmarks run through trained
models; these tensors stand in for the indexer activations at the same shapes):

* keys   k_s = z_s / sqrt(d) + sum_r a_{s,r} u_r, with z_s ~ N(0, I_d),
  u_r ~ N(0, I_d) / sqrt(d) shared by every key (a rank-R common component
  that makes the ReLU scores long-tailed) and a_{s,r} ~ N(0, coef_var);
* queries follow an independent AR(1) process along positions for every
  (head, dim) lane: q_t = rho * q_{t-1} + e_t, e_t ~ N(0, 1), q_{-1} = 0,
  so neighbouring queries are correlated;
* weights w_{t,j} ~ U(0, 1) / H;
* queries and keys are drawn in fp32 and rounded to bf16 (nearest-even).

Every draw comes from its own generator seeded by (seed, stream, chunk), so a
tensor does not depend on how other tensors were drawn. The values depend on
the device's generator (CPU and GPU draw different numbers for one seed): a
check always hands the oracle a host copy of the very tensors the GPU used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

KEY_CHUNK = 65536
QUERY_CHUNK = 4096

STREAM_KEY_NOISE = 0
STREAM_QUERY = 1
STREAM_WEIGHT = 2
STREAM_KEY_DIRS = 3
STREAM_KEY_COEF = 4
STREAM_QUERY_START = 5
STREAM_LOCAL_COEF = 6
STREAM_LOCAL_JUMP = 7
STREAM_LOCAL_OFFSET = 8
STREAM_LOCAL_SCALE = 9


def _sub_seed(seed: int, stream: int, chunk: int) -> int:
    ss = np.random.SeedSequence([int(seed), int(stream), int(chunk)])
    return int(ss.generate_state(1, np.uint64)[0] >> np.uint64(1))


def _gen(device, seed, stream, chunk):
    g = torch.Generator(device=device)
    g.manual_seed(_sub_seed(seed, stream, chunk))
    return g


def keys(L, d, rank, seed, device="cpu", coef_var=0.5, out=None):
    """Keys [L, d] bf16 (see the module recipe)."""
    device = torch.device(device)
    if out is None:
        out = torch.empty((L, d), dtype=torch.bfloat16, device=device)
    u = torch.randn((max(rank, 1), d), generator=_gen(device, seed, STREAM_KEY_DIRS, 0),
                    device=device) / math.sqrt(d)
    for c0 in range(0, L, KEY_CHUNK):
        c1 = min(L, c0 + KEY_CHUNK)
        n = c1 - c0
        chunk = c0 // KEY_CHUNK
        z = torch.randn((n, d), generator=_gen(device, seed, STREAM_KEY_NOISE, chunk),
                        device=device)
        kf = z / math.sqrt(d)
        if rank > 0:
            a = torch.randn((n, rank), generator=_gen(device, seed, STREAM_KEY_COEF, chunk),
                            device=device) * math.sqrt(coef_var)
            for r in range(rank):
                kf = kf + a[:, r:r + 1] * u[r]
        out[c0:c1] = kf.to(torch.bfloat16)
    return out


def keys_local(L, d, rank, seed, device="cpu", coef_var=0.5, rho_k=0.98, jump=1.0 / 256,
               segment=1024, noise=(0.25, 1.5), out=None):
    """Keys [L, d] bf16 with local structure, for the key-chunk coarse stage
    (whose premise is that neighbouring keys are often alike, with a spread
    that varies along the sequence):

      k_s = sigma_{s // segment} z_s / sqrt(d) + sum_r (a_{s,r} + o_{s,r}) u_r

    z_s ~ N(0, I_d); u_r ~ N(0, I_d) / sqrt(d) shared; a_{.,r} an AR(1) process
    along s with coefficient rho_k and stationary variance coef_var / 2;
    o_{.,r} piecewise constant, a fresh N(0, coef_var / 2) value at every jump
    (each position starts a new piece with probability `jump`); sigma drawn
    per segment of `segment` keys from U(noise)."""
    device = torch.device(device)
    if out is None:
        out = torch.empty((L, d), dtype=torch.bfloat16, device=device)
    u = torch.randn((max(rank, 1), d), generator=_gen(device, seed, STREAM_KEY_DIRS, 0),
                    device=device) / math.sqrt(d)
    half = math.sqrt(coef_var / 2)
    carry = None
    last_off = None
    for c0 in range(0, L, KEY_CHUNK):
        c1 = min(L, c0 + KEY_CHUNK)
        n = c1 - c0
        chunk = c0 // KEY_CHUNK
        z = torch.randn((n, d), generator=_gen(device, seed, STREAM_KEY_NOISE, chunk), device=device)
        nseg = -(-n // segment)
        sig = torch.rand((nseg, 1), generator=_gen(device, seed, STREAM_LOCAL_SCALE, chunk),
                         device=device) * (noise[1] - noise[0]) + noise[0]
        kf = z / math.sqrt(d) * sig.repeat_interleave(segment, dim=0)[:n]
        if rank > 0:
            eps = torch.randn((n, rank), generator=_gen(device, seed, STREAM_LOCAL_COEF, chunk),
                              device=device)
            if carry is None:  # stationary start
                eps[0] = eps[0] / math.sqrt(1 - rho_k * rho_k)
            a = _ar1_chunk(eps * math.sqrt(1 - rho_k * rho_k), rho_k, carry) * half
            carry = a[-1] / half
            jumps = torch.rand((n,), generator=_gen(device, seed, STREAM_LOCAL_JUMP, chunk),
                               device=device) < jump
            vals = torch.randn((n, rank), generator=_gen(device, seed, STREAM_LOCAL_OFFSET, chunk),
                               device=device) * half
            if last_off is None:
                jumps[0] = True
            piece = torch.cumsum(jumps.long(), 0) - 1  # index of the piece's first position
            starts = torch.nonzero(jumps).flatten()
            off = vals[starts][piece.clamp(min=0)] if starts.numel() else None
            if last_off is not None:
                # positions before the chunk's first jump continue the last piece
                before = piece < 0
                if off is None:
                    off = last_off[None, :].expand(n, rank).clone()
                else:
                    off[before] = last_off
            last_off = off[-1].clone()
            coef = a + off
            for r in range(rank):
                kf = kf + coef[:, r:r + 1] * u[r]
        out[c0:c1] = kf.to(torch.bfloat16)
    return out


def _ar1_chunk(eps, rho, carry):
    """x_t = sum_{tau<=t} rho^(t-tau) eps_tau + rho^(t+1) carry, by doubling."""
    x = eps
    n = x.shape[0]
    s = 1
    while s < n:
        y = x.clone()
        y[s:] += (rho ** s) * x[:-s]
        x = y
        s *= 2
    if carry is not None:
        p = torch.arange(1, n + 1, device=x.device, dtype=torch.float64)
        f = torch.pow(torch.tensor(rho, dtype=torch.float64, device=x.device), p)
        x = x + f.to(torch.float32)[:, None] * carry[None, :]
    return x


def queries(L, H, d, rho, seed, device="cpu", out=None, start=None):
    """Queries [L, H, d] bf16 following the AR(1) recipe.

    ``start`` (fp32 [H*d]) replaces q_{-1} = 0 as the state before row 0.
    """
    device = torch.device(device)
    if out is None:
        out = torch.empty((L, H, d), dtype=torch.bfloat16, device=device)
    carry = start
    for c0 in range(0, L, QUERY_CHUNK):
        c1 = min(L, c0 + QUERY_CHUNK)
        eps = torch.randn((c1 - c0, H * d),
                          generator=_gen(device, seed, STREAM_QUERY, c0 // QUERY_CHUNK),
                          device=device)
        x = _ar1_chunk(eps, rho, carry)
        carry = x[-1].clone()
        out[c0:c1] = x.view(c1 - c0, H, d).to(torch.bfloat16)
    return out


def weights(L, H, seed, device="cpu", out=None):
    """Head weights [L, H] fp32, U(0, 1) / H."""
    device = torch.device(device)
    if out is None:
        out = torch.empty((L, H), dtype=torch.float32, device=device)
    for c0 in range(0, L, QUERY_CHUNK):
        c1 = min(L, c0 + QUERY_CHUNK)
        out[c0:c1] = torch.rand((c1 - c0, H),
                                generator=_gen(device, seed, STREAM_WEIGHT, c0 // QUERY_CHUNK),
                                device=device) / H
    return out


def signed_weights(L, H, seed, device="cpu", out=None):
    """Head weights [L, H] fp32 of either sign, U(-1, 1) / H. Nothing in the
    index score makes w non-negative; these exercise negative and cancelling
    scores."""
    device = torch.device(device)
    if out is None:
        out = torch.empty((L, H), dtype=torch.float32, device=device)
    for c0 in range(0, L, QUERY_CHUNK):
        c1 = min(L, c0 + QUERY_CHUNK)
        u = torch.rand((c1 - c0, H), generator=_gen(device, seed, STREAM_WEIGHT, c0 // QUERY_CHUNK),
                       device=device)
        out[c0:c1] = (2.0 * u - 1.0) / H
    return out


def prefill(L, H, d, rho, rank, seed, device="cpu", coef_var=0.5):
    """One prefill sequence: Q [1, L, H, d] bf16, W [1, L, H] fp32, K [1, L, d] bf16."""
    Q = queries(L, H, d, rho, seed, device)
    W = weights(L, H, seed, device)
    K = keys(L, d, rank, seed, device, coef_var)
    return Q[None], W[None], K[None]


def decode(B, L, g, H, d, rho, rank, seed, device="cpu", coef_var=0.5):
    """A decode step for B requests with L cached keys each.

    The g new queries of a request are its last g positions (their keys are
    already in the cache). They continue an AR(1) chain whose state before
    them is drawn from the stationary law N(0, 1 / (1 - rho^2)).
    Returns Q [B, g, H, d] bf16, W [B, g, H] fp32, K [B, L, d] bf16.
    """
    device = torch.device(device)
    Q = torch.empty((B, g, H, d), dtype=torch.bfloat16, device=device)
    W = torch.empty((B, g, H), dtype=torch.float32, device=device)
    K = torch.empty((B, L, d), dtype=torch.bfloat16, device=device)
    for b in range(B):
        sb = _sub_seed(seed, 1000 + b, 0)
        st = torch.randn((H * d,), generator=_gen(device, sb, STREAM_QUERY_START, 0),
                         device=device) / math.sqrt(1.0 - rho * rho)
        queries(g, H, d, rho, sb, device, out=Q[b], start=st)
        weights(g, H, sb, device, out=W[b])
        keys(L, d, rank, sb, device, coef_var, out=K[b])
    return Q, W, K


def to_u16(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a bf16 tensor's bit patterns (uint16)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bf16 tensor")
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_u16(a: np.ndarray, device="cpu") -> torch.Tensor:
    """bf16 tensor holding the given uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


@dataclass(frozen=True)
class Workload:
    """A named workload: shapes, generator settings and indexer parameters."""
    name: str
    L: int
    H: int
    d: int
    rho: float
    rank: int
    k: int
    g: int = 1
    c: int = 0
    batch: int = 1
    decode: bool = False
    seed: int = 0
    variants: tuple = field(default=("dense",))


WORKLOADS = {
    "tiny": Workload("tiny", L=2048, H=4, d=32, rho=0.9, rank=2, k=64, g=4, c=128,
                     variants=("dense", "reuse", "refine")),
    "dense16k": Workload("dense16k", L=16384, H=64, d=128, rho=0.95, rank=4, k=2048),
    "pivot128k": Workload("pivot128k", L=131072, H=64, d=128, rho=0.95, rank=4, k=2048,
                          g=4, c=4096, variants=("dense", "reuse", "refine")),
    "decode64k": Workload("decode64k", L=65536, H=64, d=128, rho=0.95, rank=4, k=2048,
                          g=2, c=4096, batch=32, decode=True,
                          variants=("dense", "refine")),
    "pivot1m": Workload("pivot1m", L=1048576, H=64, d=128, rho=0.97, rank=4, k=2048,
                        g=16, c=8192, variants=("dense", "reuse", "refine")),
}


def make(w: Workload, device="cpu", seed=None):
    """Inputs (Q, W, K) for a workload on ``device``."""
    s = w.seed if seed is None else seed
    if w.decode:
        return decode(w.batch, w.L, w.g, w.H, w.d, w.rho, w.rank, s, device)
    return prefill(w.L, w.H, w.d, w.rho, w.rank, s, device)
