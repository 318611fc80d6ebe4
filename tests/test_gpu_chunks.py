"""Key-chunk coarse stage on the GPU against the oracle: chunk partitions (fixed
and score-adaptive, bit for bit), mean-key summaries (bit for bit), the
selected chunks (the parity rule of ``checker`` over the complete chunks'
summary scores), the candidate lists (exactly the expansion of the selected
chunks plus the tail), and Refine (the oracle re-scoring the GPU's own
candidates). Both kernel families (many groups: scan kernels; few rows:
split-key kernels), ragged lengths, groups with no complete chunk, and the
full budget, where the result must equal the dense indexer bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_dense_amd as dsa
import synth
from checker import Result, check_row
from parity import assert_ok

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def uneven_keys(B, L, d, block, seed):
    """Keys around a base vector that changes at random half-block boundaries
    (long runs make merges cheap, a change inside a block makes its split
    pay), with a spread that varies from block to block, bf16 [B, L, d]."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    half = max(block // 2, 1)
    nh = -(-L // half)
    seg = torch.cumsum((torch.rand((B, nh), generator=g) < 0.3).long(), dim=1)
    base = torch.randn((B, nh + 1, d), generator=g)
    base = torch.gather(base, 1, seg[:, :, None].expand(B, nh, d))
    base = base.repeat_interleave(half, dim=1)[:, :L]
    nb = -(-L // block)
    scale = (torch.rand((B, nb, 1), generator=g) * 0.45 + 0.05).repeat_interleave(block, dim=1)[:, :L]
    K = base + torch.randn((B, L, d), generator=g) * scale
    return K.to(torch.bfloat16).to(DEV).contiguous()


@pytest.mark.parametrize("L,block", [(4096, 64), (1000, 64), (77, 16), (5, 8)])
def test_fixed_chunks(L, block):
    cend = dsa.chunks_fixed(3, L, block, DEV).cpu().numpy()
    want = oracle.fixed_chunks(L, block)
    for b in range(3):
        assert np.array_equal(cend[b], want)


@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("L,block", [(4096, 64), (1001, 64), (300, 7)])
def test_chunk_means_bitexact(d, L, block):
    K = uneven_keys(2, L, d, block, seed=L + d)
    cend = dsa.chunks_fixed(2, L, block, DEV)
    Kbar = dsa.chunk_means(K, cend)
    torch.cuda.synchronize()
    for b in range(2):
        want = oracle.chunk_means(synth.to_u16(K[b]), cend[b].cpu().numpy())
        assert np.array_equal(synth.to_u16(Kbar[b]), want), b


def test_chunk_means_refresh_leaves_earlier_rows():
    L, d, block = 1000, 128, 64
    K = uneven_keys(1, L, d, block, seed=5)
    cend = dsa.chunks_fixed(1, L, block, DEV)
    nc = cend.shape[1]
    Kbar = torch.full((1, nc, d), 7.0, dtype=torch.bfloat16, device=DEV)
    dsa.chunk_means(K, cend, first=nc - 3, out=Kbar)
    torch.cuda.synchronize()
    want = oracle.chunk_means(synth.to_u16(K[0]), cend[0].cpu().numpy())
    got = synth.to_u16(Kbar[0])
    assert np.array_equal(got[nc - 3:], want[nc - 3:])
    assert np.all(Kbar[0, :nc - 3].float().cpu().numpy() == 7.0)


@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("L,block", [(4096, 64), (4000, 64), (1024, 8), (130, 16), (300000, 64), (65537, 8)])
def test_adaptive_chunks_bitexact(d, L, block):
    B = 2
    K = uneven_keys(B, L, d, block, seed=3 * L + d)
    cend = dsa.chunks_adaptive(K, block).cpu().numpy()
    moved = 0
    for b in range(B):
        want = oracle.adaptive_chunks(synth.to_u16(K[b]), block)
        assert np.array_equal(cend[b], want), (b, np.nonzero(cend[b] != want)[0][:5])
        moved += int(np.sum(np.diff(np.concatenate([[0], want])) != block))
    if L >= 1024:
        assert moved > 0  # the input makes some splits and merges worthwhile


def test_adaptive_chunks_constant_keys_stay_fixed():
    K = torch.full((1, 512, 32), 0.5, dtype=torch.bfloat16, device=DEV)
    cend = dsa.chunks_adaptive(K, 16).cpu().numpy()
    assert np.array_equal(cend[0], oracle.fixed_chunks(512, 16))


def check_chunk_refine(Q, W, K, Kbar, cend, g, nsel, max_chunk, k, out, groups=None, kind="mean", window=0):
    """Selected chunks, candidate lists and Refine rows of the groups checked."""
    idx, sc, ch, cand = [x.cpu().numpy() for x in out]
    B, q_len = Q.shape[:2]
    L = K.shape[1]
    G = -(-q_len // g)
    cw = (nsel + 1) * max_chunk
    res_s, res_c, res_r = Result(), Result(), Result()
    cend_h = cend.cpu().numpy()
    kbar_h = [synth.to_u16(Kbar[b]) for b in range(B)]
    keys_h = [synth.to_u16(K[b]) for b in range(B)]
    groups = groups if groups is not None else [(b, m) for b in range(B) for m in range(G)]
    for b, m in groups:
        r0, r1 = m * g, min(m * g + g, q_len)
        t_last = L - q_len + r1 - 1
        ce = cend_h[b]
        ncomp = int(np.sum(ce <= t_last + 1))
        Qm, Wm = synth.to_u16(Q[b, r0:r1]), W[b, r0:r1].cpu().numpy()
        qb, wb = oracle.proxy(Qm, Wm, g, 0, kind=kind, window=window)
        if ncomp:
            ref, mass = oracle.scores(qb, wb, kbar_h[b], n=ncomp)
            check_row(ch[b, m], None, np.arange(ncomp), ref, mass, nsel, res_s, f"chunks b{b} m{m}")
        elif np.any(ch[b, m] != -1):
            res_s.add(False, False, 0.0, f"chunks b{b} m{m}: no complete chunk, row not -1")
        # the list: exactly the GPU's selected chunks expanded, then the tail
        sel = ch[b, m][ch[b, m] >= 0]
        starts = np.concatenate([[0], ce[:-1]])
        want = [s for c in sel for s in range(starts[c], ce[c])]
        want += list(range(int(ce[ncomp - 1]) if ncomp else 0, t_last + 1))
        want = np.array(want + [-1] * (cw - len(want)), np.int64)
        res_c.add(bool(np.array_equal(cand[b, m], want)), True, 0.0, f"cand b{b} m{m}")
        for r in range(r0, r1):
            pos = L - q_len + r
            cm = cand[b, m]
            cp = cm[(cm >= 0) & (cm <= pos)]
            ref_i, mass_i = oracle.scores(Qm[r - r0], Wm[r - r0], np.ascontiguousarray(keys_h[b][cp]))
            check_row(idx[b, r], sc[b, r], cp, ref_i, mass_i, k, res_r, f"refine b{b} r{r}")
    return res_s, res_c, res_r


def run_chunk(Q, W, K, block, g, nsel, k, adaptive=False, kind="mean", window=0):
    B, L = K.shape[:2]
    cend = dsa.chunks_adaptive(K, block) if adaptive else dsa.chunks_fixed(B, L, block, DEV)
    Kbar = dsa.chunk_means(K, cend)
    max_chunk = 2 * block if adaptive else block
    out = dsa.chunk_refine(Q, W, K, Kbar, cend, g, nsel, max_chunk, k, proxy=kind, window=window,
                           chunks=True, cand=True)
    torch.cuda.synchronize()
    return cend, Kbar, max_chunk, out


# (B, L, q_len, H, d, block, g, nsel, k): scan kernels, then split-key kernels
SCAN_CASES = [
    (1, 2048, 2048, 4, 32, 64, 1, 4, 64),
    (1, 2048, 2048, 4, 32, 16, 4, 6, 64),
    (2, 1500, 1500, 4, 32, 32, 3, 5, 48),
    (1, 3000, 700, 4, 32, 64, 4, 3, 64),
]
SPLIT_CASES = [
    (3, 5000, 2, 4, 32, 64, 2, 8, 128),
    (2, 4099, 3, 4, 32, 32, 1, 5, 64),
    (1, 9000, 64, 4, 32, 64, 4, 4, 96),
]


@pytest.mark.parametrize("case", SCAN_CASES + SPLIT_CASES,
                         ids=[f"scan{i}" for i in range(len(SCAN_CASES))] +
                             [f"split{i}" for i in range(len(SPLIT_CASES))])
@pytest.mark.parametrize("adaptive", [False, True], ids=["fixed", "adaptive"])
def test_chunk_refine(case, adaptive):
    B, L, q_len, H, d, block, g, nsel, k = case
    if q_len == L:
        Q, W, _ = synth.prefill(L, H, d, 0.9, 2, 11, DEV)
        Q, W = Q.expand(B, -1, -1, -1).contiguous(), W.expand(B, -1, -1).contiguous()
    else:
        Q, W, _ = synth.decode(B, L, q_len, H, d, 0.9, 2, 11, DEV)
    K = uneven_keys(B, L, d, block, seed=L + block)
    cend, Kbar, mc, out = run_chunk(Q, W, K, block, g, nsel, k, adaptive=adaptive)
    G = -(-q_len // g)
    groups = [(b, m) for b in range(B) for m in range(G)]
    if len(groups) > 160:  # first groups (no complete chunk), last groups, a sample between
        rng = np.random.default_rng(B * L + q_len)
        pick = rng.choice(len(groups), 96, replace=False).tolist()
        keep = set(range(24)) | set(range(len(groups) - 24, len(groups))) | set(pick)
        groups = [groups[i] for i in sorted(keep)]
    rs, rc, rr = check_chunk_refine(Q, W, K, Kbar, cend, g, nsel, mc, k, out, groups)
    assert_ok(rs, rc, rr)
    assert rr.rows > 0


def test_chunk_refine_h64():
    L, block, g, nsel, k = 8192, 64, 4, 16, 256
    Q, W, K = synth.prefill(L, 64, 128, 0.95, 4, 21, DEV)
    cend, Kbar, mc, out = run_chunk(Q, W, K, block, g, nsel, k)
    G = L // g
    groups = [(0, m) for m in (0, 1, 15, 16, 17, 100, 511, 1024, 1500, 2000, G - 2, G - 1)]
    assert_ok(*check_chunk_refine(Q, W, K, Kbar, cend, g, nsel, mc, k, out, groups))


def test_chunk_refine_matches_oracle_end_to_end():
    """Where no near-ties sit at a selection boundary, the GPU's chunks,
    candidates and Refine rows are the oracle's exactly."""
    L, H, d, block, g, nsel, k = 1024, 4, 32, 32, 2, 6, 32
    Q, W, _ = synth.prefill(L, H, d, 0.9, 2, 13, DEV)
    K = uneven_keys(1, L, d, block, seed=99)
    cend, Kbar, mc, out = run_chunk(Q, W, K, block, g, nsel, k)
    idx, _, ch, cand = [x.cpu().numpy() for x in out]
    G = L // g
    o = oracle.chunk_groups(synth.to_u16(Q[0]), W[0].cpu().numpy(), synth.to_u16(K[0]), g,
                            cend[0].cpu().numpy(), nsel, (nsel + 1) * mc, k, list(range(G)))
    same_ch = np.mean([np.array_equal(ch[0, m], o["chunks"][m]) for m in range(G)])
    same_cand = np.mean([np.array_equal(cand[0, m], o["cand"][m]) for m in range(G)])
    same_ref = np.mean([np.array_equal(np.sort(idx[0, m * g + i]), np.sort(o["refine"][m, i]))
                        for m in range(G) for i in range(g)])
    assert same_ch > 0.98 and same_cand > 0.98 and same_ref > 0.98, (same_ch, same_cand, same_ref)


@pytest.mark.parametrize("q_len,g", [(2048, 1), (2048, 4), (3, 3)])
def test_full_budget_is_dense(q_len, g):
    """Keeping every chunk makes each list the whole prefix: Refine equals the
    dense indexer bit for bit."""
    L, H, d, block, k = 2048, 4, 32, 64, 64
    if q_len == L:
        Q, W, K = synth.prefill(L, H, d, 0.9, 2, 17, DEV)
    else:
        Q, W, K = synth.decode(1, L, q_len, H, d, 0.9, 2, 17, DEV)
    nc = L // block
    cend, Kbar, mc, out = run_chunk(Q, W, K, block, g, nc, k)
    di, ds = dsa.dense(Q, W, K, k)
    assert torch.equal(out[0], di) and torch.equal(out[1], ds)


@pytest.mark.parametrize("kind,window", [("first", 0), ("last", 0), ("mean", 2)])
def test_chunk_refine_proxy_strategies(kind, window):
    L, H, d, block, g, nsel, k = 2048, 4, 32, 32, 4, 6, 64
    Q, W, _ = synth.prefill(L, H, d, 0.9, 2, 19, DEV)
    K = uneven_keys(1, L, d, block, seed=7)
    cend, Kbar, mc, out = run_chunk(Q, W, K, block, g, nsel, k, kind=kind, window=window)
    groups = [(0, m) for m in range(0, L // g, 7)]
    assert_ok(*check_chunk_refine(Q, W, K, Kbar, cend, g, nsel, mc, k, out, groups, kind=kind, window=window))
