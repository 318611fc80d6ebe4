"""Pins for the CPU oracle: checks against things the oracle's own code cannot
produce by itself (hand-worked values, closed forms, identities of the ReLU,
library routines, and invariants the PIVOT paper states).

Every function takes the loaded oracle library, so the same battery runs on the
real oracle (tests/test_oracle_pins.py) and on deliberately broken copies of it
(tests/test_oracle_mutants.py), where at least one pin must fail.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.txt")


# ----------------------------------------------------------------- helpers
def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of float values rounded to bf16 (torch RNE)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f64(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_inputs(rng, L, H, d, q_len=None, neg_w=False):
    """Small random bf16 inputs (Q [q_len,H,d], W [q_len,H], K [L,d])."""
    q_len = L if q_len is None else q_len
    Q = bf16_bits(rng.standard_normal((q_len, H, d)))
    K = bf16_bits(rng.standard_normal((L, d)) * 0.5)
    W = rng.uniform(-1 if neg_w else 0, 1, (q_len, H)).astype(np.float32)
    return Q, W, K


def parse_golden(path=GOLDEN):
    g = dict(K={}, Q={}, W={}, I={}, MASS={}, TOPK=[], PROXYQ={}, PROXYW={}, SCAN={}, CAND={},
             REUSE={}, REFINE={}, ROUND=[], PIVOT=None)
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if ":" in line:
                head, vals = line.split(":", 1)
            else:
                head, vals = line, ""
            h = head.split()
            tag, keys = h[0], h[1:]
            if tag == "ROUND":
                g[tag].append(([int(x, 16) for x in keys], int(vals.strip(), 16)))
                continue
            v = [float(x) for x in vals.split()]
            if tag == "PIVOT":
                g[tag] = tuple(int(x) for x in keys)
            elif tag == "TOPK":
                g[tag].append((int(keys[0]), int(keys[1]), [int(x) for x in v]))
            elif tag in ("Q", "REFINE"):
                g[tag][(int(keys[0]), int(keys[1]))] = v
            else:
                g[tag][int(keys[0])] = v
    L = len(g["K"])
    H = len(g["W"][0])
    d = len(g["K"][0])
    K = np.array([g["K"][s] for s in range(L)], np.float32)
    Q = np.array([[g["Q"][(t, j)] for j in range(H)] for t in range(L)], np.float32)
    W = np.array([g["W"][t] for t in range(L)], np.float32)
    g["arrays"] = (bf16_bits(Q), W, bf16_bits(K))
    g["shape"] = (L, H, d)
    return g


# ------------------------------------------------------------------- pins
def pin_golden_scores(lib):
    g = parse_golden()
    Q, W, K = g["arrays"]
    L, H, d = g["shape"]
    for t in range(L):
        sc, ms = oracle.scores(Q[t], W[t], K, n=t + 1, lib=lib)
        assert np.array_equal(sc, np.array(g["I"][t])), (t, sc, g["I"][t])
        assert np.array_equal(ms, np.array(g["MASS"][t])), (t, ms, g["MASS"][t])


def pin_golden_topk(lib):
    g = parse_golden()
    Q, W, K = g["arrays"]
    for t, k, want in g["TOPK"]:
        got, _ = oracle.dense_rows(Q, W, K, k, [t], lib=lib)
        assert got[0].tolist() == want, (t, k, got[0].tolist(), want)


def pin_golden_pivot(lib):
    g = parse_golden()
    Q, W, K = g["arrays"]
    L, H, d = g["shape"]
    gs, c, k = g["PIVOT"]
    ng = (L + gs - 1) // gs
    for m in range(ng):
        qb, wb = oracle.proxy(Q, W, gs, m, lib=lib)
        assert np.array_equal(bits_to_f64(qb).ravel(), np.array(g["PROXYQ"][m])), m
        assert np.array_equal(wb.astype(np.float64), np.array(g["PROXYW"][m])), m
    out = oracle.pivot_groups(Q, W, K, gs, c, k, list(range(ng)), lib=lib)
    for m in range(ng):
        want_c = [int(x) for x in g["CAND"][m]]
        assert out["cand"][m].tolist() == want_c, (m, out["cand"][m])
        assert out["reuse"][m].tolist() == [int(x) for x in g["REUSE"][m]], m
        n = len(g["SCAN"][m])
        sc = np.array(g["SCAN"][m])
        for x, s in enumerate(want_c):
            if s >= 0:
                assert out["cand_score"][m][x] == sc[s]
        for i in range(gs):
            want = [int(x) for x in g["REFINE"][(m, i)]]
            assert out["refine"][m][i].tolist() == want, (m, i, out["refine"][m][i])
        assert n == min(L, (m + 1) * gs)


def pin_golden_proxy_rounding(lib):
    g = parse_golden()
    for members, want in g["ROUND"]:
        n = len(members)
        Q = np.array(members, np.uint16).reshape(n, 1, 1)
        W = np.ones((n, 1), np.float32)
        qb, wb = oracle.proxy(Q, W, n, 0, lib=lib)
        assert int(qb[0, 0]) == want, (members, hex(int(qb[0, 0])), hex(want))
        assert wb[0] == 1.0


def pin_relu_identities(lib):
    """relu(x) - relu(-x) = x and relu(x) + relu(-x) = |x|, per head.

    With q -> -q every per-head dot product flips sign exactly, so
    I(q) - I(-q) = sum_j w_j (q_j . k) and I(q) + I(-q) = sum_j w_j |q_j . k|,
    which numpy's float64 matmul computes independently of the oracle.
    """
    rng = np.random.default_rng(11)
    H, d, L = 5, 12, 40
    Q, W, K = rand_inputs(rng, L, H, d, neg_w=True)
    Kf = bits_to_f64(K)
    for t in (0, 7, 39):
        q = Q[t]
        qn = q ^ np.uint16(0x8000)
        a, ma = oracle.scores(q, W[t], K, lib=lib)
        b, _ = oracle.scores(qn, W[t], K, lib=lib)
        dots = Kf @ bits_to_f64(q).T  # [L, H]
        w = W[t].astype(np.float64)
        lin = dots @ w
        ab = np.abs(dots) @ np.abs(w)
        tol = 1e-12 * (ab + 1e-300)
        assert np.all(np.abs((a - b) - lin) <= tol)
        assert np.all(np.abs((a + b) - np.abs(dots) @ w) <= tol)
        assert np.all(ma + 1e-12 * ma >= ab * (1 - 1e-12))


def pin_exact_dyadic(lib):
    """Signed dyadic inputs: q and k are multiples of 1/2 in [-2, 2], w multiples
    of 1/4 in [-1, 1]. Every product and partial sum is then exact in fp64, in
    any order, so numpy's float64 products give the exact score
    I = max(0, K q^T) w and the exact tolerance mass A = (|K| |q|^T) |w|, and the
    oracle must equal both bit for bit (negative and zero weights included)."""
    rng = np.random.default_rng(19)
    H, d, L = 5, 12, 40
    for t in range(3):
        q = bf16_bits(rng.integers(-4, 5, (H, d)) * 0.5)
        K = bf16_bits(rng.integers(-4, 5, (L, d)) * 0.5)
        w = (rng.integers(-4, 5, H) * 0.25).astype(np.float32)
        w[t] = 0.0
        qf, Kf = bits_to_f64(q), bits_to_f64(K)
        sc, ms = oracle.scores(q, w, K, lib=lib)
        dots = Kf @ qf.T  # [L, H], exact
        want = np.maximum(dots, 0.0) @ w.astype(np.float64)
        mass = (np.abs(Kf) @ np.abs(qf).T) @ np.abs(w.astype(np.float64))
        assert np.array_equal(sc, want), (t, sc - want)
        assert np.array_equal(ms, mass), (t, ms - mass)
        assert np.any(sc < 0) and np.any(sc == 0)


def pin_homogeneity_and_heads(lib):
    """I is linear in w, positively homogeneous in q, invariant under a joint
    permutation of the heads, and the score of key s depends on k_s only."""
    rng = np.random.default_rng(12)
    H, d, L = 6, 8, 30
    Q, W, K = rand_inputs(rng, L, H, d)
    q, w = Q[L - 1], W[L - 1]
    base, _ = oracle.scores(q, w, K, lib=lib)
    two_w, _ = oracle.scores(q, (2 * w).astype(np.float32), K, lib=lib)
    assert np.array_equal(two_w, 2 * base)
    q2 = bf16_bits(bits_to_f64(q) * 2.0)
    two_q, _ = oracle.scores(q2, w, K, lib=lib)
    assert np.array_equal(two_q, 2 * base)
    perm = rng.permutation(H)
    pq, _ = oracle.scores(np.ascontiguousarray(q[perm]), np.ascontiguousarray(w[perm]), K, lib=lib)
    assert np.allclose(pq, base, rtol=1e-13, atol=0)
    # changing other keys does not change key 3's score
    K2 = K.copy()
    K2[[0, 1, 2, 4, 5]] = bf16_bits(rng.standard_normal((5, d)))
    other, _ = oracle.scores(q, w, K2, lib=lib)
    assert other[3] == base[3]
    # heads with zero weight do not contribute; an all-zero query scores 0
    wz = w.copy()
    wz[1:] = 0
    single, _ = oracle.scores(q, wz, K, lib=lib)
    dots0 = bits_to_f64(K) @ bits_to_f64(q[0])
    bound = 1e-13 * float(w[0]) * (np.abs(bits_to_f64(K)) @ np.abs(bits_to_f64(q[0])))
    assert np.all(np.abs(single - float(w[0]) * np.maximum(dots0, 0)) <= bound)
    zero, _ = oracle.scores(np.zeros_like(q), w, K, lib=lib)
    assert np.all(zero == 0)


def pin_one_hot(lib):
    """One-hot queries and keys: I(s) = sum_j w_j [a_j == b_s] max(0, alpha_j beta_s)."""
    H, d, L = 4, 6, 6
    a = [0, 2, 2, 5]
    alpha = [1.0, -2.0, 0.5, 3.0]
    b = [2, 0, 5, 1, 2, 5]
    beta = [1.0, 4.0, -1.0, 2.0, -0.25, 0.5]
    w = np.array([0.5, 0.25, 1.0, 2.0], np.float32)
    q = np.zeros((H, d), np.float32)
    for j in range(H):
        q[j, a[j]] = alpha[j]
    K = np.zeros((L, d), np.float32)
    for s in range(L):
        K[s, b[s]] = beta[s]
    sc, _ = oracle.scores(bf16_bits(q), w, bf16_bits(K), lib=lib)
    # s0 (dim2, 1.0): heads 1 (-2) and 2 (0.5) -> 1.0*0.5 = 0.5
    # s1 (dim0, 4.0): head 0 (1) -> 0.5*4 = 2
    # s2 (dim5, -1.0): head 3 (3) -> relu(-3) = 0
    # s3 (dim1): no head -> 0
    # s4 (dim2, -0.25): head 1 (-2) -> 0.5*0.25 = 0.125 ; head 2 -> 0
    # s5 (dim5, 0.5): head 3 (3) -> 2*1.5 = 3
    assert sc.tolist() == [0.5, 2.0, 0.0, 0.0, 0.125, 3.0]


def pin_select_vs_lexsort(lib):
    """Selection equals numpy's lexsort under (score desc, index asc)."""
    rng = np.random.default_rng(13)
    for n, k in ((50, 7), (200, 200), (10, 25), (1, 1), (300, 64)):
        sc = rng.integers(0, 6, n).astype(np.float64) * 0.5  # many ties
        got, gs = oracle.select(sc, k, lib=lib)
        order = np.lexsort((np.arange(n), -sc))
        m = min(n, k)
        assert got[:m].tolist() == order[:m].tolist()
        assert np.all(got[m:] == -1) and np.all(np.isneginf(gs[m:]))
        assert np.array_equal(gs[:m], sc[order[:m]])
        # explicit index lists are honoured
        idx = rng.permutation(10 * n)[:n]
        got2, _ = oracle.select(sc, k, idx=idx, lib=lib)
        order2 = np.lexsort((idx, -sc))
        assert got2[:m].tolist() == idx[order2[:m]].tolist()
    got, _ = oracle.select(np.zeros(40), 16, lib=lib)
    assert got.tolist() == list(range(16))


def pin_dense_causal(lib):
    """Row r (position L - q_len + r) is scored against exactly keys 0..pos;
    with k >= pos + 1 the whole prefix comes back."""
    rng = np.random.default_rng(14)
    L, H, d = 24, 3, 8
    for q_len in (L, 5):
        Q, W, K = rand_inputs(rng, L, H, d, q_len=q_len)
        rows = list(range(q_len))
        got, gs = oracle.dense_rows(Q, W, K, L + 3, rows, lib=lib)
        for r in rows:
            pos = L - q_len + r
            sel = got[r][got[r] >= 0]
            assert sorted(sel.tolist()) == list(range(pos + 1)), (q_len, r)
            assert np.all(np.diff(gs[r][: pos + 1]) <= 0)
        # an all-zero query ties every key: the selection is the lowest indices
        Qz = np.zeros_like(Q)
        gz, _ = oracle.dense_rows(Qz, W, K, 4, [q_len - 1], lib=lib)
        assert gz[0].tolist() == [0, 1, 2, 3]


def pin_pivot_invariants(lib):
    """Invariants PIVOT states or implies:
    g = 1: Reuse and Refine equal the dense indexer;
    c >= L: Refine equals the dense indexer;
    R_m is the top-k prefix of C_m; T_i lies in C_m restricted to [0, pos(i)];
    |union_i T_i| <= min(g k, c) (the g*k bound of observation O2);
    T_i cap D_i = C'_i cap D_i (Refine misses exactly the dense keys that the
    candidates miss)."""
    rng = np.random.default_rng(15)
    L, H, d, k = 48, 3, 8, 5
    Q, W, K = rand_inputs(rng, L, H, d)
    dense, _ = oracle.dense_rows(Q, W, K, k, list(range(L)), lib=lib)
    # g = 1
    o1 = oracle.pivot_groups(Q, W, K, 1, 9, k, list(range(L)), lib=lib)
    assert np.array_equal(o1["reuse"], dense)
    assert np.array_equal(o1["refine"][:, 0, :], dense)
    # c >= L
    for g in (3, 4, 7):
        ng = (L + g - 1) // g
        o = oracle.pivot_groups(Q, W, K, g, L, k, list(range(ng)), lib=lib)
        for m in range(ng):
            for i in range(g):
                r = m * g + i
                if r < L:
                    assert np.array_equal(o["refine"][m, i], dense[r]), (g, m, i)
                else:
                    assert np.all(o["refine"][m, i] == -1)
    # structure with a candidate budget below the prefix
    g, c = 4, 8
    ng = L // g
    o = oracle.pivot_groups(Q, W, K, g, c, k, list(range(ng)), lib=lib)
    for m in range(ng):
        cand = o["cand"][m]
        assert np.array_equal(o["reuse"][m], cand[:k])
        union = set()
        for i in range(g):
            r = m * g + i
            T = set(o["refine"][m, i][o["refine"][m, i] >= 0].tolist())
            Cp = {s for s in cand.tolist() if 0 <= s <= r}
            assert T <= Cp
            assert len(T) == min(k, len(Cp))
            D = set(dense[r][dense[r] >= 0].tolist())
            assert T & D == Cp & D
            union |= T
        assert len(union) <= min(g * k, c)


def pin_candidate_injection(lib):
    rng = np.random.default_rng(16)
    L, H, d, g, c, k = 32, 2, 8, 4, 6, 3
    Q, W, K = rand_inputs(rng, L, H, d)
    ng = L // g
    o = oracle.pivot_groups(Q, W, K, g, c, k, list(range(ng)), lib=lib)
    o2 = oracle.pivot_groups(Q, W, K, g, c, k, list(range(ng)), cand_in=o["cand"], lib=lib)
    assert np.array_equal(o["refine"], o2["refine"])
    # group 0 ends at position 3: its list holds the 4 keys 0..3, then -1 -1;
    # group 2 ends at position 11 and holds c = 6 keys
    assert o["cand"][0].tolist()[4:] == [-1, -1] and np.all(o["cand"][2] >= 0)
    bad_lists = []
    bad = o["cand"].copy()
    bad[2, 1] = bad[2, 0]  # duplicate
    bad_lists.append(("a duplicated candidate", bad))
    bad = o["cand"].copy()
    bad[2, 3] = 12  # a key after the group's last position
    bad_lists.append(("a candidate after the group's last position", bad))
    bad = o["cand"].copy()
    bad[0, 2] = 4  # the same, in a group whose list is shorter than c
    bad_lists.append(("a future candidate in a short list", bad))
    bad = o["cand"].copy()
    bad[2, 5] = -1  # a list shorter than min(c, t_last + 1)
    bad_lists.append(("a short candidate list", bad))
    bad = o["cand"].copy()
    bad[0, 3] = -1  # the same where the prefix is shorter than c
    bad_lists.append(("a short list of a short prefix", bad))
    bad = o["cand"].copy()
    bad[0, 5] = 0  # a key in the -1 tail
    bad_lists.append(("a key in the -1 tail", bad))
    bad = o["cand"].copy()
    bad[0, 4] = -2  # a tail entry other than -1
    bad_lists.append(("a tail entry other than -1", bad))
    for what, bad in bad_lists:
        try:
            oracle.pivot_groups(Q, W, K, g, c, k, list(range(ng)), cand_in=bad, lib=lib)
        except ValueError:
            pass
        else:
            raise AssertionError(f"{what} was accepted")


def pin_short_last_group(lib):
    """The last group holds the remaining rows and averages over them only."""
    rng = np.random.default_rng(17)
    L, H, d, g = 10, 2, 4, 4
    Q, W, K = rand_inputs(rng, L, H, d)
    qb, wb = oracle.proxy(Q, W, g, 2, lib=lib)  # rows 8, 9
    mean = (bits_to_f64(Q[8]) + bits_to_f64(Q[9])) / 2  # exact for two bf16 values
    assert np.array_equal(bits_to_f64(qb), bits_to_f64(bf16_bits(mean)))
    assert np.array_equal(wb, ((W[8] + W[9]) / np.float32(2)).astype(np.float32))
    # one member: the proxy is that member
    qb1, wb1 = oracle.proxy(Q, W, 1, 5, lib=lib)
    assert np.array_equal(qb1, Q[5]) and np.array_equal(wb1, W[5])
    # identical members: the proxy is the member
    Qs = np.repeat(Q[3:4], 3, axis=0)
    Ws = np.repeat(W[3:4], 3, axis=0)
    qb3, wb3 = oracle.proxy(Qs, Ws, 3, 0, lib=lib)
    assert np.array_equal(qb3, Q[3])
    o = oracle.pivot_groups(Q, W, K, g, 5, 3, [2], lib=lib)
    # the short group's scan runs to its own last position, 9
    assert np.all(o["cand"][0] <= 9) and np.all(o["cand"][0] >= 0)
    assert np.all(o["refine"][0, 2:] == -1)


def pin_proxy_strategies(lib):
    """Endpoint proxies are the endpoint member exactly; a window of w members
    is the mean of the group's last w rows (the mean of two bf16 values is
    exact before rounding); a window as wide as the group is the group mean;
    with g = 1 every strategy is the row itself."""
    rng = np.random.default_rng(23)
    L, H, d, g = 12, 2, 4, 4
    Q, W, K = rand_inputs(rng, L, H, d)
    for m in (0, 1, 2):
        r0, r1 = m * g, min(m * g + g, L)
        qf, wf = oracle.proxy(Q, W, g, m, kind="first", lib=lib)
        assert np.array_equal(qf, Q[r0]) and np.array_equal(wf, W[r0])
        ql, wl = oracle.proxy(Q, W, g, m, kind="last", lib=lib)
        assert np.array_equal(ql, Q[r1 - 1]) and np.array_equal(wl, W[r1 - 1])
        q1, w1 = oracle.proxy(Q, W, g, m, kind="mean", window=1, lib=lib)
        assert np.array_equal(q1, Q[r1 - 1]) and np.array_equal(w1, W[r1 - 1])
        q2, w2 = oracle.proxy(Q, W, g, m, kind="mean", window=2, lib=lib)
        mean2 = (bits_to_f64(Q[r1 - 2]) + bits_to_f64(Q[r1 - 1])) / 2
        assert np.array_equal(bits_to_f64(q2), bits_to_f64(bf16_bits(mean2)))
        assert np.array_equal(w2, ((W[r1 - 2] + W[r1 - 1]) / np.float32(2)).astype(np.float32))
        qa, wa = oracle.proxy(Q, W, g, m, lib=lib)
        qw, ww = oracle.proxy(Q, W, g, m, kind="mean", window=g, lib=lib)
        assert np.array_equal(qa, qw) and np.array_equal(wa, ww)
    for kind in ("first", "last", "mean"):
        o1 = oracle.pivot_groups(Q, W, K, 1, 5, 3, [4], kind=kind, lib=lib)
        ref = oracle.dense_rows(Q, W, K, 3, [4], lib=lib)
        assert np.array_equal(o1["reuse"][0], ref[0][0])


# ------------------------------------------------------- key-chunk pins
CHUNK_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "chunk_example.txt")


def parse_chunk_golden(path=CHUNK_GOLDEN):
    g = dict(CK={}, CQ={}, CW={}, MEAN={}, SEL={}, CAND={}, REF={}, CEND=None)
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            head, vals = line.split(":", 1)
            h = head.split()
            tag, keys = h[0], tuple(int(x) for x in h[1:])
            v = [float(x) for x in vals.split()]
            if tag == "CEND":
                g[tag] = [int(x) for x in v]
            elif tag in ("CK", "CQ", "CW", "MEAN"):
                g[tag][keys[0]] = v
            else:
                g[tag][keys] = [int(x) for x in v]
    L = len(g["CK"])
    K = bf16_bits(np.array([g["CK"][s] for s in range(L)], np.float32))
    Q = bf16_bits(np.array([[g["CQ"][t]] for t in range(L)], np.float32))
    W = np.array([g["CW"][t] for t in range(L)], np.float32)
    g["arrays"] = (Q, W, K)
    return g


def chunk_dispersion(Kf):
    """Squared reconstruction error of a chunk by its mean (numpy, fp64)."""
    return float(((Kf - Kf.mean(axis=0)) ** 2).sum())


def pin_golden_chunks(lib):
    g = parse_chunk_golden()
    Q, W, K = g["arrays"]
    L = K.shape[0]
    cend = oracle.fixed_chunks(L, 2)
    assert cend.tolist() == g["CEND"]
    kb = oracle.chunk_means(K, cend, lib=lib)
    for b, want in g["MEAN"].items():
        assert bits_to_f64(kb[b]).tolist() == want, (b, bits_to_f64(kb[b]))
    cw, k = 8, 2
    for gs, nsel in ((1, 2), (1, 1), (2, 1)):
        ng = -(-L // gs)
        o = oracle.chunk_groups(Q, W, K, gs, cend, nsel, cw, k, list(range(ng)), lib=lib)
        for m in range(ng):
            assert o["chunks"][m].tolist() == g["SEL"][(gs, nsel, m)], (gs, nsel, m, o["chunks"][m])
            want = g["CAND"][(gs, nsel, m)]
            assert o["cand"][m].tolist() == want + [-1] * (cw - len(want)), (gs, nsel, m, o["cand"][m])
            for i in range(gs):
                r = m * gs + i
                if r < L:
                    assert o["refine"][m, i].tolist() == g["REF"][(gs, nsel, r)], (gs, nsel, r)


def pin_chunk_means_closed_forms(lib):
    """Chunks of equal keys average to that key; three keys x-u, x, x+u average
    to x (the fp32 sum 3x is exact); a short last chunk divides by its own
    size; one-key chunks are the keys."""
    rng = np.random.default_rng(31)
    d = 6
    base = bf16_bits(rng.standard_normal((4, d)))
    K = np.empty((11, d), np.uint16)
    K[0:4] = base[0]
    K[4:8] = base[1]
    x = bits_to_f64(bf16_bits(np.full(d, 1.5)))
    K[8:11] = bf16_bits(np.stack([x - 0.25, x, x + 0.25]))
    kb = oracle.chunk_means(K, oracle.fixed_chunks(11, 4), lib=lib)
    assert np.array_equal(kb[0], base[0]) and np.array_equal(kb[1], base[1])
    assert np.array_equal(bits_to_f64(kb[2]), x)
    Kr = bf16_bits(rng.standard_normal((9, d)))
    assert np.array_equal(oracle.chunk_means(Kr, oracle.fixed_chunks(9, 1), lib=lib), Kr)
    # uneven chunks [0,2) [2,3) [3,9): the middle one is its key
    kb2 = oracle.chunk_means(Kr, np.array([2, 3, 9], np.int32), lib=lib)
    assert np.array_equal(kb2[1], Kr[2])
    m01 = (bits_to_f64(Kr[0]) + bits_to_f64(Kr[1])) / 2  # exact for two bf16 values
    assert np.array_equal(bits_to_f64(kb2[0]), bits_to_f64(bf16_bits(m01)))


def pin_chunk_reductions(lib):
    """One key per chunk makes the coarse stage the token scan: with nsel = c
    the candidates are PIVOT's top-c set and Refine is PIVOT-Refine. A budget
    of every chunk makes the candidates the whole prefix: Refine is dense."""
    rng = np.random.default_rng(32)
    L, H, d, k = 40, 3, 8, 5
    Q, W, K = rand_inputs(rng, L, H, d)
    for g, c in ((1, 7), (4, 9)):
        ng = -(-L // g)
        o = oracle.chunk_groups(Q, W, K, g, oracle.fixed_chunks(L, 1), c, c, k, list(range(ng)), lib=lib)
        p = oracle.pivot_groups(Q, W, K, g, c, k, list(range(ng)), lib=lib)
        assert np.array_equal(o["refine"], p["refine"])
        for m in range(ng):
            assert sorted(o["cand"][m][o["cand"][m] >= 0].tolist()) == sorted(
                p["cand"][m][p["cand"][m] >= 0].tolist())
    dense, _ = oracle.dense_rows(Q, W, K, k, list(range(L)), lib=lib)
    for g, blk in ((1, 4), (3, 3), (5, 6)):
        cend = oracle.fixed_chunks(L, blk)
        ng = -(-L // g)
        o = oracle.chunk_groups(Q, W, K, g, cend, cend.size, L + blk, k, list(range(ng)), lib=lib)
        for m in range(ng):
            for i in range(g):
                r = m * g + i
                if r < L:
                    assert np.array_equal(o["refine"][m, i], dense[r]), (g, blk, r)
            t_last = min(m * g + g, L) - 1
            assert o["cand"][m].tolist() == list(range(t_last + 1)) + [-1] * (L + blk - t_last - 1)


def pin_chunk_selection(lib):
    """The selected chunks are the top-nsel complete chunks by the proxy's
    score of their summaries (lexsort), the list holds exactly their keys and
    the tail keys in ascending order, and Refine keeps the top-k of the
    member's own scores over the causal part of that list."""
    rng = np.random.default_rng(33)
    L, H, d, k, g, nsel, blk = 45, 2, 8, 4, 3, 3, 4
    Q, W, K = rand_inputs(rng, L, H, d)
    cend = np.array([3, 4, 8, 10, 16, 17, 20, 28, 30, 31, 36, 40, 45], np.int32)
    starts = np.concatenate([[0], cend[:-1]])
    kb = oracle.chunk_means(K, cend, lib=lib)
    ng = -(-L // g)
    cw = nsel * 8 + 8
    o = oracle.chunk_groups(Q, W, K, g, cend, nsel, cw, k, list(range(ng)), lib=lib)
    for m in range(ng):
        t_last = min(m * g + g, L) - 1
        ncomp = int(np.sum(cend <= t_last + 1))
        qb, wb = oracle.proxy(Q, W, g, m, lib=lib)
        sc, _ = oracle.scores(qb, wb, kb, n=ncomp, lib=lib)
        order = np.lexsort((np.arange(ncomp), -sc))
        want = sorted(order[:nsel].tolist())
        assert o["chunks"][m].tolist() == want + [-1] * (nsel - len(want)), m
        keys = [s for b in want for s in range(starts[b], cend[b])]
        tail0 = cend[ncomp - 1] if ncomp else 0
        keys += list(range(tail0, t_last + 1))
        assert o["cand"][m].tolist() == keys + [-1] * (cw - len(keys)), m
        for i in range(g):
            r = m * g + i
            if r >= L:
                assert np.all(o["refine"][m, i] == -1)
                continue
            mine = [s for s in keys if s <= r]
            ss = np.array([oracle.scores(Q[r], W[r], K[s:s + 1], lib=lib)[0][0] for s in mine])
            top = np.lexsort((np.array(mine), -ss))[:k]
            got = o["refine"][m, i]
            assert got[got >= 0].tolist() == [mine[j] for j in top], (m, i)


def pin_adaptive_chunks(lib):
    """Split/merge chunking: no change on keys with no dispersion; a
    constructed case with two worthwhile split/merge steps; ties between
    equal gains go to the lower block; on random keys a partition of n chunks
    of half, one or two blocks whose total dispersion is at most that of the
    fixed blocks, with as many splits as merges, merges aligned to pairs."""
    d, blk = 2, 4
    K = bf16_bits(np.full((32, d), 0.75))
    assert oracle.adaptive_chunks(K, blk, lib=lib).tolist() == oracle.fixed_chunks(32, blk).tolist()

    def build(blocks):
        return bf16_bits(np.array([row for b in blocks for row in b], np.float32))

    const = lambda v: [[v, v]] * 4
    halves = lambda a, b: [a, a, b, b]
    K2 = build([const(1), const(1), halves([0, 0], [4, 4]), const(3),
                const(-1), const(-1), halves([1, 0], [-1, 0]), const(5)])
    assert oracle.adaptive_chunks(K2, blk, lib=lib).tolist() == [8, 10, 12, 16, 24, 26, 28, 32]
    K3 = build([const(1), const(1), halves([0, 0], [4, 4]), const(100),
                const(0), const(10), halves([0, 0], [4, 4]), const(-100)])
    assert oracle.adaptive_chunks(K3, blk, lib=lib).tolist() == [8, 10, 12, 16, 20, 24, 28, 32]

    rng = np.random.default_rng(34)
    for L, blk in ((256, 8), (203, 8), (96, 4)):
        scale = np.repeat(rng.uniform(0.05, 2.0, -(-L // blk)), blk)[:L, None]
        Kr = bf16_bits(rng.standard_normal((L, 6)) * scale)
        Kf = bits_to_f64(Kr)
        cend = oracle.adaptive_chunks(Kr, blk, lib=lib)
        n = -(-L // blk)
        assert cend.size == n and cend[-1] == L and np.all(np.diff(cend) > 0)
        starts = np.concatenate([[0], cend[:-1]])
        sizes = cend - starts
        nsplit = nmerge = 0
        for a, e, sz in zip(starts, cend, sizes):
            if sz == blk // 2:
                nsplit += 1
                assert a % (blk // 2) == 0
            elif sz == 2 * blk:
                nmerge += 1
                assert a % (2 * blk) == 0
            else:
                assert sz == blk or e == L, (a, e)
        assert nsplit == 2 * nmerge  # a split block appears as two half chunks
        fixed = oracle.fixed_chunks(L, blk)
        fstarts = np.concatenate([[0], fixed[:-1]])
        tot = sum(chunk_dispersion(Kf[a:e]) for a, e in zip(starts, cend))
        tot_fixed = sum(chunk_dispersion(Kf[a:e]) for a, e in zip(fstarts, fixed))
        assert tot <= tot_fixed + 1e-9 * tot_fixed
        if L == 256:
            assert nmerge > 0  # the uneven scales make some steps worthwhile


ALL_PINS = [
    pin_golden_scores,
    pin_golden_topk,
    pin_golden_pivot,
    pin_golden_proxy_rounding,
    pin_relu_identities,
    pin_exact_dyadic,
    pin_homogeneity_and_heads,
    pin_one_hot,
    pin_select_vs_lexsort,
    pin_dense_causal,
    pin_pivot_invariants,
    pin_candidate_injection,
    pin_short_last_group,
    pin_proxy_strategies,
    pin_golden_chunks,
    pin_chunk_means_closed_forms,
    pin_chunk_reductions,
    pin_chunk_selection,
    pin_adaptive_chunks,
]
