"""The arithmetic behind bench.py's figures, checked on the CPU: scored-pair
counts against brute force over the causal triangle, groups and candidate
lists; recall against hand-made rows; and the rule that the dense launch's
HBM traffic comes from the committed counter record only while that record
matches the workload and the kernel sources it was taken on."""
import json
import os

import pytest
import torch

import bench


def brute_dense(L, q_len):
    off = L - q_len
    return sum(off + r + 1 for r in range(q_len))


@pytest.mark.parametrize("L,q_len", [(1, 1), (7, 7), (100, 1), (100, 3), (4096, 4096), (65536, 2)])
def test_dense_pairs(L, q_len):
    assert bench.dense_pairs(L, q_len) == brute_dense(L, q_len)


def test_dense_pairs_at_the_benchmark_size():
    # the causal triangle of one 131072-token sequence, diagonal included
    assert bench.dense_pairs(131072, 131072) == 131072 * 131073 // 2 == 8_590_000_128


@pytest.mark.parametrize("L,q_len,g", [(10, 10, 4), (10, 3, 2), (4097, 4097, 4), (50, 7, 16)])
def test_proxy_pairs(L, q_len, g):
    off = L - q_len
    G = (q_len + g - 1) // g
    want = sum(off + min((m + 1) * g, q_len) for m in range(G))  # t_last(m) + 1 keys per group
    brute = 0
    for m in range(G):
        t_last = off + min(m * g + g, q_len) - 1
        brute += sum(1 for s in range(L) if s <= t_last)
    assert bench.proxy_pairs(L, q_len, g) == want == brute


def test_refine_pairs():
    L, q_len, g = 12, 6, 4  # positions 6..11; groups {6,7,8,9} and {10,11}
    cand = torch.tensor([[[0, 7, 9, 11, -1], [2, 10, 11, -1, -1]]], dtype=torch.int32)
    brute = 0
    off = L - q_len
    for m in range(cand.shape[1]):
        for i in range(g):
            r = m * g + i
            if r >= q_len:
                continue
            brute += sum(1 for s in cand[0, m].tolist() if 0 <= s <= off + r)
    assert bench.refine_pairs(cand, L, q_len, g) == brute == 13  # 1+2+2+3 and 2+3


def test_chunk_pairs():
    L, q_len, g, nsel = 20, 8, 3, 2  # positions 12..19; groups end at 14, 17, 19
    cend = torch.tensor([[4, 9, 13, 16, 20]], dtype=torch.int32)
    cand = torch.tensor([[[0, 5, 12, -1], [13, 15, 16, 17], [1, 18, 19, -1]]], dtype=torch.int32)
    off = L - q_len
    G = cand.shape[1]
    coarse = refine = 0
    for m in range(G):
        t_last = off + min(m * g + g, q_len) - 1
        coarse += sum(1 for e in cend[0].tolist() if e - 1 <= t_last)  # complete chunks only
        for i in range(g):
            r = m * g + i
            if r < q_len:
                refine += sum(1 for s in cand[0, m].tolist() if 0 <= s <= off + r)
    assert bench.chunk_pairs(torch, cend, cand, L, q_len, g, nsel) == (coarse, refine)


def test_recall():
    d = torch.tensor([[0, 3, 5, -1], [1, 2, -1, -1]], dtype=torch.int32)
    assert bench.recall(d.clone(), d) == 1.0
    t = torch.tensor([[0, 4, 5, -1], [2, 7, -1, -1]], dtype=torch.int32)
    assert bench.recall(t, d) == pytest.approx((2 / 3 + 1 / 2) / 2)
    # padding in the tested rows never counts as a hit
    t = torch.tensor([[-1, -1, -1, -1], [-1, 1, -1, -1]], dtype=torch.int32)
    assert bench.recall(t, d) == pytest.approx((0 + 1 / 2) / 2)
    # rows are processed in chunks: the mean is over all rows
    big_d = torch.arange(10, dtype=torch.int32).repeat(9, 1)
    big_t = big_d.clone()
    big_t[::2, 0] = 99
    assert bench.recall(big_t, big_d, chunk=4) == pytest.approx(1 - 5 * 0.1 / 9)


def record(tmp_path, **kw):
    tr = {"kernel_hash": bench.kernel_hash(), "workload": "pivot128k", "hbm_bytes_per_launch": 1234.0}
    tr.update(kw)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(tr))
    return str(p)


def test_traffic_used_only_for_its_workload_and_sources(tmp_path):
    assert bench.dense_traffic("pivot128k", record(tmp_path)) == 1234.0
    assert bench.dense_traffic("dense16k", record(tmp_path)) is None
    assert bench.dense_traffic("pivot128k", record(tmp_path, kernel_hash="0" * 16)) is None
    assert bench.dense_traffic("pivot128k", str(tmp_path / "missing.json")) is None


def test_kernel_hash_covers_every_source(tmp_path, monkeypatch):
    files = []
    for i in range(3):
        f = tmp_path / f"src{i}.txt"
        f.write_bytes(b"kernel source %d" % i)
        files.append(f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [f.name for f in files])
    h0 = bench.kernel_hash()
    for f in files:
        old = f.read_bytes()
        f.write_bytes(old + b" ")
        assert bench.kernel_hash() != h0, f.name
        f.write_bytes(old)
    assert bench.kernel_hash() == h0


def test_committed_traffic_record_is_consistent():
    with open(bench.TRAFFIC_FILE) as f:
        tr = json.load(f)
    for p in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(bench.ROOT, p)), p
    want = tr["fetch_kib"] * 1024 * tr["fetch_scale"] + tr["write_kib"] * 1024 * tr["write_scale"]
    assert tr["hbm_bytes_per_launch"] == pytest.approx(want, rel=1e-9)
    # on the 1 GiB copy that calibrates them, FETCH_SIZE counts half of the
    # bytes read and WRITE_SIZE all of the bytes written
    assert 0.9 < tr["write_scale"] < 1.1 and 1.8 < tr["fetch_scale"] < 2.2
    assert len(tr["kernel_hash"]) == 16
