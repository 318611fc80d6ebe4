"""Benchmark of the DSA indexer and PIVOT Reuse/Refine on one MI355X.

A step is one pass of the whole prefill hot path over one synthetic sequence of
L = 131072 tokens (H_I = 64, d_I = 128, bf16; g = 4, c = 4096, k = 2048):
the dense indexer, PIVOT-Reuse and PIVOT-Refine (pooling, proxy scan, top-c,
re-score, top-k). Inputs are resident in HBM before timing starts. The line
printed at the end reports scored (query, key) pairs per second for the whole
step, top-k rows per second, the dense kernel against the bf16 MFMA roofline,
recall of Reuse/Refine against dense, a decode step (32 requests x 65536
cached keys, 2 new rows each, Refine) against the HBM roofline, the dense
indexer alone at L = 16384 against the MFMA roofline, the key-chunk
coarse stage (fixed and score-adaptive partitions of 64-key blocks, chunk scan
and Refine, on keys with local structure) with its recall against dense, and
the CPU oracle timed on a bounded sample of the same workload.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-pivot1m]
                       [--sweep | --guard-sweep | --chunk-sweep | --chunk-only PARTITION,G,NSEL]
                       [--no-decode] [--no-chunks] [--no-dense16k] [--variants dense,reuse,refine]
       python bench.py --decode-only [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SOURCES = ["sparse_attention_indexer_dense_amd/csrc/scan.hip",
                  "sparse_attention_indexer_dense_amd/csrc/device.h",
                  "sparse_attention_indexer_dense_amd/csrc/kernels.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dense_scan_pivot128k.json")


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dense_traffic(workload, path=TRAFFIC_FILE):
    """HBM bytes of one dense launch from the committed counter record
    (FETCH_SIZE and WRITE_SIZE, each scaled by a 1 GiB copy), or None when the
    record is missing, belongs to another workload or was taken on other
    kernel sources."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_hash") == kernel_hash() and tr.get("workload") == workload:
        return tr.get("hbm_bytes_per_launch")
    return None


def dense_pairs(L, q_len):
    off = L - q_len
    return sum_range(off + 1, L)  # row r scores pos(r) + 1 keys


def sum_range(a, b):
    """a + (a+1) + ... + b."""
    return (a + b) * (b - a + 1) // 2


def proxy_pairs(L, q_len, g):
    G = (q_len + g - 1) // g
    off = L - q_len
    return sum(off + min((m + 1) * g, q_len) for m in range(G))


def refine_pairs(cand, L, q_len, g):
    """Member-candidate pairs Refine scores: candidates at or before the member."""
    import torch
    B, G, c = cand.shape
    off = L - q_len
    total = 0
    for i in range(g):
        r = torch.arange(G, device=cand.device) * g + i
        valid = r < q_len
        pos = (off + r).view(1, G, 1)
        n = ((cand >= 0) & (cand <= pos)).sum(dim=2)
        total += int((n * valid.view(1, G)).sum())
    return total


def recall(test_idx, ref_idx, chunk=4096):
    """Mean over rows of |T cap D| / |D| (rows hold ascending indices, -1 padded)."""
    import torch
    t = test_idx.reshape(-1, test_idx.shape[-1])
    d = ref_idx.reshape(-1, ref_idx.shape[-1])
    big = torch.iinfo(torch.int32).max
    acc = 0.0
    for s in range(0, t.shape[0], chunk):
        tt = t[s:s + chunk]
        dd = d[s:s + chunk]
        ds = torch.where(dd < 0, torch.full_like(dd, big), dd).contiguous()
        pos = torch.searchsorted(ds, tt.contiguous()).clamp(max=ds.shape[1] - 1)
        hit = (torch.gather(ds, 1, pos) == tt) & (tt >= 0)
        nd = (dd >= 0).sum(dim=1).clamp(min=1)
        acc += float((hit.sum(dim=1).double() / nd.double()).sum())
    return acc / t.shape[0]


# ------------------------------------------------------------- CPU baseline
_KEYS = None


def _attach_keys(name, shape):
    global _KEYS
    import numpy as np
    from multiprocessing import shared_memory
    shm = shared_memory.SharedMemory(name=name)
    _KEYS = (shm, np.ndarray(shape, dtype=np.uint16, buffer=shm.buf))


def _oracle_row(args):
    """One dense row through the oracle: (pairs scored, seconds of this process)."""
    import oracle
    q, w, n, k = args
    t0 = time.perf_counter()
    sc, _ = oracle.scores(q, w, _KEYS[1], n=n)
    oracle.select(sc, k)
    return n, time.perf_counter() - t0


def cpu_baseline(Q, W, K, k, L, q_len, budget_rows, seed=0):
    """The fp64 oracle (dense rows) on a bounded random sample of rows, timed on
    the host cores with one single-threaded oracle per worker process."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from multiprocessing import shared_memory

    import numpy as np

    import oracle
    import synth
    oracle.load()
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(q_len, size=budget_rows, replace=False))
    Kh = synth.to_u16(K[0])
    Qh = synth.to_u16(Q[0, rows])
    Wh = W[0, rows].cpu().numpy()
    off = L - q_len
    work = [(Qh[i], Wh[i], off + int(r) + 1, k) for i, r in enumerate(rows)]
    workers = max(1, min(16, os.cpu_count() or 1, len(work)))
    shm = shared_memory.SharedMemory(create=True, size=Kh.nbytes)
    try:
        np.ndarray(Kh.shape, dtype=np.uint16, buffer=shm.buf)[:] = Kh
        ctx = mp.get_context("spawn")
        with ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_attach_keys,
                                 initargs=(shm.name, Kh.shape)) as ex:
            list(ex.map(_oracle_row, [(Qh[0], Wh[0], 1, k)] * workers))  # start the workers
            t0 = time.perf_counter()
            done = list(ex.map(_oracle_row, work))
            dt = time.perf_counter() - t0
    finally:
        shm.close()
        shm.unlink()
    pairs = sum(n for n, _ in done)
    busy = sum(t for _, t in done)  # seconds the workers spent on the rows
    full = dense_pairs(L, q_len)
    return {"value": pairs / dt, "unit": "pairs/s", "cores": workers, "kind": "oracle",
            "host_cpu_count": os.cpu_count(),
            "sample": f"dense rows of the same L={L} sequence: {len(rows)} rows drawn uniformly "
                      f"(seed {seed}), {pairs:.3e} scored pairs, fp64 single-threaded oracle per "
                      f"worker process, {dt:.1f} s wall",
            "seconds": dt,
            "per_core_pairs_per_s": pairs / busy,
            "dense_launch_s_extrapolated": {"one_core": full / (pairs / busy),
                                            f"{workers}_cores": full / (pairs / dt)}}


# ------------------------------------------------------------------- decode
def decode_scan(dsa, torch, Q, W, K, g, c, k, ws, out, reps=5):
    """The decode step's proxy scan alone (split_score_kernel over every
    cached key of each request) against the HBM roofline: algorithmic bytes =
    the key cache once, the proxy rows in and one fp32 score per key out; time
    = the median over `reps` steps of that kernel's own device time, from
    torch's profiler."""
    B, L, d = K.shape
    H = Q.shape[2]
    total = B * L * d * 2 + B * (H * d * 2 + H * 4) + B * L * 4
    times = []
    try:
        for _ in range(reps):
            ms, n, name = kernel_ms(torch, lambda: dsa.pivot_refine(Q, W, K, g, c, k, ws=ws, out=out),
                                    ("split_score_kernel<64, 128, false, 1>",))
            if ms is None:
                return {"error": "no proxy scan kernel in the profile"}
            times.append(ms)
    except Exception as e:  # noqa: BLE001 - report, do not fail the bench line
        return {"error": f"profiler: {e!r}"}
    ms = sorted(times)[len(times) // 2]
    if total / (ms * 1e-3) / 1e9 > 4 * PEAK_HBM_GBS:
        return {"error": f"implausible profiler time {ms:.6f} ms (another tracer attached?)"}
    return {"kernel": name, "kernel_us": ms * 1e3, "algorithmic_bytes": total,
            "achieved_GBps": total / (ms * 1e-3) / 1e9, "hbm_frac": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def bench_decode(dsa, synth, torch, iters=20, warmup=3, scan=True):
    """One PIVOT-Refine decode step (32 requests x 65536 cached keys, g = 2)
    timed with HIP events over `iters` steps, against the HBM roofline; with
    `scan`, also the proxy scan kernel alone."""
    w = synth.WORKLOADS["decode64k"]
    Q, W, K = synth.make(w, device="cuda")
    ws = dsa.Workspace()
    B, g, c, k, L = w.batch, w.g, w.c, w.k, w.L
    out = (torch.empty((B, g, k), dtype=torch.int32, device="cuda"),
           torch.empty((B, g, k), dtype=torch.float32, device="cuda"),
           torch.empty((B, 1, c), dtype=torch.int32, device="cuda"))
    for _ in range(warmup):
        dsa.pivot_refine(Q, W, K, g, c, k, ws=ws, out=out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        dsa.pivot_refine(Q, W, K, g, c, k, ws=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    # algorithmic bytes: every cached key once, the candidate rows once, queries,
    # weights and the outputs
    H, d = w.H, w.d
    nbytes = (B * L * d * 2 + B * c * d * 2 + B * g * H * d * 2 + B * g * H * 4
              + B * g * k * 8 + B * c * 4)
    d_idx, _ = dsa.dense(Q, W, K, k, ws=ws)
    rec = recall(out[0], d_idx)
    gbs = nbytes / (ms * 1e-3) / 1e9
    line = {"workload": "decode64k", "B": B, "L": L, "g": g, "c": c, "k": k,
            "variant": "refine", "ms_per_step": ms, "rows_per_s": B * g / (ms * 1e-3),
            "algorithmic_bytes": nbytes, "achieved_GBps": gbs,
            "hbm_frac": gbs / PEAK_HBM_GBS, "recall_vs_dense": rec}
    if scan:
        line["proxy_scan"] = decode_scan(dsa, torch, Q, W, K, g, c, k, ws, out)
    return line


def bench_dense16k(dsa, synth, torch, iters=10, warmup=2):
    """The dense indexer alone on the L = 16384 prefill sequence (H_I = 64,
    d_I = 128, k = 2048): kernel time per launch (HIP events) against the bf16
    MFMA roofline."""
    w = synth.WORKLOADS["dense16k"]
    Q, W, K = synth.make(w, device="cuda")
    ws = dsa.Workspace()
    out = (torch.empty((1, w.L, w.k), dtype=torch.int32, device="cuda"),
           torch.empty((1, w.L, w.k), dtype=torch.float32, device="cuda"))
    for _ in range(warmup):
        dsa.dense(Q, W, K, w.k, ws=ws, out=out)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record()
    for i in range(iters):
        dsa.dense(Q, W, K, w.k, ws=ws, out=out)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
    ms = ev[0].elapsed_time(ev[-1]) / iters
    pairs = dense_pairs(w.L, w.L)
    flop = pairs * 2 * w.H * w.d
    return {"workload": "dense16k", "L": w.L, "k": w.k, "ms": ms, "median_ms": t[len(t) // 2],
            "pairs_per_s": pairs / (ms * 1e-3), "queries_per_s": w.L / (ms * 1e-3),
            "achieved_TFLOPs": flop / (ms * 1e-3) / 1e12,
            "mfma_frac": flop / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)}


# -------------------------------------------------------------------- sweep
SWEEP_G = (2, 4, 8, 16)
SWEEP_C = (2048, 4096, 8192)
SWEEP_PROXY = (("mean", 0), ("mean", 4), ("first", 0), ("last", 0))


def sweep(dsa, torch, Q, W, K, k, steps=2):
    """Recall of Reuse and Refine against dense, and kernel time, over group
    sizes, candidate budgets and proxy strategies (one sequence). Prints one
    JSON line per configuration."""
    Qp, Wp, Kp = Q[0].contiguous(), W[0].contiguous(), K[0].contiguous()
    L, q = [K.shape[1]], [Q.shape[1]]
    ws = dsa.Workspace()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            out = fn()
        e1.record()
        torch.cuda.synchronize()
        return out, e0.elapsed_time(e1) / steps

    (d_idx, _), d_ms = timed(lambda: dsa.dense_varlen(Qp, Wp, Kp, L, q, k, scores=False, ws=ws))
    print(json.dumps({"sweep": "dense", "ms": d_ms}), flush=True)
    for g in SWEEP_G:
        for kind, window in SWEEP_PROXY:
            if window and window >= g:
                continue
            (r_idx, _, _), r_ms = timed(lambda: dsa.pivot_reuse_varlen(
                Qp, Wp, Kp, L, q, g, k, proxy=kind, window=window, scores=False, ws=ws))
            print(json.dumps({"sweep": "reuse", "g": g, "proxy": kind, "window": window, "ms": r_ms,
                              "speedup_vs_dense": d_ms / r_ms, "recall_vs_dense": recall(r_idx, d_idx)}),
                  flush=True)
            del r_idx
            for c in SWEEP_C:
                (f_idx, _, _), f_ms = timed(lambda: dsa.pivot_refine_varlen(
                    Qp, Wp, Kp, L, q, g, c, k, proxy=kind, window=window, scores=False, ws=ws))
                print(json.dumps({"sweep": "refine", "g": g, "c": c, "proxy": kind, "window": window,
                                  "ms": f_ms, "speedup_vs_dense": d_ms / f_ms,
                                  "recall_vs_dense": recall(f_idx, d_idx)}), flush=True)
                del f_idx


# ------------------------------------------------------------ key chunks
CHUNK_BLOCK = 64
CHUNK_CONFIGS = (("fixed", 1, 64), ("adaptive", 1, 64), ("fixed", 4, 64), ("adaptive", 4, 64))
CHUNK_SWEEP = tuple((p, g, n) for p in ("fixed", "adaptive") for g in (1, 4, 16) for n in (32, 48, 64, 96, 128))


def chunk_pairs(torch, cend, cand, L, q_len, g, nsel):
    """Scored pairs of a chunk call: the coarse scan (each group against the
    summaries of its complete chunks) plus Refine (each member against its
    causal candidates)."""
    G = cand.shape[1]
    m = torch.arange(G, device=cand.device)
    t_last = L - q_len + torch.clamp((m + 1) * g, max=q_len) - 1
    ncomp = torch.searchsorted(cend[0].to(torch.int64), t_last + 1, right=True)
    coarse = int(ncomp.sum())
    refine = 0
    for o in range(g):
        r = m * g + (g - 1 - o)
        live = r < q_len
        pos = L - q_len + r
        ok = (cand[0] >= 0) & (cand[0] <= pos[:, None]) & live[:, None]
        refine += int(ok.sum())
    return coarse, refine


def bench_chunks(dsa, synth, torch, w, Q, W, configs=CHUNK_CONFIGS, steps=3):
    """The key-chunk path at the workload's size on keys with local structure
    (synth.keys_local): index build (fixed or adaptive partition, summaries)
    and chunk scan + Refine, against the dense indexer on the same keys."""
    dev = Q.device
    L, d, k, H = w.L, w.d, w.k, w.H
    q_len = Q.shape[1]
    K = synth.keys_local(L, d, w.rank, w.seed, dev)[None]
    ws = dsa.Workspace()

    def timed(fn, n=steps):
        out = fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            out = fn()
        e1.record()
        torch.cuda.synchronize()
        return out, e0.elapsed_time(e1) / n

    (d_idx, _), d_ms = timed(lambda: dsa.dense(Q, W, K, k, scores=False, ws=ws), 1)
    parts = {"fixed": timed(lambda: dsa.chunks_fixed(1, L, CHUNK_BLOCK, dev)),
             "adaptive": timed(lambda: dsa.chunks_adaptive(K, CHUNK_BLOCK, ws=ws))}
    means = {p: timed(lambda: dsa.chunk_means(K, parts[p][0])) for p in parts}
    (p_idx, _, _), p_ms = timed(lambda: dsa.pivot_refine(Q, W, K, 4, 4096, k, scores=False, ws=ws))
    res = {"keys": "synth.keys_local", "block": CHUNK_BLOCK, "dense_ms": d_ms,
           "pivot_refine_g4_c4096": {"ms": p_ms, "speedup_vs_dense": d_ms / p_ms,
                                     "recall_vs_dense": recall(p_idx, d_idx)},
           "index_build_ms": {p: parts[p][1] + means[p][1] for p in parts},
           "partition_ms": {p: parts[p][1] for p in parts},
           "summary_ms": {p: means[p][1] for p in parts}, "runs": []}
    del p_idx
    flop_per_pair = 2 * H * d
    for part, g, nsel in configs:
        cend, Kbar = parts[part][0], means[part][0]
        mc = 2 * CHUNK_BLOCK if part == "adaptive" else CHUNK_BLOCK
        (idx, _, _, cand), ms = timed(lambda: dsa.chunk_refine(Q, W, K, Kbar, cend, g, nsel, mc, k,
                                                               scores=False, cand=True, ws=ws))
        coarse, refine = chunk_pairs(torch, cend, cand, L, q_len, g, nsel)
        # the Refine launch alone: each group's candidate keys gathered once
        # (every row's own list at g = 1; most of them hit in the L2, so the
        # gathered rate is set against the HBM peak for scale only) and its
        # MFMA share
        rk_ms, _, rk_name = kernel_ms(torch, lambda: dsa.chunk_refine(Q, W, K, Kbar, cend, g, nsel, mc, k,
                                                                      scores=False, cand=True, ws=ws),
                                      ("refine_lds_kernel", "scan_select_kernel<64, 128, 1, 2>",
                                       "scan_select_kernel<64, 128, 4, 2>", "scan_select_kernel<64, 128, 8, 2>"))
        gathered = int((cand >= 0).sum())
        print(f"[bench] chunks {part} g={g} nsel={nsel}: {ms:.2f} ms", file=sys.stderr, flush=True)
        run = {"partition": part, "g": g, "nsel": nsel, "max_chunk": mc, "ms": ms,
               "speedup_vs_dense": d_ms / ms, "recall_vs_dense": recall(idx, d_idx),
               "coarse_pairs": coarse, "refine_pairs": refine,
               "mean_candidates": refine / q_len,
               "mfma_frac": (coarse + refine) * flop_per_pair / (ms * 1e-3) /
               (PEAK_BF16_TFLOPS * 1e12)}
        if rk_ms:
            gb = gathered * 2 * d
            run["refine_kernel"] = {"kernel": rk_name, "kernel_ms": rk_ms, "gathered_keys": gathered,
                                    "gather_bytes": gb, "gather_GBps": gb / (rk_ms * 1e-3) / 1e9,
                                    "gather_vs_hbm_peak": gb / (rk_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                    "mfma_frac": refine * flop_per_pair / (rk_ms * 1e-3) /
                                    (PEAK_BF16_TFLOPS * 1e12)}
        res["runs"].append(run)
        del idx, cand
    return res


# --------------------------------------------------------------------- step
def bench_step(dsa, torch, Q, W, K, w, variants, steps, warmup):
    """Warm-up passes, then `steps` timed passes of the variants (dense, Reuse,
    Refine) over the same inputs, HIP events between the calls; work counted
    outside the timed region."""
    B, L, q_len, H, d = dsa._shapes(Q, W, K)
    k, g, c = w.k, w.g, w.c
    dev = Q.device

    def alloc(cand_c=None):
        G = (q_len + g - 1) // g
        return (torch.empty((B, q_len, k), dtype=torch.int32, device=dev),
                torch.empty((B, q_len, k), dtype=torch.float32, device=dev),
                torch.empty((B, G, cand_c), dtype=torch.int32, device=dev) if cand_c else None)

    outs = {v: alloc(c if v == "refine" else None) for v in variants}
    wss = {v: dsa.Workspace() for v in variants}

    def run(v):
        if v == "dense":
            dsa.dense(Q, W, K, k, ws=wss[v], out=outs[v][:2])
        elif v == "reuse":
            dsa.pivot_reuse(Q, W, K, g, k, ws=wss[v], out=outs[v])
        else:
            dsa.pivot_refine(Q, W, K, g, c, k, ws=wss[v], out=outs[v])

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(warmup):
        for v in variants:
            run(v)
    torch.cuda.synchronize()

    print("[bench] timed steps", file=sys.stderr, flush=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(variants) + 1)]
          for _ in range(steps)]
    t0 = time.perf_counter()
    torch.cuda.synchronize()
    for s in range(steps):
        ev[s][0].record()
        for i, v in enumerate(variants):
            run(v)
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_variant = {v: 0.0 for v in variants}
    samples = {v: [] for v in variants}
    step_ms = 0.0
    for s in range(steps):
        for i, v in enumerate(variants):
            t = ev[s][i].elapsed_time(ev[s][i + 1])
            per_variant[v] += t / steps
            samples[v].append(t)
        step_ms += ev[s][0].elapsed_time(ev[s][-1]) / steps

    # work accounting (outside the timed region)
    pd = dense_pairs(L, q_len) * B
    pp = proxy_pairs(L, q_len, g) * B if g > 0 else 0
    pairs = {"dense": pd}
    if "reuse" in variants:
        pairs["reuse"] = pp
    if "refine" in variants:
        pairs["refine"] = pp + refine_pairs(outs["refine"][2], L, q_len, g)
    total_pairs = sum(pairs[v] for v in variants)
    flop_per_pair = 2 * H * d
    detail = {}
    for v in variants:
        ms = per_variant[v]
        detail[v] = {"ms": ms, "median_ms": sorted(samples[v])[len(samples[v]) // 2], "scored_pairs": pairs[v],
                     "pairs_per_s": pairs[v] / (ms * 1e-3),
                     "dense_equiv_pairs_per_s": pd / (ms * 1e-3),
                     "queries_per_s": B * q_len / (ms * 1e-3),
                     "mfma_frac": pairs[v] * flop_per_pair / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)}
        if v != "dense":
            detail[v]["speedup_vs_dense"] = per_variant["dense"] / ms
            detail[v]["recall_vs_dense"] = recall(outs[v][0], outs["dense"][0])
    return {"outs": outs, "per_variant": per_variant, "detail": detail, "step_ms": step_ms,
            "total_pairs": total_pairs, "wall": wall, "dense_pairs": pd}


def bench_pivot1m(dsa, synth, torch, dev):
    """The long-context workload (L = 1048576, g = 16, c = 8192, k = 2048):
    one warm-up and one timed pass of dense, Reuse and Refine on the same
    inputs (HIP events around each call), recall of Reuse and Refine against
    dense over every row."""
    w = synth.WORKLOADS["pivot1m"]
    Q, W, K = synth.make(w, device=dev)
    step = bench_step(dsa, torch, Q, W, K, w, list(w.variants), 1, 1)
    det = step["detail"]
    res = {"workload": w.name, "L": w.L, "g": w.g, "c": w.c, "k": w.k, "steps": 1, "warmup": 1,
           "ms_per_step": step["step_ms"], "pairs_per_s": step["total_pairs"] / (step["step_ms"] * 1e-3),
           "variants": {v: {x: det[v][x] for x in ("ms", "scored_pairs", "pairs_per_s", "queries_per_s",
                                                   "mfma_frac", "speedup_vs_dense", "recall_vs_dense")
                            if x in det[v]} for v in det}}
    del step, Q, W, K
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------ guard sweep
GUARD_L = (2048, 4096, 8192, 16384, 32768, 65536, 131072)


def guard_sweep(dsa, synth, torch, steps=3, g=4, c=4096, k=2048):
    """Dense against PIVOT-Refine without and with the guard (guard = c: a
    group whose whole prefix fits in c keys is scored densely, which for
    Refine leaves the results unchanged; guard = 2c: groups whose prefix holds
    up to 2c keys are scored densely, their rows exact) and PIVOT-Reuse, at
    short and long sequences, through the variable-length entry points. One
    JSON line per L."""
    ws = dsa.Workspace()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            out = fn()
        e1.record()
        torch.cuda.synchronize()
        return out, e0.elapsed_time(e1) / steps

    rows = []
    for L in GUARD_L:
        Q, W, K = synth.prefill(L, 64, 128, 0.95, 4, seed=0, device="cuda")
        Qp, Wp, Kp = Q[0].contiguous(), W[0].contiguous(), K[0].contiguous()
        del Q, W, K
        kk = min(k, L)
        (d_idx, _), d_ms = timed(lambda: dsa.dense_varlen(Qp, Wp, Kp, [L], [L], kk, scores=False, ws=ws))
        (r_idx, _, _), r_ms = timed(lambda: dsa.pivot_refine_varlen(Qp, Wp, Kp, [L], [L], g, c, kk, guard=0,
                                                                    scores=False, ws=ws))
        (q_idx, _, _), q_ms = timed(lambda: dsa.pivot_refine_varlen(Qp, Wp, Kp, [L], [L], g, c, kk, guard=c,
                                                                    scores=False, ws=ws))
        (q2_idx, _, _), q2_ms = timed(lambda: dsa.pivot_refine_varlen(Qp, Wp, Kp, [L], [L], g, c, kk,
                                                                      guard=2 * c, scores=False, ws=ws))
        (u_idx, _, _), u_ms = timed(lambda: dsa.pivot_reuse_varlen(Qp, Wp, Kp, [L], [L], g, kk, scores=False,
                                                                   ws=ws))
        row = {"sweep": "guard", "L": L, "g": g, "c": c, "k": kk, "dense_ms": d_ms, "refine_ms": r_ms,
               "refine_guarded_ms": q_ms, "refine_guarded_2c_ms": q2_ms, "reuse_ms": u_ms,
               "guarded_groups": min(c // g, (L + g - 1) // g),
               "guarded_groups_2c": min(2 * c // g, (L + g - 1) // g),
               "guarded_refine_le_dense": q_ms <= d_ms, "guarded_2c_refine_le_dense": q2_ms <= d_ms,
               "recall_refine_guarded_2c": recall(q2_idx, d_idx),
               "refine_identical_with_guard": bool(torch.equal(r_idx, q_idx)),
               "recall_refine": recall(r_idx, d_idx), "recall_reuse": recall(u_idx, d_idx)}
        print(json.dumps(row), flush=True)
        rows.append(row)
        del d_idx, r_idx, q_idx, q2_idx, u_idx, Qp, Wp, Kp
        torch.cuda.empty_cache()
    return rows


def copy_1gib(torch, dev):
    """One 1 GiB device-to-device copy: a dispatch of known traffic for
    scaling the HBM counters of the same profiled run."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def kernel_ms(torch, fn, patterns):
    """Mean device time (ms) of the kernels whose name contains one of
    `patterns`, their count and the first such name, over one call of fn, from
    torch's profiler (which traces every HIP kernel launched in the process,
    the library's included)."""
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    times, name = [], None
    for e in prof.events():
        if not any(pt in e.name for pt in patterns):
            continue
        us = getattr(e, "device_time", None)
        if us is None:
            us = getattr(e, "cuda_time", None)
        if us:
            times.append(float(us) / 1e3)
            name = name or e.name
    if not times:
        return None, 0, None
    return sum(times) / len(times), len(times), name


def refine_gather(dsa, torch, Q, W, K, g, c, k, cand):
    """The prefill Refine re-score (refine_lds_kernel for groups of up to four
    members and up to 4096 candidates, else scan_select_kernel in its Refine
    mode: each group's candidate keys gathered once for its members) against
    the HBM roofline: algorithmic bytes = every group's causal candidate keys
    (2 d bytes each) plus its list, the members' queries and weights, and their
    outputs; time = that kernel's own device time, from torch's profiler."""
    B, q_len, H, d = Q.shape
    L = K.shape[1]
    G = cand.shape[1]
    ar = torch.arange(G, device=cand.device)
    t_last = torch.clamp((ar + 1) * g, max=q_len) - 1 + (L - q_len)
    per_group = torch.clamp(t_last + 1, max=c)
    ncand = int(per_group.sum()) * B
    # every member scores its group's whole list (causality is applied when
    # it selects): members x list length pairs, 2 H d flop each
    members = torch.clamp(q_len - ar * g, max=g)
    pairs = int((per_group * members).sum()) * B
    gather = ncand * 2 * d
    total = gather + ncand * 4 + B * q_len * (H * d * 2 + H * 4 + k * 8)
    try:
        ms, n, name = kernel_ms(torch, lambda: dsa.pivot_refine(Q, W, K, g, c, k, scores=False),
                                ("refine_lds_kernel", ", 2>(dsaidx::ScanParams)"))
    except Exception as e:  # noqa: BLE001 - report, do not fail the bench line
        return {"error": f"profiler: {e!r}"}
    if ms is None:
        return {"error": "no Refine scan kernel in the profile"}
    if total / (ms * 1e-3) / 1e9 > 4 * PEAK_HBM_GBS:
        # torch's profiler under another tracer (rocprofv3) reports sub-microsecond
        # durations; no kernel moves these bytes at 4x the HBM peak
        return {"error": f"implausible profiler time {ms:.6f} ms (another tracer attached?)"}
    tflops = pairs * 2.0 * H * d / (ms * 1e-3) / 1e12
    return {"kernel": name, "launches": n, "kernel_ms": ms,
            "candidate_keys": ncand, "gather_bytes": gather, "algorithmic_bytes": total,
            "gather_GBps": gather / (ms * 1e-3) / 1e9, "achieved_GBps": total / (ms * 1e-3) / 1e9,
            "hbm_frac": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "scored_pairs": pairs, "achieved_TFLOPs": tflops, "mfma_frac": tflops / PEAK_BF16_TFLOPS}


# --------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="pivot128k")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="rows of the oracle CPU baseline (0 disables it)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="instead of the step: only the decode Refine step (--steps timed calls; for traces)")
    ap.add_argument("--variants", default=None, metavar="dense[,reuse][,refine]",
                    help="variants run in the step (default: all the workload has; for counter runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: recall and time of Reuse/Refine over g, c and proxy")
    ap.add_argument("--no-chunks", action="store_true", help="skip the key-chunk measurement")
    ap.add_argument("--no-dense16k", action="store_true", help="skip the L=16384 dense measurement")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="instead of the step: the key-chunk path over partitions, g and nsel")
    ap.add_argument("--guard-sweep", action="store_true",
                    help="instead of the step: dense vs Refine with and without the guard over L")
    ap.add_argument("--no-pivot1m", action="store_true", help="skip the L=1048576 pass")
    ap.add_argument("--no-gather", action="store_true",
                    help="skip the profiler timing of the Refine re-score kernel (for counter runs)")
    ap.add_argument("--chunk-only", default=None, metavar="PARTITION,G,NSEL",
                    help="instead of the step: build one partition and run only that chunk call "
                         "(--steps times; for kernel traces)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library does not shard the "
              "indexer across GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_indexer_dense_amd as dsa
    import synth

    dsa.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode_only:
        line = bench_decode(dsa, synth, torch, iters=args.steps, warmup=args.warmup, scan=False)
        if args.calibrate_copy:
            copy_1gib(torch, dev)
        print(json.dumps(line), flush=True)
        return
    if args.guard_sweep:
        guard_sweep(dsa, synth, torch)
        return
    w = synth.WORKLOADS[args.workload]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    Q, W, K = synth.make(w, device=dev)
    B, L, q_len, H, d = dsa._shapes(Q, W, K)
    k, g, c = w.k, w.g, w.c
    variants = list(w.variants)
    if args.variants:
        want = args.variants.split(",")
        if "dense" not in want or any(v not in variants for v in want):
            print(f"--variants must name dense and a subset of {variants}", file=sys.stderr)
            sys.exit(2)
        variants = [v for v in variants if v in want]
    if args.sweep:
        sweep(dsa, torch, Q, W, K, k)
        return
    if args.chunk_only:
        part, cg, cn = args.chunk_only.split(",")
        del K
        Kl = synth.keys_local(L, d, w.rank, w.seed, dev)[None]
        cend = dsa.chunks_adaptive(Kl, CHUNK_BLOCK) if part == "adaptive" else dsa.chunks_fixed(1, L, CHUNK_BLOCK, dev)
        Kbar = dsa.chunk_means(Kl, cend)
        mc = 2 * CHUNK_BLOCK if part == "adaptive" else CHUNK_BLOCK
        ws = dsa.Workspace()
        for i in range(args.steps):
            dsa.chunk_refine(Q, W, Kl, Kbar, cend, int(cg), int(cn), mc, k, scores=False, ws=ws)
            torch.cuda.synchronize()
            print(f"[bench] chunk call {i} done", file=sys.stderr, flush=True)
        if args.calibrate_copy:
            copy_1gib(torch, dev)
        return
    if args.chunk_sweep:
        del K
        print(json.dumps(bench_chunks(dsa, synth, torch, w, Q, W, configs=CHUNK_SWEEP, steps=2)), flush=True)
        return

    step = bench_step(dsa, torch, Q, W, K, w, variants, args.steps, args.warmup)
    outs, per_variant, detail = step["outs"], step["per_variant"], step["detail"]
    step_ms, total_pairs, wall, pd = step["step_ms"], step["total_pairs"], step["wall"], step["dense_pairs"]
    flop_per_pair = 2 * H * d

    dense_ms = per_variant["dense"]
    achieved = pd * flop_per_pair / (dense_ms * 1e-3) / 1e12
    traffic = dense_traffic(w.name)
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "kernel": "scan_select_kernel<64,128,8,dense>",
                "flop_per_launch": pd * flop_per_pair}

    gather = None
    if "refine" in variants and not args.no_gather:
        print("[bench] Refine re-score kernel (profiler)", file=sys.stderr, flush=True)
        gather = refine_gather(dsa, torch, Q, W, K, g, c, k, outs["refine"][2])
        detail["refine"]["gather"] = gather

    if args.calibrate_copy:
        copy_1gib(torch, dev)

    decode = None
    if not args.no_decode:
        print("[bench] decode step", file=sys.stderr, flush=True)
        decode = bench_decode(dsa, synth, torch)

    d16 = None
    if not args.no_dense16k:
        print("[bench] dense indexer at L=16384", file=sys.stderr, flush=True)
        d16 = bench_dense16k(dsa, synth, torch)

    chunks = None
    if not args.no_chunks:
        print("[bench] key-chunk path", file=sys.stderr, flush=True)
        chunks = bench_chunks(dsa, synth, torch, w, Q, W)

    cpu = None
    if args.cpu_rows > 0:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(Q, W, K, k, L, q_len, args.cpu_rows)
        cpu["gpu_over_cpu"] = (total_pairs / (step_ms * 1e-3)) / cpu["value"]

    p1m = None
    if not args.no_pivot1m and w.name == "pivot128k":
        del outs, step, Q, W, K
        torch.cuda.empty_cache()
        print("[bench] L=1048576 pass", file=sys.stderr, flush=True)
        p1m = bench_pivot1m(dsa, synth, torch, dev)

    value = total_pairs / (step_ms * 1e-3)
    line = {
        "metric": "indexer (query,key) pairs/s + top-k queries/s at L=128K; % MFMA / HBM peak",
        "value": value, "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "L": L, "q_len": q_len, "H_I": H, "d_I": d,
                   "k": k, "g": g, "c": c, "variants": variants},
        "queries_per_s": B * q_len * len(variants) / (step_ms * 1e-3),
        "variants": detail,
        "roofline": roofline,
        "decode": decode,
        "dense16k": d16,
        "chunks": chunks,
        "pivot1m": p1m,
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
