"""HIP graph capture of whole indexer calls. The library enqueues kernels only
(no memset, copy, allocation or synchronisation), so a call can be captured
once and replayed, as a serving loop does with a decode step. Each captured
call here replays to the same bits as the eager call, replay after replay,
with the program's own eager work and synchronisations in between, and it
reads its inputs when it replays: inputs overwritten in place between replays
give the eager results on the new inputs. Covered: the decode shape (split
kernels), a prefill sequence (scan kernels, dense and Refine in one graph), a
variable-length batch with the guard, and the entry point that needs no
workspace (for callers that cannot allocate while capturing)."""
import ctypes

import pytest
import torch

import sparse_attention_indexer_dense_amd as dsa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def assert_same(got, ref):
    assert len(got) == len(ref)
    for a, b in zip(got, ref):
        if b is None:
            assert a is None
            continue
        assert torch.equal(bits(a), bits(b))


def replay_checked(graph, outs, ref):
    """Replays `graph` REPLAYS times; before each, eager work overwrites the
    outputs; after each, they must equal `ref` bit for bit."""
    for _ in range(REPLAYS):
        for x in outs:
            if x is not None:
                x.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_same(outs, ref)


def capture(fn):
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    torch.cuda.synchronize()
    return graph, out


def test_graph_decode_refine():
    B, L, g, c, k = 4, 20000, 2, 1024, 512
    Q, W, K = synth.decode(B, L, g, 64, 128, 0.95, 4, seed=21, device=DEV)
    ws_e, ws_g = dsa.Workspace(), dsa.Workspace()
    ref = dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws_e)
    out = tuple(torch.empty_like(x) for x in ref)
    dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws_g, out=out)  # sizes ws_g
    torch.cuda.synchronize()
    graph, _ = capture(lambda: dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws_g, out=out))
    replay_checked(graph, out, ref)
    # the next step's inputs, written in place
    Q2, W2, K2 = synth.decode(B, L, g, 64, 128, 0.95, 4, seed=22, device=DEV)
    Q.copy_(Q2)
    W.copy_(W2)
    K.copy_(K2)
    ref2 = dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws_e)
    torch.cuda.synchronize()
    assert not torch.equal(ref2[0], ref[0])
    replay_checked(graph, out, ref2)


def test_graph_prefill_dense_and_refine():
    L, g, c, k = 1500, 4, 256, 64
    Q, W, K = synth.prefill(L, 4, 32, 0.9, 2, 23, DEV)
    ws_e, ws_d, ws_r = dsa.Workspace(), dsa.Workspace(), dsa.Workspace()
    ref_d = dsa.dense(Q, W, K, k, ws=ws_e)
    ref_r = dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws_e)
    out_d = tuple(torch.empty_like(x) for x in ref_d)
    out_r = tuple(torch.empty_like(x) for x in ref_r)
    dsa.dense(Q, W, K, k, ws=ws_d, out=out_d)
    dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws_r, out=out_r)
    torch.cuda.synchronize()

    def step():
        dsa.dense(Q, W, K, k, ws=ws_d, out=out_d)
        dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws_r, out=out_r)

    graph, _ = capture(step)
    replay_checked(graph, out_d + out_r, ref_d + ref_r)
    Q2, W2, K2 = synth.prefill(L, 4, 32, 0.9, 2, 24, DEV)
    Q.copy_(Q2)
    W.copy_(synth.signed_weights(L, 4, 25, DEV)[None])
    K.copy_(K2)
    ref_d2 = dsa.dense(Q, W, K, k, ws=ws_e)
    ref_r2 = dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws_e)
    torch.cuda.synchronize()
    replay_checked(graph, out_d + out_r, ref_d2 + ref_r2)


def test_graph_varlen_refine_guarded():
    Ls, qs, g, c, k, guard = [3000, 9000, 700], [3000, 2, 0], 4, 512, 128, 1000
    reqs = [synth.prefill(L, 4, 32, 0.9, 2, 30 + r, DEV) for r, L in enumerate(Ls)]
    Qp = torch.cat([x[0][0, L - q:] for x, L, q in zip(reqs, Ls, qs)]).contiguous()
    Wp = torch.cat([x[1][0, L - q:] for x, L, q in zip(reqs, Ls, qs)]).contiguous()
    Kp = torch.cat([x[2][0] for x in reqs]).contiguous()
    ws_e, ws_g = dsa.Workspace(), dsa.Workspace()
    ref = dsa.pivot_refine_varlen(Qp, Wp, Kp, Ls, qs, g, c, k, guard=guard, cand=True, ws=ws_e)
    dsa.pivot_refine_varlen(Qp, Wp, Kp, Ls, qs, g, c, k, guard=guard, cand=True, ws=ws_g)  # sizes ws_g
    torch.cuda.synchronize()
    # the outputs are allocated while capturing, from the graph's own pool
    graph, out = capture(lambda: dsa.pivot_refine_varlen(Qp, Wp, Kp, Ls, qs, g, c, k, guard=guard, cand=True,
                                                         ws=ws_g))
    replay_checked(graph, out, ref)
    Kp.copy_(torch.cat([synth.prefill(L, 4, 32, 0.9, 2, 40 + r, DEV)[2][0] for r, L in enumerate(Ls)]))
    ref2 = dsa.pivot_refine_varlen(Qp, Wp, Kp, Ls, qs, g, c, k, guard=guard, cand=True, ws=ws_e)
    torch.cuda.synchronize()
    assert not torch.equal(ref2[0], ref[0])
    replay_checked(graph, out, ref2)


def test_graph_noalloc_decode():
    B, L, g, c, k, H, d = 3, 12000, 2, 1024, 512, 64, 128
    Q, W, K = synth.decode(B, L, g, H, d, 0.95, 4, seed=51, device=DEV)
    G = 1
    ws = dsa.Workspace()
    ref = dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws)
    out = (torch.empty((B, g, k), dtype=torch.int32, device=DEV),
           torch.empty((B, g, k), dtype=torch.float32, device=DEV),
           torch.empty((B, G, c), dtype=torch.int32, device=DEV))
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def call():
        stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
        rc = dsa.indexer_pivot_refine_noalloc(ptr(Q), ptr(W), ptr(K), B, L, g, H, d, g, c, k, ptr(out[0]),
                                              ptr(out[1]), ptr(out[2]), stream)
        assert rc == 0, dsa.indexer_last_error()

    call()  # first call on the device: takes the scratch array's address
    torch.cuda.synchronize()
    assert_same(out, ref)
    graph, _ = capture(call)
    replay_checked(graph, out, ref)
    Q2, W2, K2 = synth.decode(B, L, g, H, d, 0.95, 4, seed=52, device=DEV)
    Q.copy_(Q2)
    W.copy_(W2)
    K.copy_(K2)
    ref2 = dsa.pivot_refine(Q, W, K, g, c, k, cand=True, ws=ws)
    torch.cuda.synchronize()
    replay_checked(graph, out, ref2)
