"""The entry points captured in a HIP graph (as the benchmark runs them): every replay, with
eager work and synchronizations between replays, gives the eager result bit for bit."""
import pytest
import torch

import gen
from block_quantized_matrix_amd import bqm
from tests._gpu import DEV, packed, say, weights

pytestmark = pytest.mark.gpu


def replays_match_eager(run, outputs, n=3):
    """run(): launches on the current stream.  Eager result first, then capture and replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    for i in range(n):
        for o in outputs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV) * 3.0   # eager work between replays
        junk.sum().item()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert torch.equal(o, e), f"replay {i} differs from the eager result"


def test_graph_dependent_chain():
    say("graph: dependent chain")
    shapes = [(1024, 4096), (4096, 1024), (512, 4096)]
    Ks = [4096, 1024, 4096]
    x0 = gen.normal((1, 4096), ("g-chain-x",), device=DEV)
    ys = [torch.empty((1, N), device=DEV) for N, _ in shapes]
    mats = [packed("q4_0", weights("q4_0", N, K, ("g-chain", i)), N, K) for i, (N, K) in enumerate(shapes)]
    xs = [x0, ys[0], ys[1]]
    descs = [bqm.gemv("q4_0", w, x, y, N, K, wait=i > 0)
             for i, ((N, K), w, x, y) in enumerate(zip(shapes, mats, xs, ys))]
    ws = torch.zeros(bqm.chain_workspace_bytes(len(descs)), dtype=torch.uint8, device=DEV)
    bqm.bqm_chain_prepare(descs, ws)
    replays_match_eager(lambda: bqm.qmv_chain("q4_0", 1, ws, len(descs)), ys)
    assert bqm.bqm_chain_status(ws) == 0


def test_graph_moe_decode_layer():
    say("graph: MoE decode layer")
    E, F, H, T, top_k = 16, 384, 1024, 4, 4
    ids = torch.from_numpy(gen.router_ids(T, E, top_k, ("g-moe",))).to(DEV)
    rw = torch.from_numpy(gen.router_weights(T, top_k, ("g-moe",))).to(DEV)
    gate = packed("q4_0", weights("q4_0", E * F, H, ("g-moe", "g")), E * F, H)
    up = packed("q4_0", weights("q4_0", E * F, H, ("g-moe", "u")), E * F, H)
    down = packed("q4_0", weights("q4_0", E * H, F, ("g-moe", "d")), E * H, F)
    x = gen.normal((T, H), ("g-moe-x",), device=DEV)
    h = torch.empty((T, top_k, F), device=DEV)
    ys = torch.empty((T, top_k, H), device=DEV)
    y = torch.empty((T, H), device=DEV)

    def run():
        bqm.qmv_id_gate_up("q4_0", gate, up, E, F, H, ids, T, top_k, x, H, 0, h)
        bqm.qmv_id_sum("q4_0", down, E, H, F, ids, rw, T, top_k, h, top_k * F, F, ys, y)

    replays_match_eager(run, [h, ys, y])


def test_graph_prefill_products():
    say("graph: prefill products")
    M, N, K, E, top_k = 96, 256, 1024, 8, 2
    X = gen.normal((M, K), ("g-pre-x",), device=DEV)
    Xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    dx = torch.empty((M, K // 32), device=DEV)
    w4 = packed("q4_0", weights("q4_0", N, K, ("g-pre",)), N, K)
    we = packed("q8_0", weights("q8_0", E * N, K, ("g-pre-e",)), E * N, K)
    ids = torch.from_numpy(gen.router_ids(M, E, top_k, ("g-pre",))).to(DEV)
    Y = torch.empty((M, N), device=DEV)
    Yi = torch.empty((M, top_k, N), device=DEV)

    def run():
        bqm.bqm_quantize_q8_act(X, Xq, dx, M, K)
        bqm.qmm_q4_0(w4, Xq, dx, Y, M, N, K)
        bqm.qmm_id("q8_0", we, E, N, K, ids, M, top_k, Xq, dx, 1, 0, Yi)

    replays_match_eager(run, [Y, Yi])
    assert not torch.isnan(Y).any() and not torch.isnan(Yi).any()
