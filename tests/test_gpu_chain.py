"""GPU parity of GEMV chains (qmv_chain): one launch, device-wide waits between GEMVs."""
import numpy as np
import pytest
import torch

import gen
import oracle
from block_quantized_matrix_amd import bqm
from tests._gpu import DEV, check_close, host, packed, say, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _oracle():
    oracle.build(force=False)


def make_chain(fmt, shapes, key, dependent=True, M=1):
    """GEMVs i = 0..n-1 with W_i [N_i][K_i], inputs [M][K_i], outputs [M][N_i]; if
    dependent, x_{i+1} is y_i (N_i == K_{i+1}) and every GEMV after the first waits, else
    none waits (one segment)."""
    Ws, Wps, xs, ys, descs = [], [], [], [], []
    x = gen.normal((M, shapes[0][1]), key + ("x0",), device=DEV)
    for i, (N, K) in enumerate(shapes):
        Wi = weights(fmt, N, K, key + (i,))
        Wp = packed(fmt, Wi, N, K)
        if not dependent and i > 0:
            x = gen.normal((M, K), key + ("x", i), device=DEV)
        y = torch.full((M, N), float("nan"), device=DEV)
        Ws.append(Wi); Wps.append(Wp); xs.append(x); ys.append(y)
        descs.append(bqm.gemv(fmt, Wp, x, y, N, K, wait=dependent and i > 0, M=M))
        if dependent:
            x = y
    ws = torch.zeros(bqm.chain_workspace_bytes(len(descs)), dtype=torch.uint8, device=DEV)
    bqm.bqm_chain_prepare(descs, ws)
    return Ws, Wps, xs, ys, descs, ws


def check_stages(fmt, shapes, Ws, xs, ys, M=1):
    for i, (N, K) in enumerate(shapes):
        xi = host(xs[i]).reshape(M, K)
        assert np.all(np.isfinite(xi)), f"stage {i} read an input that was never written"
        Yr, S = oracle.qmv(fmt, host(Ws[i]), xi, N, K)
        check_close(host(ys[i]).reshape(M, N), Yr, S, f"chain stage {i} ({N}x{K}, M={M})")


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_chain_dependent_stages(fmt):
    """Each GEMV reads the previous one's output: a missing device-wide wait would read the
    NaN the output buffers start with."""
    shapes = [(5120, 4096), (17408, 5120), (5120, 17408), (1536, 5120), (4096, 1536), (96, 4096)]
    say("chain dependent", fmt)
    Ws, Wps, xs, ys, descs, ws = make_chain(fmt, shapes, ("chain-dep", fmt))
    bqm.qmv_chain(fmt, 1, ws, len(descs))
    assert bqm.bqm_chain_status(ws) == 0
    check_stages(fmt, shapes, Ws, xs, ys)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M", [2, 4, 8])
def test_chain_batched_dependent_stages(fmt, M):
    """Batch M through dependent GEMVs; K = 17408 with M >= 4 does not fit the LDS at once,
    so that GEMV is walked in chunks of K with per-row partial sums."""
    shapes = [(4096, 1536), (17408, 4096), (1536, 17408), (520, 1536)]
    say("chain batched", fmt, M)
    Ws, Wps, xs, ys, descs, ws = make_chain(fmt, shapes, ("chain-bat", fmt, M), M=M)
    bqm.qmv_chain(fmt, M, ws, len(descs))
    assert bqm.bqm_chain_status(ws) == 0
    check_stages(fmt, shapes, Ws, xs, ys, M=M)


@pytest.mark.parametrize("M", [3, 8])
def test_chain_batched_ragged_one_segment(M):
    """Independent GEMVs of a batched chain form one segment, whose rows of all GEMVs are
    split between the workgroups together: ragged and tiny shapes, and one long K."""
    shapes = [(37, 96), (300, 1184), (1, 9600), (2049, 32768)]
    say("chain batched one segment", M)
    Ws, Wps, xs, ys, descs, ws = make_chain("q8_0", shapes, ("chain-bq", M), dependent=False, M=M)
    bqm.qmv_chain("q8_0", M, ws, len(descs))
    assert bqm.bqm_chain_status(ws) == 0
    check_stages("q8_0", shapes, Ws, xs, ys, M=M)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M", [1, 8])
def test_chain_many_gemvs_in_segments(fmt, M):
    """150 small GEMVs with waits at 40, 41 and 130 (segments of 40, 1, 89 and 20 GEMVs); a
    waiting GEMV reads the output of the one before it.  A workgroup's share touches few of
    a segment's GEMVs, and most workgroups hold no row of the last segment (they enter only
    its wait), so the GEMVs each enters are linked across the 64-GEMV words of its table;
    every output meets the bar, and a replay gives the same bits."""
    waits = {40, 41, 130}
    Ns, Ks = [1, 7, 64, 300, 33], [256, 512, 1024]
    # the last segment: 20 GEMVs of 1-7 rows of 256 weights (about 2.5 blocks per workgroup)
    Kof = [Ks[i % 3] if i < 130 else 256 for i in range(150)]
    shapes = []
    for i in range(150):
        N = Ns[(3 * i) % 5] if i < 130 else [1, 7, 3][i % 3]
        if i + 1 in waits:
            N = Kof[i + 1]  # the next GEMV reads this output
        shapes.append((N, Kof[i]))
    say("chain many GEMVs", fmt, M)
    Ws, Wps, xs, ys, descs = [], [], [], [], []  # the descriptors hold raw pointers: keep all alive
    for i, (N, K) in enumerate(shapes):
        Wi = weights(fmt, N, K, ("chain-many", fmt, i))
        Wp = packed(fmt, Wi, N, K)
        x = ys[i - 1] if i in waits else gen.normal((M, K), ("chain-many-x", fmt, M, i), device=DEV)
        y = torch.full((M, N), float("nan"), device=DEV)
        Ws.append(Wi); Wps.append(Wp); xs.append(x); ys.append(y)
        descs.append(bqm.gemv(fmt, Wp, x, y, N, K, wait=i in waits, M=M))
    ws = torch.zeros(bqm.chain_workspace_bytes(len(descs)), dtype=torch.uint8, device=DEV)
    bqm.bqm_chain_prepare(descs, ws)
    outs = []
    for _ in range(2):
        bqm.qmv_chain(fmt, M, ws, len(descs))
        assert bqm.bqm_chain_status(ws) == 0
        outs.append([host(y).copy() for y in ys])
    check_stages(fmt, shapes, Ws, xs, ys, M=M)
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


def test_chain_segments_with_mixed_waits():
    """Segments of several GEMVs with different K: A and B read x0; C (waits) reads A's
    output and D (same segment) B's; E (waits) reads C's.  A workgroup whose share of a
    segment misses a GEMV still takes part in that segment's wait."""
    fmt = "q4_0"
    say("chain mixed waits")
    sh = {"A": (5120, 4096), "B": (320, 4096), "C": (96, 5120), "D": (2000, 320), "E": (4096, 96)}
    Wi = {k: weights(fmt, N, K, ("chain-mix", k)) for k, (N, K) in sh.items()}
    Wp = {k: packed(fmt, Wi[k], *sh[k]) for k in sh}
    y = {k: torch.full((1, N), float("nan"), device=DEV) for k, (N, K) in sh.items()}
    x0 = gen.normal((1, 4096), ("chain-mix-x",), device=DEV)
    xin = {"A": x0, "B": x0, "C": y["A"], "D": y["B"], "E": y["C"]}
    wait = {"A": False, "B": False, "C": True, "D": False, "E": True}
    order = ["A", "B", "C", "D", "E"]
    descs = [bqm.gemv(fmt, Wp[k], xin[k], y[k], *sh[k], wait=wait[k]) for k in order]
    ws = torch.zeros(bqm.chain_workspace_bytes(len(descs)), dtype=torch.uint8, device=DEV)
    bqm.bqm_chain_prepare(descs, ws)
    for rep in range(2):
        for k in order:
            y[k].fill_(float("nan"))
        bqm.qmv_chain(fmt, 1, ws, len(descs))
        assert bqm.bqm_chain_status(ws) == 0
        for k in order:
            N, K = sh[k]
            xi = host(xin[k]).reshape(1, K)
            assert np.all(np.isfinite(xi)), f"{k} read an input that was never written"
            Yr, S = oracle.qmv(fmt, host(Wi[k]), xi, N, K)
            check_close(host(y[k]).reshape(1, N), Yr, S, f"mixed waits {k} (replay {rep})")


def test_chain_ragged_and_tiny_shapes():
    """Ragged K (K/32 not a multiple of the lane group), rows fewer than CUs, tiny shapes."""
    say("chain ragged")
    shapes = [(37, 96), (3, 1184), (300, 96), (1, 9600), (65, 32), (2049, 1536)]
    Ws, Wps, xs, ys, descs, ws = make_chain("q4_0", shapes, ("chain-ragged",), dependent=False)
    bqm.qmv_chain("q4_0", 1, ws, len(descs))
    assert bqm.bqm_chain_status(ws) == 0
    check_stages("q4_0", shapes, Ws, xs, ys)


def test_chain_replays_are_bit_identical():
    """Every replay of a chain gives the same bits (and matches the oracle)."""
    shapes = [(7168, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]
    say("chain replays")
    Ws, Wps, xs, ys, descs, ws = make_chain("q4_0", shapes, ("chain-eq",), dependent=False)
    first = None
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        bqm.qmv_chain("q4_0", 1, ws, len(descs))
        assert bqm.bqm_chain_status(ws) == 0
        if first is None:
            first = [y.clone() for y in ys]
            check_stages("q4_0", shapes, Ws, xs, ys)
        for y, y0 in zip(ys, first):
            assert torch.equal(y, y0), f"replay {rep}"


def test_chain_mismatch_is_reported_and_computes_nothing():
    shapes = [(64, 512), (64, 64)]
    Ws, Wps, xs, ys, descs, ws = make_chain("q4_0", shapes, ("chain-mis",))
    bqm.qmv_chain("q4_0", 1, ws, 3)        # wrong n
    assert bqm.bqm_chain_status(ws) == 2
    assert torch.all(torch.isnan(ys[0]))
    bqm.bqm_chain_prepare(descs, ws)       # prepare again: clean state
    bqm.qmv_chain("q8_0", 1, ws, 2)        # wrong format
    assert bqm.bqm_chain_status(ws) == 2
    bqm.bqm_chain_prepare(descs, ws)
    bqm.qmv_chain("q4_0", 4, ws, 2)        # wrong batch
    assert bqm.bqm_chain_status(ws) == 2
    assert torch.all(torch.isnan(ys[0]))
    bqm.bqm_chain_prepare(descs, ws)
    bqm.qmv_chain("q4_0", 1, ws, 2)
    assert bqm.bqm_chain_status(ws) == 0
    check_stages("q4_0", shapes, Ws, xs, ys)


def test_chain_prepare_rejects_bad_descriptors():
    W = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    x = torch.zeros(64, device=DEV)
    y = torch.zeros(64, device=DEV)
    ws = torch.zeros(bqm.chain_workspace_bytes(2), dtype=torch.uint8, device=DEV)
    good = bqm.gemv("q4_0", W, x, y, 64, 64, False)
    def g(w=W.data_ptr(), K=64, fmt=2, M=1):
        return bqm.Gemv(w, x.data_ptr(), y.data_ptr(), 64, K, fmt, 0, M, 0)
    for bad in (g(K=48), g(K=0), g(K=32800),  # K % 32, K = 0, K too long
                g(fmt=8), g(M=2), g(w=0)):    # mixed format, mixed batch, null matrix
        with pytest.raises(bqm.BqmError):
            bqm.bqm_chain_prepare([good, bad], ws)


def test_chain_prepare_rejects_bad_batch():
    W = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    x = torch.zeros(64 * 9, device=DEV)
    y = torch.zeros(64 * 9, device=DEV)
    ws = torch.zeros(bqm.chain_workspace_bytes(1), dtype=torch.uint8, device=DEV)
    for M in (0, 9):
        with pytest.raises(bqm.BqmError):
            bqm.bqm_chain_prepare([bqm.Gemv(W.data_ptr(), x.data_ptr(), y.data_ptr(), 64, 64, 2, 0, M, 0)], ws)
