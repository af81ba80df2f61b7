"""GPU parity of GEMVs and chains at batches of 5 to 8 inputs whose K is a multiple of 256
(256 x 32 weights: the matrix-core form of the chain), against the oracle: single calls over
ragged row counts and chunked K, exact probes, dependent chains, one independent segment,
graph-free replays."""
import numpy as np
import pytest
import torch

import gen
import oracle
from block_quantized_matrix_amd import bqm
from tests._gpu import DEV, check_close, host, packed, say, weights
from tests.test_gpu_chain import check_stages, make_chain

pytestmark = pytest.mark.gpu

FMTS = ["q4_0", "q8_0"]
QMV = {"q4_0": bqm.qmv_q4_0, "q8_0": bqm.qmv_q8_0}
# rows: one, ragged tiles, more rows than workgroups; K: one step, whole, chunked, the longest;
# K = 128 and 384 (whole 128-byte steps of Q8_0 rows; the vector form for Q4_0, whose steps
# are 256 weights)
SHAPES = [(1, 256), (17, 512), (300, 4096), (70, 17408), (33, 32768), (2049, 1536), (3, 128), (257, 384)]


@pytest.fixture(scope="module", autouse=True)
def _oracle():
    oracle.build(force=False)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [5, 6, 7, 8])
@pytest.mark.parametrize("N,K", SHAPES)
def test_mc_single_call_parity(fmt, M, N, K):
    say("mc single", fmt, M, N, K)
    Wi = weights(fmt, N, K, ("mc", fmt, N, K))
    X = gen.normal((M, K), ("mc-x", M, K), device=DEV)
    Y = torch.full((M, N), float("nan"), device=DEV)
    Yg = torch.full((M + 1, N), float("nan"), device=DEV)  # one guard row past the output
    QMV[fmt](packed(fmt, Wi, N, K), X, Yg[:M], M, N, K)
    Y.copy_(Yg[:M])
    Yr, S = oracle.qmv(fmt, host(Wi), host(X), N, K)
    check_close(host(Y), Yr, S, f"{fmt} M={M} N={N} K={K}")
    assert np.all(np.isnan(host(Yg[M]))), "a store past the output"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [5, 8])
@pytest.mark.parametrize("N,K", [(300, 4096), (19, 17408)])
def test_mc_exact_probe(fmt, M, N, K):
    """Exact inputs (integer x, power-of-two scales, small codes): bit for bit."""
    say("mc exact", fmt, M, N, K)
    if fmt == "q4_0":
        Wi = gen.raw_q4_0(N, K, ("mc-probe", N, K), device=DEV)
    else:
        Wi = gen.raw_q8_0(N, K, ("mc-probe", N, K), codes=(-8, 8), device=DEV)
    X = gen.small_int((M, K), ("mc-probe-x", M, K), device=DEV)
    Y = torch.empty((M, N), device=DEV)
    QMV[fmt](packed(fmt, Wi, N, K), X, Y, M, N, K)
    Yr, _ = oracle.qmv(fmt, host(Wi), host(X), N, K)
    assert np.array_equal(host(Y).astype(np.float64), Yr)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [5, 7])
def test_mc_chain_dependent_stages(fmt, M):
    """Each GEMV reads the previous one's output (a missing wait reads NaN); K = 17408 goes
    in chunks; every replay gives the same bits."""
    shapes = [(1536, 4096), (4096, 1536), (17408, 4096), (1024, 17408), (256, 1024)]
    say("mc chain dependent", fmt, M)
    Ws, Wps, xs, ys, descs, ws = make_chain(fmt, shapes, ("mc-dep", fmt, M), M=M)
    outs = []
    for rep in range(2):
        bqm.qmv_chain(fmt, M, ws, len(descs))
        assert bqm.bqm_chain_status(ws) == 0
        outs.append([host(y).copy() for y in ys])
    check_stages(fmt, shapes, Ws, xs, ys, M=M)
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("fmt", FMTS)
def test_mc_chain_one_segment(fmt):
    """Independent GEMVs of one segment (their rows split between the workgroups together),
    tiny to long shapes, at batch 8."""
    M = 8
    shapes = [(37, 256), (300, 1280 if fmt == "q8_0" else 1536), (1, 9728), (2049, 32768), (5, 512)]
    say("mc chain one segment", fmt)
    Ws, Wps, xs, ys, descs, ws = make_chain(fmt, shapes, ("mc-seg", fmt), dependent=False, M=M)
    bqm.qmv_chain(fmt, M, ws, len(descs))
    assert bqm.bqm_chain_status(ws) == 0
    check_stages(fmt, shapes, Ws, xs, ys, M=M)


def test_mc_chain_with_a_ragged_k_uses_the_vector_form():
    """A chain in which one GEMV's K is not a multiple of 256 runs whole on the vector form;
    the results meet the same bar."""
    fmt, M = "q4_0", 6
    shapes = [(512, 4096), (96, 512), (300, 96)]
    say("mc chain with ragged K")
    Ws, Wps, xs, ys, descs, ws = make_chain(fmt, shapes, ("mc-rag",), M=M)
    bqm.qmv_chain(fmt, M, ws, len(descs))
    assert bqm.bqm_chain_status(ws) == 0
    check_stages(fmt, shapes, Ws, xs, ys, M=M)
