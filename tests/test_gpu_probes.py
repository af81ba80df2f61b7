"""Exact probes at the full workload shapes: inputs for which every single-precision step of
any summation order is exact (scales in {0.5, 1, 2}, integer inputs in [-8, 8], codes with
|code| <= 8), so the GPU result must equal the oracle bit for bit.  At these sizes the
relative tolerance could not see one wrong code, scale or index (a single weight is about
S/K of a sum); here any such slip changes an output.

Shapes: the 4096 x 4096 Q4_0 GEMV; the 27B-dense layer shapes as the benchmark runs them
(q|k|v 7168 x 5120, o 5120 x 5120, gate|up 34816 x 5120, down 5120 x 17408), Q4_0 at batch 1
and Q8_0 at batches 1, 4 and 8; the 128-expert top-8 MoE layer (gate and up 1536 x 4096,
down 4096 x 1536 per expert) at 1 and 16 tokens in the indexed, gate+up and weighted-sum
forms.  The bound on every partial sum (|sum| / granularity < 2^24) is asserted per case.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from block_quantized_matrix_amd import bqm
from tests._gpu import DEV, host, packed, say

pytestmark = pytest.mark.gpu

QMV = {"q4_0": bqm.qmv_q4_0, "q8_0": bqm.qmv_q8_0}


@pytest.fixture(scope="module", autouse=True)
def _oracle():
    oracle.build(force=False)


def raw(fmt, rows, K, key):
    if fmt == "q4_0":
        return gen.raw_q4_0(rows, K, key, device=DEV)      # codes n - 8 in [-8, 7]
    return gen.raw_q8_0(rows, K, key, codes=(-8, 8), device=DEV)


def exact_bound_ok(K):
    """|partial sums| / 0.5 < 2^24: K products of |code| <= 8, |x| <= 8, d <= 2, in units of
    the scales' granularity 0.5."""
    return K * 8 * 8 * 2 / 0.5 < 2 ** 24


def dense_probe(fmt, M, N, K, key):
    assert exact_bound_ok(K)
    say("exact probe", fmt, M, N, K)
    Wi = raw(fmt, N, K, key)
    X = gen.small_int((M, K), key + ("x",), device=DEV)
    Y = torch.full((M, N), float("nan"), device=DEV)
    QMV[fmt](packed(fmt, Wi, N, K), X, Y, M, N, K)
    Yr, _ = oracle.qmv(fmt, host(Wi), host(X), N, K)
    y = host(Y).astype(np.float64)
    bad = y != Yr
    assert not bad.any(), f"{fmt} M={M} {N}x{K}: {int(bad.sum())} outputs differ, first at {np.argwhere(bad)[0]}"


def test_probe_gemv_4096():
    dense_probe("q4_0", 1, 4096, 4096, ("probe-4096",))


@pytest.mark.parametrize("name,N,K", gen.DENSE27B_FUSED_SHAPES)
def test_probe_27b_q4_0_batch1(name, N, K):
    dense_probe("q4_0", 1, N, K, ("probe-27b", name))


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("name,N,K", gen.DENSE27B_FUSED_SHAPES)
def test_probe_27b_q8_0(name, N, K, M):
    dense_probe("q8_0", M, N, K, ("probe-27b-q8", name, M))


def test_probe_27b_layer_chain():
    """One 27B layer as the benchmark runs it (four GEMVs, each waiting for the earlier
    ones, in one chain launch), every output exact."""
    say("exact probe chain")
    descs, refs, keep = [], [], []
    for i, (name, N, K) in enumerate(gen.DENSE27B_FUSED_SHAPES):
        Wi = raw("q4_0", N, K, ("probe-chain", name))
        X = gen.small_int((1, K), ("probe-chain-x", name), device=DEV)
        Y = torch.full((1, N), float("nan"), device=DEV)
        Wp = packed("q4_0", Wi, N, K)
        keep += [Wp, X, Y]
        descs.append(bqm.gemv("q4_0", Wp, X, Y, N, K, wait=i > 0))
        refs.append((Y, oracle.qmv("q4_0", host(Wi), host(X), N, K)[0]))
    ws = torch.zeros(bqm.chain_workspace_bytes(len(descs)), dtype=torch.uint8, device=DEV)
    bqm.bqm_chain_prepare(descs, ws)
    bqm.qmv_chain("q4_0", 1, ws, len(descs))
    assert bqm.bqm_chain_status(ws) == 0
    for Y, Yr in refs:
        assert np.array_equal(host(Y).astype(np.float64), Yr)


# ---- the MoE layer ---------------------------------------------------------------------

def moe_ids(T):
    sh = gen.MOE_SHAPE
    return gen.router_ids(T, sh["E"], sh["top_k"], ("moe-router", T))


@pytest.mark.parametrize("T", [1, 16])
@pytest.mark.parametrize("proj", ["gate", "down"])
def test_probe_moe_qmv_id(T, proj):
    sh = gen.MOE_SHAPE
    E, top_k = sh["E"], sh["top_k"]
    N, K = (sh["ffn"], sh["hidden"]) if proj == "gate" else (sh["hidden"], sh["ffn"])
    assert exact_bound_ok(K)
    ids = moe_ids(T)
    say("exact probe qmv_id", T, proj)
    Wi = raw("q4_0", E * N, K, ("probe-moe", proj))
    if proj == "gate":
        X = gen.small_int((T, K), ("probe-moe-x", T), device=DEV)
        xts, xss = K, 0
    else:
        X = gen.small_int((T, top_k, K), ("probe-moe-x", T, "down"), device=DEV)
        xts, xss = top_k * K, K
    Y = torch.full((T, top_k, N), float("nan"), device=DEV)
    bqm.qmv_id("q4_0", packed("q4_0", Wi, E * N, K), E, N, K, torch.from_numpy(ids).to(DEV), T,
               top_k, X, xts, xss, Y)
    Yr, _ = oracle.qmv_id("q4_0", host(Wi), E, N, K, ids, host(X).reshape(-1), xts, xss)
    assert np.array_equal(host(Y).astype(np.float64), Yr)


@pytest.mark.parametrize("T", [1, 16])
def test_probe_moe_gate_up(T):
    """Fused gate+up: g and u are exact here, so the output must be the single-precision
    evaluation of silu(g) * u (expf, a correctly rounded division, two products) to a few
    ulp -- one wrong code or index would move g or u by at least 0.5 and the output by far
    more than that."""
    sh = gen.MOE_SHAPE
    E, top_k, N, K = sh["E"], sh["top_k"], sh["ffn"], sh["hidden"]
    ids = moe_ids(T)
    say("exact probe gate_up", T)
    Wg, Wu = raw("q4_0", E * N, K, ("probe-gu", "g")), raw("q4_0", E * N, K, ("probe-gu", "u"))
    X = gen.small_int((T, K), ("probe-gu-x", T), device=DEV)
    Y = torch.full((T, top_k, N), float("nan"), device=DEV)
    bqm.qmv_id_gate_up("q4_0", packed("q4_0", Wg, E * N, K), packed("q4_0", Wu, E * N, K), E, N, K,
                       torch.from_numpy(ids).to(DEV), T, top_k, X, K, 0, Y)
    g, _ = oracle.qmv_id("q4_0", host(Wg), E, N, K, ids, host(X).reshape(-1), K, 0)
    u, _ = oracle.qmv_id("q4_0", host(Wu), E, N, K, ids, host(X).reshape(-1), K, 0)
    g32, u32 = g.astype(np.float32), u.astype(np.float32)
    assert np.array_equal(g32.astype(np.float64), g) and np.array_equal(u32.astype(np.float64), u)
    with np.errstate(over="ignore"):
        want = (g32 / (np.float32(1) + np.exp(-g32)) * u32).astype(np.float64)
    y = host(Y).astype(np.float64)
    assert np.all(np.abs(y - want) <= 4 * 2.0 ** -23 * np.abs(want) + 1e-30), \
        float(np.max(np.abs(y - want) / (np.abs(want) + 1e-30)))


@pytest.mark.parametrize("T", [1, 16])
def test_probe_moe_weighted_sum(T):
    """Router-weighted down projection and slot sum with weights in {0.5, 1}: every product
    and every sum is exact, so the layer output equals the oracle bit for bit."""
    sh = gen.MOE_SHAPE
    E, top_k, N, K = sh["E"], sh["top_k"], sh["hidden"], sh["ffn"]
    assert K * 8 * 8 * 2 * top_k / 0.25 < 2 ** 24
    ids = moe_ids(T)
    say("exact probe weighted sum", T)
    Wi = raw("q4_0", E * N, K, ("probe-sum",))
    X = gen.small_int((T, top_k, K), ("probe-sum-x", T), device=DEV)
    w = (1 + (np.random.default_rng(T).integers(0, 2, (T, top_k)))).astype(np.float32) * np.float32(0.5)
    Ys = torch.full((T, top_k, N), float("nan"), device=DEV)
    Y = torch.full((T, N), float("nan"), device=DEV)
    bqm.qmv_id_sum("q4_0", packed("q4_0", Wi, E * N, K), E, N, K, torch.from_numpy(ids).to(DEV),
                   torch.from_numpy(w).to(DEV), T, top_k, X, top_k * K, K, Ys, Y)
    Yr, _ = oracle.qmv_id_sum("q4_0", host(Wi), E, N, K, ids, w, host(X).reshape(-1), top_k * K, K)
    assert np.array_equal(host(Y).astype(np.float64), Yr)
