"""qmv_id_sum_noalloc (the router-weighted expert sum for callers that cannot allocate) against
qmv_id_sum, through the C ABI: two calls in a row, the second with a smaller input, each
bit for bit equal to qmv_id_sum with a caller buffer and within the bar of the oracle."""
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


def _case(fmt, E, N, K, T, top_k, key):
    Wi = weights(fmt, E * N, K, key)
    ids = gen.router_ids(T, E, top_k, key + ("ids",))
    ids[0, top_k - 1] = -1  # a padding slot
    w = gen.router_weights(T, top_k, key + ("w",))
    X = gen.normal((T, top_k, K), key + ("x",), device=DEV)
    return Wi, ids, w, X


def test_noalloc_matches_qmv_id_sum_on_consecutive_calls():
    cases = [("q4_0", 128, 4096, 1536, 16, 8),   # the MoE down projection, 16 tokens: 2 MiB of rows
             ("q8_0", 6, 200, 544, 3, 3)]        # then a smaller call reusing the array
    for fmt, E, N, K, T, top_k in cases:
        assert T * top_k * N <= bqm.NOALLOC_SLOT_FLOATS
        say("noalloc", fmt, E, N, K, T, top_k)
        Wi, ids, w, X = _case(fmt, E, N, K, T, top_k, ("noalloc", fmt, T))
        Wp = packed(fmt, Wi, E * N, K)
        idd, wd = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
        Ys = torch.full((T, top_k, N), float("nan"), device=DEV)
        Y_ref = torch.full((T, N), float("nan"), device=DEV)
        bqm.qmv_id_sum(fmt, Wp, E, N, K, idd, wd, T, top_k, X, top_k * K, K, Ys, Y_ref)
        Y = torch.full((T, N), float("nan"), device=DEV)
        bqm.qmv_id_sum_noalloc(fmt, Wp, E, N, K, idd, wd, T, top_k, X, top_k * K, K, Y)
        assert torch.equal(Y.view(torch.int32), Y_ref.view(torch.int32))
        Yr, S = oracle.qmv_id_sum(fmt, host(Wi), E, N, K, ids, w, host(X).reshape(-1), top_k * K, K)
        check_close(host(Y), Yr, S, f"noalloc {fmt} T={T}")


def test_noalloc_rejects_more_rows_than_the_array_holds():
    T, top_k, N, K, E = bqm.QMV_ID_MAX_T, bqm.QMV_ID_MAX_TOPK, 1024, 32, 4
    assert T * top_k * N > bqm.NOALLOC_SLOT_FLOATS
    Y = torch.full((T, N), 3.0, device=DEV)
    ids = torch.zeros((T, top_k), dtype=torch.int32, device=DEV)
    w = torch.ones((T, top_k), device=DEV)
    X = torch.zeros((T, K), device=DEV)
    W = torch.zeros(bqm.packed_bytes("q4_0", E * N, K), dtype=torch.uint8, device=DEV)
    with pytest.raises(bqm.BqmError) as e:
        bqm.qmv_id_sum_noalloc("q4_0", W, E, N, K, ids, w, T, top_k, X, K, 0, Y)
    assert e.value.status == 2
    assert np.all(host(Y) == 3.0)
