"""The seeded input generator: determinism, the encoder readings, error bounds, router ids."""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import gen
from tests import _npref

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")))


def _sha(t):
    return hashlib.sha256(t.contiguous().numpy().tobytes()).hexdigest()


def test_determinism_and_key_sensitivity():
    a = gen.encode_q4_0(gen.normal((64, 256), ("det", 0), std=0.02))
    b = gen.encode_q4_0(gen.normal((64, 256), ("det", 0), std=0.02))
    c = gen.encode_q4_0(gen.normal((64, 256), ("det", 1), std=0.02))
    assert _sha(a) == _sha(b) and _sha(a) != _sha(c)
    assert gen.seed_of("x", 1) != gen.seed_of("x", 2)
    assert np.array_equal(gen.router_ids(4, 128, 8, ("r", 3)), gen.router_ids(4, 128, 8, ("r", 3)))


def test_round_half_away():
    v = torch.tensor([2.5, -2.5, 0.5, -0.5, 1.49999988, 0.49999997, 3.0, -0.0, 7.5])
    assert gen.round_half_away(v).tolist() == [3.0, -3.0, 1.0, -1.0, 1.0, 0.0, 3.0, 0.0, 8.0]


def test_encode_q4_0_stored_scale_reading():
    case = GOLDEN["encode_q4_0"][0]
    w = torch.zeros(1, 32)
    w[0, :5] = torch.tensor(case["w_first5"])
    blk = gen.encode_q4_0(w)[0].numpy()
    assert int(blk[0]) | (int(blk[1]) << 8) == int(case["d_bits"], 16)
    qs = blk[2:]
    codes = np.concatenate([qs & 15, qs >> 4])
    assert list(codes[:5]) == case["codes_first5"]
    assert np.all(codes[5:] == 8)


def test_zero_blocks():
    w = torch.zeros(2, 64)
    q4 = gen.encode_q4_0(w).numpy().reshape(2, 2, 18)
    q8 = gen.encode_q8_0(w).numpy().reshape(2, 2, 34)
    assert np.all(q4[:, :, :2] == 0) and np.all(q4[:, :, 2:] == 0x88)
    assert np.all(q8 == 0)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_encoder_error_bounds(fmt):
    N, K = 64, 512
    w = gen.normal((N, K), ("bound", fmt), std=0.02)
    W = (gen.encode_q4_0(w) if fmt == "q4_0" else gen.encode_q8_0(w)).numpy()
    deq = _npref.dequant(fmt, W, N, K)
    bb = 18 if fmt == "q4_0" else 34
    d = np.abs(W.reshape(N, K // 32, bb)[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64))
    dd = np.repeat(d, 32, axis=1)
    err = np.abs(w.numpy().astype(np.float64) - deq)
    if fmt == "q4_0":
        blk = W.reshape(N, K // 32, 18)[:, :, 2:]
        codes = np.concatenate([blk & 15, blk >> 4], axis=2).reshape(N, K)
        clamped = codes == 15
        assert np.all(err[~clamped] <= dd[~clamped] / 2 * (1 + 1e-6))
        assert np.all(err[clamped] <= dd[clamped] * (1 + 1e-6))
        # the element of largest magnitude maps to code 0 (value -8 d)
        wb = w.numpy().reshape(N, K // 32, 32)
        k = np.abs(wb).argmax(axis=2)
        c = codes.reshape(N, K // 32, 32)
        assert np.all(np.take_along_axis(c, k[:, :, None], 2) == 0)
    else:
        assert np.all(err <= dd / 2 * (1 + 1e-6))


def test_raw_blocks_ranges():
    W = gen.raw_q8_0(8, 128, ("raw",), codes=(-8, 8)).numpy().reshape(8, 4, 34)
    q = W[:, :, 2:].view(np.int8)
    assert q.min() >= -8 and q.max() <= 8
    d = W[:, :, 0:2].copy().view(np.float16)[:, :, 0]
    assert set(np.unique(d).tolist()) <= {0.5, 1.0, 2.0}


def test_router_ids_skewed_topk():
    T, E, k = 4096, 128, 8
    ids = gen.router_ids(T, E, k, ("router", 0))
    assert ids.shape == (T, k) and ids.dtype == np.int32
    assert ids.min() >= 0 and ids.max() < E
    assert all(len(set(r)) == k for r in ids[:256])
    counts = np.bincount(ids.reshape(-1), minlength=E)
    # skew: the first experts are far more popular than the last ones
    assert counts[:8].sum() > 10 * max(1, counts[-8:].sum())
    # at 16 tokens several tens of distinct experts are touched, not just 8
    uniq = [len(np.unique(gen.router_ids(16, E, k, ("router", s)))) for s in range(20)]
    assert 16 < np.mean(uniq) < 64
