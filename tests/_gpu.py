"""Helpers for the GPU parity tests: device inputs, the tolerance check, oracle access."""
import sys

import numpy as np
import torch

import gen
from block_quantized_matrix_amd import bqm

DEV = "cuda"


def say(*a):
    """Print (flushed) what the next GPU step is, so a crash names its case."""
    print(*a, flush=True)
    sys.stdout.flush()


def encode(fmt, w):
    return gen.encode_q4_0(w) if fmt == "q4_0" else gen.encode_q8_0(w)


def weights(fmt, N, K, key, device=DEV, std=0.02):
    """Seeded Gaussian weights quantized to interchange bytes, on `device`."""
    return encode(fmt, gen.normal((N, K), key, std=std, device=device))


def packed(fmt, W_inter_dev, N, K):
    return bqm.repack(fmt, W_inter_dev.reshape(-1), N, K)


def check_close(y, Y_ref, S, what=""):
    """Acceptance: |y - y_ref| <= 1e-3 * S per output; S == 0 forces y == 0 exactly."""
    y64 = np.asarray(y, np.float64)
    err = np.abs(y64 - Y_ref)
    bad = ~(err <= 1e-3 * S)   # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs out of tolerance, e.g. at {idx.tolist()}: "
                             f"got {y64[tuple(idx[0])]}, want {Y_ref[tuple(idx[0])]}, S {S[tuple(idx[0])]}")
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(S > 0, err / S, 0.0)
    return float(rel.max()) if rel.size else 0.0


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()
