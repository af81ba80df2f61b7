"""Seeded synthetic inputs (see the package docstring for what this module is not).

Every generator takes a *key*: a tuple of ints and strings naming the tensor
(workload, layer, tensor name, ...).  The key is hashed into a seed, so the same
key always gives the same bytes on the same device type.  Gaussian draws use
torch's generator of the target device (the CPU and GPU streams differ; each
test feeds the *same bytes* to both sides of a comparison, so this does not
matter for parity).

Block byte layout produced here (the interchange layout read by the library's
repack call and by the oracle):
  Q4_0, 18 bytes per 32 weights: binary16 scale d (little endian), then 16 bytes;
        byte j holds weight j in its low nibble and weight j+16 in its high nibble.
  Q8_0, 34 bytes per 32 weights: binary16 scale d, then 32 signed bytes.
Q4_0 and Q8_0 are the formats named in the quantization-format table of the page
"V100跑Qwen 27B：量化与KV Cache调优" (lmnt.cn), section 4.1; the page does not spell
out the block layout, so the conventional ggml layout above is used.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

__all__ = [
    "QK", "Q4_0_BLOCK_BYTES", "Q8_0_BLOCK_BYTES", "seed_of", "normal", "round_half_away",
    "encode_q4_0", "encode_q8_0", "raw_q4_0", "raw_q8_0", "small_int", "router_ids", "router_weights",
    "DENSE27B_LAYERS", "DENSE27B_SHAPES", "DENSE27B_FUSED_SHAPES", "MOE_SHAPE", "MOE_PREFILL_T", "PREFILL_SHAPE",
    "block_bytes",
]

QK = 32                 # weights per block
Q4_0_BLOCK_BYTES = 18   # 2-byte scale + 16 bytes of nibbles
Q8_0_BLOCK_BYTES = 34   # 2-byte scale + 32 signed bytes

# 27B-dense decode stream: 64 layers, each (name, N = output rows, K = input length).
DENSE27B_LAYERS = 64
DENSE27B_SHAPES = (
    ("q", 5120, 5120), ("k", 1024, 5120), ("v", 1024, 5120), ("o", 5120, 5120),
    ("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408),
)
# Same weights grouped by shared input: q|k|v rows stacked, gate|up rows stacked.
DENSE27B_FUSED_SHAPES = (
    ("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408),
)
# 128-expert MoE layer: gate/up 4096 -> 1536 and down 1536 -> 4096 per expert, top-8.
MOE_SHAPE = dict(E=128, top_k=8, hidden=4096, ffn=1536)
# MoE prefill: the MoE layer's experts over a 512-token prompt.
MOE_PREFILL_T = 512
# Prefill GEMM: 512 tokens through a 5120 -> 17408 projection.
PREFILL_SHAPE = dict(M=512, K=5120, N=17408)


def block_bytes(fmt: str) -> int:
    return {"q4_0": Q4_0_BLOCK_BYTES, "q8_0": Q8_0_BLOCK_BYTES}[fmt]


def seed_of(*key) -> int:
    """Stable 63-bit seed from a key of ints and strings."""
    words = []
    for k in key:
        if isinstance(k, str):
            words.append(int.from_bytes(hashlib.sha256(k.encode()).digest()[:4], "little"))
        else:
            words.append(int(k) & 0xFFFFFFFF)
    st = np.random.SeedSequence(words).generate_state(2, dtype=np.uint32)
    return (int(st[0]) | (int(st[1]) << 32)) & ((1 << 63) - 1)


def _gen(key, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key))
    return g


def normal(shape, key, std: float = 1.0, device="cpu") -> torch.Tensor:
    """fp32 draws from N(0, std^2)."""
    t = torch.randn(tuple(shape), generator=_gen(key, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def round_half_away(v: torch.Tensor) -> torch.Tensor:
    """Round to nearest, ties away from zero (C roundf), without the x+0.5 pitfall."""
    t = torch.trunc(v)
    frac = v - t  # exact for |v| < 2^23
    return t + torch.where(frac.abs() >= 0.5, torch.sign(v), torch.zeros_like(v))


def _scale_bytes(d16: torch.Tensor) -> torch.Tensor:
    # [..., 1] float16 -> [..., 2] uint8, little endian
    return d16.contiguous().view(torch.int16).view(torch.uint8).reshape(*d16.shape[:-1], 2)


def encode_q4_0(w: torch.Tensor) -> torch.Tensor:
    """Quantize fp32 weights [rows, K] to Q4_0 interchange bytes [rows, K/32*18].

    Per 32-weight block: take the element of largest magnitude (first one on ties),
    d = that element / -8, stored as binary16 (round to nearest even); the codes are
    chosen with the *stored* d: code = clamp(round_half_away(w / d) + 8, 0, 15).
    An all-zero block (or one whose d rounds to zero) gets d = +0 and codes 8.
    """
    rows, K = w.shape
    assert K % QK == 0, "K must be a multiple of 32"
    wb = w.to(torch.float32).reshape(rows, K // QK, QK)
    idx = wb.abs().argmax(dim=-1, keepdim=True)
    vmax = torch.gather(wb, -1, idx)
    d16 = (vmax / -8.0).to(torch.float16)
    dq = d16.to(torch.float32)
    zero = dq == 0
    d16 = torch.where(zero, torch.zeros_like(d16), d16)
    safe = torch.where(zero, torch.ones_like(dq), dq)
    code = (round_half_away(wb / safe) + 8).clamp(0, 15)
    code = torch.where(zero, torch.full_like(code, 8), code).to(torch.uint8)
    qs = code[..., :16] | (code[..., 16:] << 4)
    return torch.cat([_scale_bytes(d16), qs], dim=-1).reshape(rows, (K // QK) * Q4_0_BLOCK_BYTES)


def encode_q8_0(w: torch.Tensor) -> torch.Tensor:
    """Quantize fp32 weights [rows, K] to Q8_0 interchange bytes [rows, K/32*34].

    Per block: d = max|w| / 127 stored as binary16; code = clamp(round_half_away(w / d),
    -127, 127) with the stored d.  A zero block gets d = +0 and codes 0.
    """
    rows, K = w.shape
    assert K % QK == 0, "K must be a multiple of 32"
    wb = w.to(torch.float32).reshape(rows, K // QK, QK)
    amax = wb.abs().amax(dim=-1, keepdim=True)
    d16 = (amax / 127.0).to(torch.float16)
    dq = d16.to(torch.float32)
    zero = dq == 0
    d16 = torch.where(zero, torch.zeros_like(d16), d16)
    safe = torch.where(zero, torch.ones_like(dq), dq)
    code = round_half_away(wb / safe).clamp(-127, 127)
    code = torch.where(zero, torch.zeros_like(code), code).to(torch.int8)
    return torch.cat([_scale_bytes(d16), code.view(torch.uint8)], dim=-1).reshape(
        rows, (K // QK) * Q8_0_BLOCK_BYTES)


def _scales_from(values, shape, key, device):
    vals = torch.tensor(list(values), dtype=torch.float16, device=device)
    pick = torch.randint(0, len(vals), shape, generator=_gen(key + ("d",), device), device=device)
    return vals[pick].unsqueeze(-1)


def raw_q4_0(rows: int, K: int, key, scales=(0.5, 1.0, 2.0), codes=(0, 15), device="cpu"):
    """Q4_0 blocks with uniformly drawn codes in [codes[0], codes[1]] and scales drawn
    from a given set (exact-arithmetic probes use powers of two)."""
    nb = K // QK
    c = torch.randint(codes[0], codes[1] + 1, (rows, nb, QK), generator=_gen(key + ("q",), device),
                      device=device, dtype=torch.int32).to(torch.uint8)
    qs = c[..., :16] | (c[..., 16:] << 4)
    d16 = _scales_from(scales, (rows, nb), key, device)
    return torch.cat([_scale_bytes(d16), qs], dim=-1).reshape(rows, nb * Q4_0_BLOCK_BYTES)


def raw_q8_0(rows: int, K: int, key, scales=(0.5, 1.0, 2.0), codes=(-8, 8), device="cpu"):
    """Q8_0 blocks with codes uniform in [codes[0], codes[1]] and scales from a set."""
    nb = K // QK
    c = torch.randint(codes[0], codes[1] + 1, (rows, nb, QK), generator=_gen(key + ("q",), device),
                      device=device, dtype=torch.int32).to(torch.int8)
    d16 = _scales_from(scales, (rows, nb), key, device)
    return torch.cat([_scale_bytes(d16), c.view(torch.uint8)], dim=-1).reshape(rows, nb * Q8_0_BLOCK_BYTES)


def small_int(shape, key, lo: int = -8, hi: int = 8, device="cpu", dtype=torch.float32):
    """Integers uniform in [lo, hi] (as fp32 by default)."""
    return torch.randint(lo, hi + 1, tuple(shape), generator=_gen(key, device), device=device,
                         dtype=torch.int32).to(dtype)


def router_weights(T: int, top_k: int, key) -> np.ndarray:
    """Router weights [T, top_k] fp32: a softmax over top_k N(0, 1) draws per token, so
    each token's weights are positive and sum to about 1 (the usual normalised top-k
    gating; the pages give no weights of their own)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed_of(*key) & 0xFFFFFFFF, 7]))
    z = rng.standard_normal((T, top_k))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return np.ascontiguousarray((e / e.sum(axis=1, keepdims=True)).astype(np.float32))


def router_ids(T: int, E: int, top_k: int, key, s: float = 1.1) -> np.ndarray:
    """Expert ids [T, top_k] int32: top-k of N(0,1) router logits plus a skewed per-expert
    bias -s*ln(e+1) (the log of a Zipf(s) weight over expert rank e+1), in descending score
    order, ties to the lower expert index.  The skew makes some experts far more popular
    than others, as observed for MoE expert selection on the page "ik_llama.cpp 老工作站多
    GPU 部署 Qwen3-235B-A22B 实战指南" (nxmr.cn), section on general multi-GPU tuning.
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed_of(*key) & 0xFFFFFFFF]))
    logits = rng.standard_normal((T, E))
    bias = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    order = np.argsort(-(logits + bias), axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :top_k].astype(np.int32))
