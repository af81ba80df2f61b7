"""CPU emulation of the GEMV kernels' per-block arithmetic, in single precision.

The acceptance bound is |y - y_exact| <= 1e-3 * S per output with S = sum |w_i x_i|.  How
the fp32 sums are formed decides whether every input meets it:

- offset form: sum n_j x_j over the unsigned codes n (Q4_0 nibbles; Q8_0 codes + 128), then
  minus 8 * sum x_j (Q8_0: 128 * sum x_j).  Its rounding error grows with sum (n_j + 8)|x_j|,
  not with S, so a block whose codes are all near the offset can lose its whole value.
- signed form (what the kernels compute): each code is turned into its signed value
  (n - 8, or the int8 code) exactly before the multiply; every product is exact inside a
  fused multiply-add, so the block sum's error is at most 31 roundings of partial sums
  each bounded by sum |(n - 8) x|, i.e. well inside 1e-3 * S.

Block format: the Q4_0 / Q8_0 blocks of the format table of the page "V100跑Qwen 27B：量化与
KV Cache调优，从4到64 tok/s" (lmnt.cn), section 4.1: 32 weights and one binary16 scale d, a
Q4_0 weight (nibble - 8) d, a Q8_0 weight int8 d.  No GPU here: this pins the reasoning
behind the kernels' arithmetic, not the kernels.
"""
import numpy as np

f32 = np.float32


def fma32(a, b, c):
    """Single-precision fused multiply-add: the product exact, one rounding (emulated in
    double: a code times an fp32 value is exact there; the sum can double-round only in
    rare last-bit ties, immaterial at the 1e-3 scale)."""
    return f32(np.float64(a) * np.float64(b) + np.float64(c))


def offset_form_q4(codes, x, d):
    """The offset form over one Q4_0 block: two chains of sixteen (low nibbles against x,
    high nibbles taken as 16 n against x / 16), their sum, minus 8 times the block's input
    sum formed in the same order, times d."""
    x = x.astype(f32)
    h0 = f32(f32(codes[0]) * x[0])
    for j in range(1, 16):
        h0 = fma32(codes[j], x[j], h0)
    xs = (x[16:] * f32(0.0625)).astype(f32)
    h1 = f32(f32(16 * codes[16]) * xs[0])
    for j in range(1, 16):
        h1 = fma32(16 * codes[16 + j], xs[j], h1)
    c = f32(h0 + h1)
    s0 = x[0]
    for j in range(1, 16):
        s0 = f32(s0 + x[j])
    s1 = f32(xs[0] * f32(16))
    for j in range(1, 16):
        s1 = f32(s1 + f32(xs[j] * f32(16)))
    sx = f32(s0 + s1)
    r = fma32(-8, sx, c)
    return f32(np.float64(d) * np.float64(r))


def signed_form(codes_signed, x, d):
    """The signed form over one block: one chain over positions 0..31 of (signed code) * x,
    each step a fused multiply-add, then d times the sum (also fused: acc + d * c)."""
    x = x.astype(f32)
    c = f32(f32(codes_signed[0]) * x[0])
    for j in range(1, 32):
        c = fma32(codes_signed[j], x[j], c)
    return fma32(d, c, f32(0))


def exact(codes_signed, x, d):
    p = np.asarray(codes_signed, np.float64) * np.float64(d) * x.astype(np.float64)
    return p.sum(), np.abs(p).sum()


def _near_neutral_cases(n_blocks, seed, fmt):
    """Blocks whose codes are all the offset except a few +-1, placed on small inputs,
    with large inputs elsewhere (the adversarial case for the offset form)."""
    rng = np.random.default_rng(seed)
    for _ in range(n_blocks):
        x = rng.uniform(1.0, 300.0, 32) * rng.choice([-1.0, 1.0], 32)
        k = rng.integers(1, 4)
        pos = rng.choice(32, size=k, replace=False)
        x[pos] = rng.uniform(1e-3, 1.0, k) * rng.choice([-1.0, 1.0], k)
        s = np.zeros(32, np.int64)
        s[pos] = rng.choice([-1, 1], k)
        yield s, x.astype(f32), 1.0 if fmt == "q4_0" else 0.5


def test_offset_form_loses_a_near_neutral_block():
    """d = 1, every nibble 8 except a 9 on the input 1e-3, inputs 100 elsewhere: the exact
    block value is 1e-3; the offset form returns 0 (an error of 100 % of S)."""
    codes = np.full(32, 8, np.int64)
    codes[3] = 9
    x = np.full(32, 100.0, f32)
    x[3] = f32(1e-3)
    y_exact, S = exact(codes - 8, x, 1.0)
    y_off = offset_form_q4(codes, x, 1.0)
    assert abs(float(y_off) - y_exact) > 1e-3 * S  # the bound is broken
    assert float(y_off) == 0.0
    y_sig = signed_form(codes - 8, x, 1.0)
    assert abs(float(y_sig) - y_exact) <= 1e-6 * S


def test_offset_form_breaks_bound_signed_form_meets_it():
    """2000 near-neutral blocks with inputs spanning 1e-3..300: the offset form breaks the
    bound on some; the signed form keeps every block within 2^-19 S (31 roundings)."""
    bad_offset, worst_signed = 0, 0.0
    for s, x, d in _near_neutral_cases(2000, 11, "q4_0"):
        y_exact, S = exact(s, x, d)
        if abs(float(offset_form_q4(s + 8, x, d)) - y_exact) > 1e-3 * S:
            bad_offset += 1
        worst_signed = max(worst_signed, abs(float(signed_form(s, x, d)) - y_exact) / S)
    assert bad_offset > 0
    assert worst_signed <= 2.0 ** -19


def test_signed_form_q8_extremes():
    """Q8_0 blocks with codes -128..127 (including -128, which the kernels accept) and
    near-neutral codes on mixed-magnitude inputs: within 2^-19 S."""
    rng = np.random.default_rng(5)
    worst = 0.0
    for i in range(500):
        if i % 2:
            s = rng.integers(-128, 128, 32)
            s[0] = -128
        else:
            s = np.zeros(32, np.int64)
            s[rng.integers(0, 32)] = rng.choice([-1, 1])
        x = (rng.uniform(1e-3, 300.0, 32) * rng.choice([-1.0, 1.0], 32)).astype(f32)
        y_exact, S = exact(s, x, 0.25)
        worst = max(worst, abs(float(signed_form(s, x, 0.25)) - y_exact) / S)
    assert worst <= 2.0 ** -19


def test_signed_form_neutral_block_is_exactly_zero():
    """All codes equal to the offset give a signed chain of exact zeros: y = 0 exactly."""
    x = np.random.default_rng(2).standard_normal(32).astype(f32) * f32(1e6)
    assert float(signed_form(np.zeros(32, np.int64), x, 3.0)) == 0.0


def test_q4_nibble_to_half_pairs():
    """The kernels turn nibbles into signed binary16 values without a conversion
    instruction: a nibble n OR-ed into the mantissa of 1024.0 (0x6400) reads as 1024 + n,
    and a nibble sitting at bits 4..7 OR-ed into 64.0 (0x5400) reads as 64 + n (the
    mantissa step there is 1/16); subtracting 1032 and 72 gives n - 8 exactly."""
    n = np.arange(16, dtype=np.uint16)
    lo = (np.uint16(0x6400) | n).view(np.float16).astype(np.float64) - 1032.0
    hi = (np.uint16(0x5400) | (n << np.uint16(4))).view(np.float16).astype(np.float64) - 72.0
    assert np.array_equal(lo, n - 8.0) and np.array_equal(hi, n - 8.0)
    # the subtraction itself is exact in binary16 (integers below 2048)
    assert np.array_equal((np.uint16(0x6400) | n).view(np.float16) - np.float16(1032),
                          (n.astype(np.float64) - 8).astype(np.float16))
