"""Planted-mistake check: each plausible slip in the oracle, compiled on the CPU from a
modified copy of oracle.c, must make the pin suite fail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "nibble_halves_swapped": [("int lo = qs[j] & 0x0f;", "int lo = (qs[j] >> 4) & 0x0f;"),
                              ("int hi = (qs[j] >> 4) & 0x0f;", "int hi = qs[j] & 0x0f;")],
    "q4_offset_dropped": [("(double)(lo - 8) * d", "(double)(lo) * d")],
    "q8_codes_unsigned": [("(double)(int8_t)qs[j] * d", "(double)qs[j] * d")],
    "half_exponent_bias": [("e - 25", "e - 24")],
    "x_transposed": [("w[k] * (double)X[m * K + k]", "w[k] * (double)X[k * M + m]")],
    "qmm_block_scale_index": [("(double)dx[m * nb + b]", "(double)dx[m * nb]")],
    "qmm_codes_unsigned": [("acc += (int32_t)qw[j] * (int32_t)qx[j];",
                            "acc += (int32_t)(uint8_t)qw[j] * (int32_t)qx[j];")],
    "qmm_q4_offset_dropped": [("const int32_t lo = (qs[j] & 0x0f) - 8, hi = ((qs[j] >> 4) & 0x0f) - 8;",
                               "const int32_t lo = (qs[j] & 0x0f), hi = ((qs[j] >> 4) & 0x0f);")],
    "qmm_q4_halves_swapped": [("lo * (int32_t)qx[j] + hi * (int32_t)qx[j + 16]",
                               "hi * (int32_t)qx[j] + lo * (int32_t)qx[j + 16]")],
    "qmm_id_slot_row": [("const int64_t r = t * x_tok_rows + s * x_slot_rows;",
                         "const int64_t r = t * x_tok_rows;")],
    "qmm_id_expert_offset": [("W + (int64_t)e * N * row_bytes;", "W + (int64_t)e * row_bytes;")],
    "act_round_to_even": [("roundf(x[j] / d)", "rintf(x[j] / d)")],
    "act_signed_max": [("float v = fabsf(x[j]);", "float v = x[j];")],
    "id_slot_stride": [("s * x_slot_stride", "t * x_slot_stride")],
    "id_padding_ignored": [("if (e >= 0) {", "if (1) { const int32_t ee = e < 0 ? 0 : e; (void)ee;")],
    "sum_unweighted": [("y += r * ys;", "y += ys;")],
    "sum_weight_index": [("(double)weights[t * top_k + s]", "(double)weights[s]")],
    "silu_sign": [("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));")],
    "gate_up_swapped": [("y = sl * u;", "y = oracle_silu(u) * g;")],
    # the tolerance scales S, which set the acceptance bar of the GPU parity tests
    "qmv_scale_x10": [("        s += fabs(p);", "        s += 10 * fabs(p);")],
    "id_scale_x10": [("sa += fabs(p);", "sa += 10 * fabs(p);")],
    "sum_scale_weight_signed": [("sa += fabs(r) * ss;", "sa += r * ss;")],
    "qmm_scale_x10": [("sa += fabs(scale) * (double)aabs;", "sa += 10 * fabs(scale) * (double)aabs;")],
    "qmm_scale_signed": [("sa += fabs(scale) * (double)aabs;", "sa += scale * (double)aabs;")],
    "qmm_scale_abs_sums_multiplied": [
        ("int32_t acc = 0, aabs = 0;", "int32_t acc = 0, aabs = 0, aw = 0, ax = 0;"),
        ("aabs += abs((int32_t)qw[j] * (int32_t)qx[j]);",
         "aw += abs((int32_t)qw[j]); ax += abs((int32_t)qx[j]); aabs = aw * ax;")],
    "gate_up_scale_gate_term_dropped": [
        ("sy = 1.1 * sg * (fabs(u) + 1e-3 * su) + fabs(sl) * su + 1e-3 * fabs(y);",
         "sy = fabs(sl) * su + 1e-3 * fabs(y);")],
    "gate_up_scale_x10": [
        ("sy = 1.1 * sg * (fabs(u) + 1e-3 * su) + fabs(sl) * su + 1e-3 * fabs(y);",
         "sy = 10 * (1.1 * sg * (fabs(u) + 1e-3 * su) + fabs(sl) * su + 1e-3 * fabs(y));")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor missing: {old}"
        src = src.replace(old, new)
    if name == "id_padding_ignored":
        src = src.replace("W + ((int64_t)e * N + n) * row_bytes", "W + ((int64_t)(e < 0 ? 0 : e) * N + n) * row_bytes")
        for t in ("Wg", "Wu"):
            src = src.replace(f"{t} + ((int64_t)e * N + n) * row_bytes",
                              f"{t} + ((int64_t)(e < 0 ? 0 : e) * N + n) * row_bytes")
    c = tmp_path / "mutant.c"
    c.write_text(src)
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(so), str(c), "-lm"], check=True)
    env = dict(os.environ, BQM_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
