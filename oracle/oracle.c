/*
 * oracle.c - plain, slow CPU oracle for block-quantized matrix products.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header, table or
 * helper with the GPU library; it reads the *interchange* block layout directly.
 *
 * What is computed (each function below restates its definition):
 *   - Q4_0 / Q8_0 are the block formats named in the format table of the page
 *     "V100跑Qwen 27B：量化与KV Cache调优，从4到64 tok/s" (lmnt.cn), section 4.1.
 *     A block holds 32 weights and one binary16 scale d; a Q4_0 weight is
 *     (nibble - 8) * d and a Q8_0 weight is int8 * d.  The page names the formats
 *     only; the ggml byte layout is used (scale first, little endian; Q4_0 byte j
 *     holds weight j in its low nibble and weight j+16 in its high nibble).
 *   - The decode product y = dequant(W) x streams every weight once per token; the
 *     same page, section 1.2, explains why that makes decode bandwidth-bound.
 *   - The expert-indexed product follows the description of mul_mat_id on the page
 *     "ik_llama.cpp 老工作站多 GPU 部署 Qwen3-235B-A22B 实战指南" (nxmr.cn), background
 *     and split-mode sections: a 3D expert tensor and per-token expert ids.
 *
 * Floating point: every weight and product is formed exactly in fp64 (a binary16
 * scale times a small integer times an fp32 input needs at most 11+8+24 bits) and
 * sums are accumulated in fp64 in index order.  The activation quantizer is the one
 * fp32 routine: it must take the same integer decisions as the GPU, in IEEE single
 * precision (build with -ffp-contract=off, no fast-math).
 *
 * Parallelism: OpenMP over independent outputs only; every single output is a
 * sequential sum, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_Q4_0 2
#define ORACLE_Q8_0 8

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* IEEE 754 binary16 -> double, by definition: sign s, 5-bit exponent e, 10-bit
 * fraction f.  e == 0: (-1)^s * f * 2^-24 (zero and subnormals);
 * 1 <= e <= 30: (-1)^s * (1024 + f) * 2^(e - 25);  e == 31: infinity or NaN. */
double oracle_half_to_double(uint16_t h) {
  int s = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double mag;
  if (e == 0)
    mag = ldexp((double)f, -24);
  else if (e < 31)
    mag = ldexp((double)(1024 + f), e - 25);
  else
    mag = f ? NAN : INFINITY;
  return s ? -mag : mag;
}

static int block_bytes(int fmt) { return fmt == ORACLE_Q4_0 ? 18 : 34; }

/* Dequantize one row of K weights (K/32 interchange blocks) into w[0..K-1]. */
int oracle_decode_row(int fmt, const uint8_t* blocks, int64_t K, double* w) {
  if (K % 32 != 0 || (fmt != ORACLE_Q4_0 && fmt != ORACLE_Q8_0)) return -1;
  const int bb = block_bytes(fmt);
  for (int64_t b = 0; b < K / 32; b++) {
    const uint8_t* blk = blocks + b * bb;
    double d = oracle_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    const uint8_t* qs = blk + 2;
    if (fmt == ORACLE_Q4_0) {
      for (int j = 0; j < 16; j++) {
        int lo = qs[j] & 0x0f;        /* weight j      */
        int hi = (qs[j] >> 4) & 0x0f; /* weight j + 16 */
        w[32 * b + j] = (double)(lo - 8) * d;
        w[32 * b + 16 + j] = (double)(hi - 8) * d;
      }
    } else {
      for (int j = 0; j < 32; j++) w[32 * b + j] = (double)(int8_t)qs[j] * d;
    }
  }
  return 0;
}

/* Y[m][n] = sum_k w[n][k] * X[m][k]  (W is [N][K] in blocks, X is [M][K] fp32)
 * S[m][n] = sum_k |w[n][k] * X[m][k]|  (the scale of the acceptance bound). */
int oracle_qmv(int fmt, const uint8_t* W, const float* X, int64_t M, int64_t N, int64_t K,
               double* Y, double* S) {
  if (K % 32 != 0 || (fmt != ORACLE_Q4_0 && fmt != ORACLE_Q8_0)) return -1;
  const int64_t row_bytes = (K / 32) * block_bytes(fmt);
  int err = 0;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t n = 0; n < N; n++) {
    double* w = (double*)malloc((size_t)K * sizeof(double));
    if (!w) { err = -2; continue; }
    oracle_decode_row(fmt, W + n * row_bytes, K, w);
    for (int64_t m = 0; m < M; m++) {
      double y = 0.0, s = 0.0;
      for (int64_t k = 0; k < K; k++) {
        double p = w[k] * (double)X[m * K + k];
        y += p;
        s += fabs(p);
      }
      Y[m * N + n] = y;
      if (S) S[m * N + n] = s;
    }
    free(w);
  }
  return err;
}

/* Expert-indexed product.  W holds E matrices [N][K] back to back (expert e starts at
 * e * N * row_bytes).  For token t and slot s: e = ids[t][s]; a negative id is a
 * padding slot whose output row is zero; otherwise
 *   Y[t][s][n] = sum_k w_e[n][k] * X[t * x_tok_stride + s * x_slot_stride + k]. */
int oracle_qmv_id(int fmt, const uint8_t* W, int64_t E, int64_t N, int64_t K,
                  const int32_t* ids, int64_t T, int64_t top_k, const float* X,
                  int64_t x_tok_stride, int64_t x_slot_stride, double* Y, double* S) {
  if (K % 32 != 0 || (fmt != ORACLE_Q4_0 && fmt != ORACLE_Q8_0)) return -1;
  const int64_t row_bytes = (K / 32) * block_bytes(fmt);
  for (int64_t i = 0; i < T * top_k; i++)
    if (ids[i] >= E) return -3;
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int64_t ts = 0; ts < T * top_k; ts++) {
    for (int64_t n = 0; n < N; n++) {
      const int64_t t = ts / top_k, s = ts % top_k;
      const int32_t e = ids[ts];
      double y = 0.0, sa = 0.0;
      if (e >= 0) {
        double* w = (double*)malloc((size_t)K * sizeof(double));
        if (!w) { err = -2; continue; }
        oracle_decode_row(fmt, W + ((int64_t)e * N + n) * row_bytes, K, w);
        const float* x = X + t * x_tok_stride + s * x_slot_stride;
        for (int64_t k = 0; k < K; k++) {
          double p = w[k] * (double)x[k];
          y += p;
          sa += fabs(p);
        }
        free(w);
      }
      Y[ts * N + n] = y;
      if (S) S[ts * N + n] = sa;
    }
  }
  return err;
}

/* Output of a mixture-of-experts layer over the routed experts: for token t and row n,
 *     Y[t][n] = sum_s weights[t][s] * (sum_k W[e][n][k] x_ts[k]),   e = ids[t][s] >= 0,
 * each expert product in double over the exactly dequantized weights in index order, the
 * slots added in order; a padding slot (negative id) adds nothing.  S[t][n] =
 * sum_s |weights[t][s]| * sum_k |W[e][n][k] x_ts[k]|, the tolerance scale. */
int oracle_qmv_id_sum(int fmt, const uint8_t* W, int64_t E, int64_t N, int64_t K,
                      const int32_t* ids, const float* weights, int64_t T, int64_t top_k,
                      const float* X, int64_t x_tok_stride, int64_t x_slot_stride, double* Y,
                      double* S) {
  if (K % 32 != 0 || (fmt != ORACLE_Q4_0 && fmt != ORACLE_Q8_0)) return -1;
  const int64_t row_bytes = (K / 32) * block_bytes(fmt);
  for (int64_t i = 0; i < T * top_k; i++)
    if (ids[i] >= E) return -3;
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int64_t t = 0; t < T; t++) {
    for (int64_t n = 0; n < N; n++) {
      double y = 0.0, sa = 0.0;
      double* w = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
      if (!w) { err = -2; continue; }
      for (int64_t s = 0; s < top_k; s++) {
        const int32_t e = ids[t * top_k + s];
        if (e < 0) continue;
        oracle_decode_row(fmt, W + ((int64_t)e * N + n) * row_bytes, K, w);
        const float* x = X + t * x_tok_stride + s * x_slot_stride;
        double ys = 0.0, ss = 0.0;
        for (int64_t k = 0; k < K; k++) {
          double p = w[k] * (double)x[k];
          ys += p;
          ss += fabs(p);
        }
        const double r = (double)weights[t * top_k + s];
        y += r * ys;
        sa += fabs(r) * ss;
      }
      free(w);
      Y[t * N + n] = y;
      if (S) S[t * N + n] = sa;
    }
  }
  return err;
}

/* silu(z) = z / (1 + e^-z), in double precision. */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* Fused expert gate+up (the fused MoE path of the ik_llama.cpp MoE page, recommended-
 * command section, read as the SwiGLU feed-forward): per slot (t, s) with expert
 * e = ids[t][s] >= 0 and row n,
 *     g = sum_k Wg[e][n][k] x[k],  u = sum_k Wu[e][n][k] x[k],  Y = silu(g) * u,
 * each sum in double over the exactly dequantized weights in index order.  A padding slot
 * gives 0.  S is the tolerance scale for |y - Y| <= 1e-3 S: with |dg| <= 1e-3 Sg and
 * |du| <= 1e-3 Su (the bar of each sum, Sg = sum |wg x|, Su = sum |wu x|) and |silu'| <= 1.1,
 *     |silu(g + dg)(u + du) - silu(g) u| <= 1.1 |dg| (|u| + |du|) + |silu(g)| |du|,
 * so S = 1.1 Sg (|u| + 1e-3 Su) + |silu(g)| Su, plus 1e-3 |Y| for the single-precision
 * evaluation of silu and the product. */
int oracle_qmv_id_gate_up(int fmt, const uint8_t* Wg, const uint8_t* Wu, int64_t E, int64_t N,
                          int64_t K, const int32_t* ids, int64_t T, int64_t top_k,
                          const float* X, int64_t x_tok_stride, int64_t x_slot_stride,
                          double* Y, double* S) {
  if (K % 32 != 0 || (fmt != ORACLE_Q4_0 && fmt != ORACLE_Q8_0)) return -1;
  const int64_t row_bytes = (K / 32) * block_bytes(fmt);
  for (int64_t i = 0; i < T * top_k; i++)
    if (ids[i] >= E) return -3;
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int64_t ts = 0; ts < T * top_k; ts++) {
    for (int64_t n = 0; n < N; n++) {
      const int64_t t = ts / top_k, s = ts % top_k;
      const int32_t e = ids[ts];
      double y = 0.0, sy = 0.0;
      if (e >= 0) {
        double* w = (double*)malloc((size_t)2 * K * sizeof(double));
        if (!w) { err = -2; continue; }
        oracle_decode_row(fmt, Wg + ((int64_t)e * N + n) * row_bytes, K, w);
        oracle_decode_row(fmt, Wu + ((int64_t)e * N + n) * row_bytes, K, w + K);
        const float* x = X + t * x_tok_stride + s * x_slot_stride;
        double g = 0.0, u = 0.0, sg = 0.0, su = 0.0;
        for (int64_t k = 0; k < K; k++) {
          const double pg = w[k] * (double)x[k], pu = w[K + k] * (double)x[k];
          g += pg;
          u += pu;
          sg += fabs(pg);
          su += fabs(pu);
        }
        free(w);
        const double sl = oracle_silu(g);
        y = sl * u;
        sy = 1.1 * sg * (fabs(u) + 1e-3 * su) + fabs(sl) * su + 1e-3 * fabs(y);
      }
      Y[ts * N + n] = y;
      if (S) S[ts * N + n] = sy;
    }
  }
  return err;
}

/* Activation quantizer for the prefill product, per row m and 32-wide block b, in
 * IEEE single precision:
 *   a  = max_j |x_j|;  dx = a / 127 (correctly rounded division);
 *   dx == 0: every code 0 and dx = +0;
 *   else  q_j = round_half_away_from_zero(x_j / dx) clamped to [-127, 127]. */
int oracle_quantize_q8_act(const float* X, int64_t M, int64_t K, int8_t* Xq, float* dx) {
  if (K % 32 != 0) return -1;
  const int64_t nb = K / 32;
#pragma omp parallel for
  for (int64_t m = 0; m < M; m++) {
    for (int64_t b = 0; b < nb; b++) {
      const float* x = X + m * K + 32 * b;
      float a = 0.0f;
      for (int j = 0; j < 32; j++) {
        float v = fabsf(x[j]);
        if (v > a) a = v;
      }
      float d = a / 127.0f;
      dx[m * nb + b] = d == 0.0f ? 0.0f : d;
      for (int j = 0; j < 32; j++) {
        int q = 0;
        if (d != 0.0f) {
          float r = roundf(x[j] / d);
          if (r > 127.0f) r = 127.0f;
          if (r < -127.0f) r = -127.0f;
          q = (int)r;
        }
        Xq[m * K + 32 * b + j] = (int8_t)q;
      }
    }
  }
  return 0;
}

/* Prefill product with Q8_0 weights and block-quantized activations:
 *   isum[m][n][b] = sum_{j<32} qw[n][32b+j] * qx[m][32b+j]            (exact int32)
 *   Y[m][n]       = sum_b d_w[n][b] * dx[m][b] * isum[m][n][b]          (fp64)
 *   S[m][n]       = sum_b |d_w[n][b] * dx[m][b]| * sum_j |qw * qx|      (bound scale)
 * isum may be NULL; otherwise it is [M][N][K/32]. */
int oracle_qmm_q8_0(const uint8_t* W, const int8_t* Xq, const float* dx, int64_t M, int64_t N,
                    int64_t K, int32_t* isum, double* Y, double* S) {
  if (K % 32 != 0) return -1;
  const int64_t nb = K / 32;
  const int64_t row_bytes = nb * 34;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; m++) {
    for (int64_t n = 0; n < N; n++) {
      double y = 0.0, sa = 0.0;
      for (int64_t b = 0; b < nb; b++) {
        const uint8_t* blk = W + n * row_bytes + b * 34;
        double dw = oracle_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
        const int8_t* qw = (const int8_t*)(blk + 2);
        const int8_t* qx = Xq + m * K + 32 * b;
        int32_t acc = 0, aabs = 0;
        for (int j = 0; j < 32; j++) {
          acc += (int32_t)qw[j] * (int32_t)qx[j];
          aabs += abs((int32_t)qw[j] * (int32_t)qx[j]);
        }
        if (isum) isum[(m * N + n) * nb + b] = acc;
        double scale = dw * (double)dx[m * nb + b];
        y += scale * (double)acc;
        sa += fabs(scale) * (double)aabs;
      }
      Y[m * N + n] = y;
      if (S) S[m * N + n] = sa;
    }
  }
  return 0;
}

/* Prefill product with Q4_0 weights: the same definition as oracle_qmm_q8_0 with the
 * weight codes q - 8 (q the nibble; weight j of a block in the low nibble of byte j,
 * weight j + 16 in the high one):
 *   isum[m][n][b] = sum_j (q[n][32b+j] - 8) * Xq[m][32b+j]   (exact int32)
 *   Y[m][n]       = sum_b (double)d_w[n][b] * (double)dx[m][b] * isum[m][n][b]. */
int oracle_qmm_q4_0(const uint8_t* W, const int8_t* Xq, const float* dx, int64_t M, int64_t N,
                    int64_t K, int32_t* isum, double* Y, double* S) {
  if (K % 32 != 0) return -1;
  const int64_t nb = K / 32;
  const int64_t row_bytes = nb * 18;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; m++) {
    for (int64_t n = 0; n < N; n++) {
      double y = 0.0, sa = 0.0;
      for (int64_t b = 0; b < nb; b++) {
        const uint8_t* blk = W + n * row_bytes + b * 18;
        double dw = oracle_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
        const uint8_t* qs = blk + 2;
        const int8_t* qx = Xq + m * K + 32 * b;
        int32_t acc = 0, aabs = 0;
        for (int j = 0; j < 16; j++) {
          const int32_t lo = (qs[j] & 0x0f) - 8, hi = ((qs[j] >> 4) & 0x0f) - 8;
          acc += lo * (int32_t)qx[j] + hi * (int32_t)qx[j + 16];
          aabs += abs(lo * (int32_t)qx[j]) + abs(hi * (int32_t)qx[j + 16]);
        }
        if (isum) isum[(m * N + n) * nb + b] = acc;
        double scale = dw * (double)dx[m * nb + b];
        y += scale * (double)acc;
        sa += fabs(scale) * (double)aabs;
      }
      Y[m * N + n] = y;
      if (S) S[m * N + n] = sa;
    }
  }
  return 0;
}

/* Expert-indexed prefill product (the prefill counterpart of oracle_qmv_id): for slot
 * (t, s) with expert e = ids[t][s] >= 0 and input row r = t * x_tok_rows + s * x_slot_rows
 * of the quantized activations, the prefill product of that one row with expert e's
 * N x K matrix (oracle_qmm_q8_0 / oracle_qmm_q4_0 with M = 1):
 *   Y[t][s][n] = sum_b d_w[e][n][b] * dx[r][b] * sum_j qw[e][n][32b+j] * Xq[r][32b+j].
 * A padding slot (negative id) gives a zero row; an id >= E is rejected. */
int oracle_qmm_id(int fmt, const uint8_t* W, int64_t E, int64_t N, int64_t K, const int32_t* ids,
                  int64_t T, int64_t top_k, const int8_t* Xq, const float* dx, int64_t x_tok_rows,
                  int64_t x_slot_rows, double* Y, double* S) {
  if (K % 32 != 0 || (fmt != ORACLE_Q4_0 && fmt != ORACLE_Q8_0)) return -1;
  const int64_t nb = K / 32, row_bytes = nb * block_bytes(fmt);
  for (int64_t i = 0; i < T * top_k; i++)
    if (ids[i] >= E) return -3;
  for (int64_t ts = 0; ts < T * top_k; ts++) {
    const int64_t t = ts / top_k, s = ts % top_k;
    const int32_t e = ids[ts];
    double* y = Y + ts * N;
    double* sa = S ? S + ts * N : NULL;
    if (e < 0) {
      for (int64_t n = 0; n < N; n++) {
        y[n] = 0.0;
        if (sa) sa[n] = 0.0;
      }
      continue;
    }
    const int64_t r = t * x_tok_rows + s * x_slot_rows;
    const uint8_t* We = W + (int64_t)e * N * row_bytes;
    const int st = fmt == ORACLE_Q8_0 ? oracle_qmm_q8_0(We, Xq + r * K, dx + r * nb, 1, N, K, NULL, y, sa)
                                      : oracle_qmm_q4_0(We, Xq + r * K, dx + r * nb, 1, N, K, NULL, y, sa);
    if (st != 0) return st;
  }
  return 0;
}
