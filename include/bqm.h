/*
 * bqm.h - block-quantized matrix products on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What the library computes.  Decode streams every weight once per token, so its
 * speed is set by how many weight bytes cross HBM ("V100跑Qwen 27B：量化与KV Cache调优，
 * 从4到64 tok/s", lmnt.cn, section 1.2); the compact block formats Q4_0 and Q8_0 named
 * in that page's format table (section 4.1) cut those bytes.  Every product here is
 *     y = dequant(W) . x
 * with W stored in 32-weight blocks that each carry one binary16 scale d:
 *     Q4_0 weight = (nibble - 8) * d        Q8_0 weight = int8 * d.
 *
 * Interchange block layout (host or device bytes, what bqm_repack reads):
 *     Q4_0: 18 bytes per block = binary16 d (little endian), then 16 bytes; byte j
 *           holds weight j in its low nibble and weight j+16 in its high nibble.
 *     Q8_0: 34 bytes per block = binary16 d, then 32 signed bytes (weight j = byte j).
 *     A matrix W[N][K] is N rows of K/32 consecutive blocks.
 * The pages name the formats but do not print their bytes; this is the ggml layout.
 *
 * Packed (device) layout, what the products read: produced by bqm_repack, opaque to
 * callers except for its size, bqm_packed_bytes().  It separates the 16-byte aligned
 * code bytes from the scales so that every code load is a full 16-byte load.
 *
 * Conventions shared by every call:
 *   - Pointers are DEVICE pointers unless stated; the caller owns all memory.  The
 *     library allocates nothing and frees nothing (qmv_id_sum_noalloc keeps its slot rows
 *     in a fixed device array that is part of the library); work is queued on `stream` (a HIP
 *     stream; 0 = the null stream) and the call returns without synchronizing (only
 *     bqm_chain_prepare and bqm_chain_status wait, as their entries say).
 *   - Argument errors are found on the host before anything is launched: the call
 *     returns a non-zero bqm_status and leaves every output untouched.  A failed launch
 *     returns BQM_E_LAUNCH.  Faults inside a kernel surface at the caller's next
 *     synchronization, as for any HIP kernel.
 *   - Sizes may be zero (nothing is launched, except that N > 0 with K = 0 writes
 *     zeros, the value of an empty sum).  K must be a multiple of 32.
 *   - Pointers passed to the products must be 16-byte aligned (torch allocations are).
 *   - Outputs must not alias inputs.  Results are deterministic: no atomic updates of
 *     data, a fixed summation order, the same bits on every run with the same launch.
 *   - Host-side state, all safe to use from several threads: per device, the compute-unit
 *     count and the device address of qmv_id_sum_noalloc's array (cached once); per kernel,
 *     whether its static local memory fits (checked once); per workspace prepared by
 *     bqm_chain_prepare, whether the chain has a waiting GEMV (under a mutex).
 *   - Floating-point outputs are fp32 and satisfy, per output,
 *         |y - y_exact| <= 1e-3 * sum_i |w_i * x_i|
 *     (y_exact in exact arithmetic); integer and byte outputs are exact.
 */
#ifndef BQM_H
#define BQM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BQM_OK = 0,
  BQM_E_NULL = 1,        /* a required pointer is NULL                          */
  BQM_E_SHAPE = 2,       /* negative size, K % 32 != 0, or a size over a limit  */
  BQM_E_ALIGN = 3,       /* a pointer is not 16-byte aligned                    */
  BQM_E_UNSUPPORTED = 4, /* unknown format code                                 */
  BQM_E_LAUNCH = 5       /* the HIP runtime refused a launch                    */
} bqm_status;

typedef enum { BQM_Q4_0 = 2, BQM_Q8_0 = 8 } bqm_fmt;

/* Largest M accepted by qmv_q4_0 / qmv_q8_0, the small-batch decode width. */
#define BQM_QMV_MAX_M 8
/* Limits of qmv_id: token count, experts per token, number of experts (the per-expert
 * slot tables are built in LDS). */
#define BQM_QMV_ID_MAX_T 64
#define BQM_QMV_ID_MAX_TOPK 32
#define BQM_QMV_ID_MAX_E 4096
/* Token limit of qmm_id (top_k and E as for qmv_id). */
#define BQM_QMM_ID_MAX_T 16384

/* Bytes of the packed layout of a rows x K matrix in format fmt (0 for an unknown
 * format or a K that is not a multiple of 32).  Host function, no device work. */
size_t bqm_packed_bytes(int fmt, int64_t rows, int64_t K);

/* One-time layout transform: interchange blocks (w_interchange, rows x K/32 blocks,
 * 2-byte aligned) -> packed layout (w_packed, bqm_packed_bytes(fmt, rows, K) bytes,
 * 16-byte aligned).  Every byte of the packed buffer is written.  Precedent: weights
 * re-laid out once for the unit that runs them, like the interleaved repack on the page
 * "ik_llama.cpp 老工作站多 GPU 部署 Qwen3-235B-A22B 实战指南" (nxmr.cn), section on -rtr. */
int bqm_repack(int fmt, const void* w_interchange, void* w_packed, int64_t rows, int64_t K,
               hipStream_t stream);

/* Inverse of bqm_repack (packed -> interchange), byte exact.  For tests and export. */
int bqm_unpack(int fmt, const void* w_packed, void* w_interchange, int64_t rows, int64_t K,
               hipStream_t stream);

/* Decode GEMV and small-batch GEMV ("V100跑Qwen 27B" page, section 1.2: every weight read
 * once per token):
 *     Y[m][n] = sum_k dequant(W)[n][k] * X[m][k],   0 <= m < M <= 8, 0 <= n < N.
 * w_packed: packed N x K matrix.  X: fp32 [M][K] row-major.  Y: fp32 [M][N] row-major.
 * M = 0 or N = 0: nothing to do.  M > 8, or one workgroup's share of the rows reaching
 * 2 GiB of codes: BQM_E_SHAPE.  (A chain of one GEMV: see qmv_chain.) */
int qmv_q4_0(const void* w_packed, const float* X, float* Y, int M, int64_t N, int64_t K,
             hipStream_t stream);
int qmv_q8_0(const void* w_packed, const float* X, float* Y, int M, int64_t N, int64_t K,
             hipStream_t stream);

/* Expert-indexed GEMV, the mul_mat_id of the page "ik_llama.cpp 老工作站多 GPU 部署
 * Qwen3-235B-A22B 实战指南" (nxmr.cn), background and split-mode sections: a 3D expert
 * tensor W[E][N][K] and per-token expert ids.
 *     e = ids[t][s];  Y[t][s][n] = sum_k dequant(W)[e][n][k] * x_ts[k]
 *     x_ts = X + t * x_tok_stride + s * x_slot_stride      (strides in floats)
 * x_slot_stride = 0 broadcasts one input per token (gate/up projections); = K gives each
 * slot its own input (down projection).  A negative id marks a padding slot: its Y row is
 * written with zeros.  An id >= E is a contract violation: its Y row is filled with NaN
 * and nothing outside the arrays is read.  Each selected expert's rows are streamed once
 * per group of the slots routed to it: groups of up to 4 (fp32 vector products), or from
 * T >= 8 tokens with K a multiple of 128 groups of up to 16 (bf16 matrix-core products with
 * each input split into two bf16 parts but for a remainder below 2^-14 |x|; the result
 * meets the same 1e-3 * sum |w x| bound for inputs below 2^86 in magnitude).
 * w_packed: the expert tensor packed as ONE matrix of E*N rows (bqm_repack with
 * rows = E*N).  ids: int32 [T][top_k], device memory.  Y: fp32 [T][top_k][N].
 * fmt: BQM_Q4_0 or BQM_Q8_0.  Limits: T <= 64, top_k <= 32, E <= 4096. */
int qmv_id(int fmt, const void* w_packed, int E, int64_t N, int64_t K, const int32_t* ids, int T,
           int top_k, const float* X, int64_t x_tok_stride, int64_t x_slot_stride, float* Y,
           hipStream_t stream);

/* Fused expert gate+up, the fused MoE path (`-fmoe`, `fused_moe 1`) of the page
 * "ik_llama.cpp 老工作站多 GPU 部署 Qwen3-235B-A22B 实战指南" (nxmr.cn), recommended-command
 * section.  The page names the path without defining it; read as the SwiGLU feed-forward
 * of the models it runs:
 *     g = W_gate[e] x_ts,  u = W_up[e] x_ts,  Y[t][s][n] = silu(g[n]) * u[n],
 *     silu(z) = z / (1 + exp(-z))
 * One pass: each selected expert's gate and up rows are streamed once per group of its
 * slots (groups as for qmv_id), both sums share every input read.  w_gate and w_up: two expert
 * tensors of the same format and shape, each packed as one matrix of E*N rows.  Everything
 * else (ids, strides, padding and out-of-range ids, limits, errors) as qmv_id. */
int qmv_id_gate_up(int fmt, const void* w_gate, const void* w_up, int E, int64_t N, int64_t K,
                   const int32_t* ids, int T, int top_k, const float* X, int64_t x_tok_stride,
                   int64_t x_slot_stride, float* Y, hipStream_t stream);

/* Expert-indexed GEMV with the router-weighted sum over each token's slots: the output of
 * a mixture-of-experts feed-forward layer (the top-k routed experts of the page
 * "ik_llama.cpp 老工作站多 GPU 部署 Qwen3-235B-A22B 实战指南" (nxmr.cn), background
 * section), its small decode-time steps merged as the "llama.cpp-v100" README
 * (shadowgraph.io) describes in its kernels-and-runtime list: the weighting is done in the
 * product's store, the sum by one small kernel after it.  Read as
 *     Y_slots[t][s][n] = weights[t][s] * sum_k dequant(W)[e][n][k] * x_ts[k]
 *     Y[t][n]          = sum_{s < top_k} Y_slots[t][s][n]     (fp32, s ascending)
 * with e, x_ts, padding and out-of-range ids as in qmv_id: a padding slot's row is 0 (it
 * adds 0), an id >= E gives a NaN row (Y[t][n] is NaN).  Deterministic.
 * weights: fp32 [T][top_k], 4-byte aligned.  Y_slots: fp32 [T][top_k][N] (device memory
 * the caller owns; written as qmv_id's Y, scaled by the weights).  Y: fp32 [T][N], 16-byte
 * aligned, not overlapping Y_slots.  top_k = 0 writes Y = 0.  Limits and status codes as
 * qmv_id; a null or misaligned weights pointer: BQM_E_NULL / BQM_E_ALIGN. */
int qmv_id_sum(int fmt, const void* w_packed, int E, int64_t N, int64_t K, const int32_t* ids,
               const float* weights, int T, int top_k, const float* X, int64_t x_tok_stride,
               int64_t x_slot_stride, float* Y_slots, float* Y, hipStream_t stream);

/* qmv_id_sum for callers that cannot allocate device memory (code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc): the same computation and
 * results as qmv_id_sum, without the Y_slots argument.  The weighted slot rows are kept in a
 * device array inside the library, BQM_NOALLOC_SLOT_FLOATS floats (4 MiB) per GPU, held
 * from the first call on that GPU until the process ends; the call itself allocates
 * nothing.  T * top_k * N above BQM_NOALLOC_SLOT_FLOATS: BQM_E_SHAPE.  Every call on one GPU
 * uses that GPU's array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must not be issued.  Other arguments, limits and status codes as
 * qmv_id_sum; BQM_E_LAUNCH also if the array's address cannot be obtained. */
#define BQM_NOALLOC_SLOT_FLOATS (1 << 20)
int qmv_id_sum_noalloc(int fmt, const void* w_packed, int E, int64_t N, int64_t K,
                       const int32_t* ids, const float* weights, int T, int top_k, const float* X,
                       int64_t x_tok_stride, int64_t x_slot_stride, float* Y, hipStream_t stream);

/* ---- chains of GEMVs in one launch ----------------------------------------------------
 * Decode runs one GEMV after another, each reading the previous one's output (through
 * the layers' other operations); launching them one by one pays a kernel start and drain
 * per GEMV.  The pages remove that per-launch cost by capturing decode in graphs and fusing
 * operators (page "v100llm：专为NVIDIA V100 GPU打造的高性能大模型推理引擎" (zingnex.cn),
 * section 4) and by merging the many small decode operators ("llama.cpp-v100" README
 * (shadowgraph.io), kernels-and-runtime list); here the GEMVs of a decode step share one
 * persistent launch.  A chain runs a list of GEMVs in order in ONE launch: a GEMV marked `wait`
 * starts only after every earlier GEMV of the chain has finished and its outputs are
 * visible device-wide (so its x may be an earlier GEMV's y); the weights of the next GEMV
 * are already streaming while the previous one finishes.  Every GEMV of a chain has the
 * same batch M (1..8).  Same arithmetic and tolerance as qmv_q4_0 / qmv_q8_0. */
typedef struct bqm_gemv {
  const void* w_packed;  /* packed N x K matrix (device)                              */
  const float* x;        /* [M][K] fp32 inputs (device), row-major, 16-byte aligned   */
  float* y;              /* [M][N] fp32 outputs (device), row-major                   */
  int64_t N, K;          /* 1 <= N <= 2^30; 32 <= K <= BQM_CHAIN_MAX_K, K % 32 == 0   */
  int32_t fmt;           /* BQM_Q4_0 or BQM_Q8_0, the same for every GEMV of a chain  */
  int32_t wait;          /* nonzero: start after all earlier GEMVs of the chain       */
  int32_t M;             /* batch, 1..8, the same for every GEMV of a chain           */
  int32_t reserved;      /* set to 0                                                  */
} bqm_gemv;

/* Largest K of a chain GEMV.  The chain keeps a 64-byte table row per GEMV and the staged
 * inputs in the LDS of each workgroup: bqm_chain_prepare returns BQM_E_SHAPE when the table
 * leaves no room for 32 blocks of K per input row (about 1900 GEMVs at M = 1; the inputs of
 * a long K are then staged in chunks). */
#define BQM_CHAIN_MAX_K 32768

/* Device bytes of the workspace of an n-GEMV chain (0 if n < 1). */
size_t bqm_chain_workspace_bytes(int n);

/* Validates the n host-side descriptors, then writes them, the staging plan and a zeroed
 * synchronization header into `workspace` (device memory, bqm_chain_workspace_bytes(n)
 * bytes, 16-byte aligned, owned by the caller).  A set-up call: it synchronizes `stream`
 * before it returns, so `descs` may be freed afterwards.  Errors: BQM_E_SHAPE (sizes, M
 * differing between GEMVs, a chain too long for the LDS), BQM_E_NULL, BQM_E_ALIGN,
 * BQM_E_UNSUPPORTED (mixed or unknown formats), BQM_E_LAUNCH. */
int bqm_chain_prepare(const bqm_gemv* descs, int n, void* workspace, hipStream_t stream);

/* Runs a prepared chain in one launch on `stream`; fmt, M and n must be those it was
 * prepared with (the kernel checks fmt, n and the class of M against the workspace and
 * otherwise computes nothing and records error 2).  A chain with a waiting GEMV runs as a
 * cooperative launch (all workgroups resident at once); one without (independent GEMVs,
 * split between the workgroups together) as an ordinary launch.  The workspace is left
 * ready for the next call; calls sharing one workspace must not overlap in time. */
int qmv_chain(int fmt, int M, void* workspace, int n, hipStream_t stream);

/* Synchronizes `stream` and returns the chain's error word: 0 = ok, 1 = a device-wide
 * wait timed out (results invalid; prepare again), 2 = fmt/M/n mismatch, -1 = copy failed. */
int bqm_chain_status(const void* workspace, hipStream_t stream);

/* Activation quantizer for the prefill product.  The prefill kernels the pages describe
 * work on Q8_0-format blocks ("llama.cpp-v100" README (shadowgraph.io): its SM70 kernels
 * adapted to Q8_0, computing-kernels item); the activations are read as taking the same
 * 32-wide int8 block shape with an fp32 scale, per row m and block b, in IEEE single
 * precision:  a = max_j |x_j|;  dx = a / 127 (correctly rounded);  dx == 0 gives all-zero
 * codes and dx = +0; otherwise Xq_j = round_half_away_from_zero(x_j / dx) clamped to
 * [-127, 127].  X: fp32 [M][K];  Xq: int8 [M][K];  dx: fp32 [M][K/32].  Bit exact. */
int bqm_quantize_q8_act(const float* X, int8_t* Xq, float* dx, int64_t M, int64_t K,
                        hipStream_t stream);

/* Prefill product with Q8_0 weights (the llama-bench pp512 shape of the page "llama.cpp
 * 0.9.0" analysis (ai-v5 LLMNews), section 2 table):
 *     isum[m][n][b] = sum_{j<32} qw[n][32b+j] * Xq[m][32b+j]        exact int32 (int8 MFMA)
 *     Y[m][n]       = sum_b (d_w[n][b] * dx[m][b]) * isum[m][n][b]    fp32, b ascending
 * The scale product d_w * dx comes from the matrix cores as an fp32 sum of six exact
 * partial products (d_w and dx split into bf16 parts); it may differ from the correctly
 * rounded product in the last bits, well within the float tolerance.
 * w_packed: packed Q8_0 N x K matrix.  Xq, dx: from bqm_quantize_q8_act.  Y: fp32 [M][N].
 * Operands are addressed with 32-bit offsets: M*K or N*K code bytes of 2 GiB or more give
 * BQM_E_SHAPE. */
int qmm_q8_0(const void* w_packed, const int8_t* Xq, const float* dx, float* Y, int64_t M,
             int64_t N, int64_t K, hipStream_t stream);

/* Prefill product with Q4_0 weights (the pp512 prompt-processing rows of Q4_0 (QAT)
 * models in the same section of the "llama.cpp 0.9.0" analysis page): the definition of
 * qmm_q8_0 with qw the nibble - 8 (weight j of a block in the low nibble of code byte j,
 * weight j + 16 in the high one).  The nibbles are widened to int8 on the way into local
 * memory, so the integer sums are exact and the scaling is that of qmm_q8_0.
 * w_packed: packed Q4_0 N x K matrix; the rest as for qmm_q8_0.  Same status codes. */
int qmm_q4_0(const void* w_packed, const int8_t* Xq, const float* dx, float* Y, int64_t M,
             int64_t N, int64_t K, hipStream_t stream);

/* Expert-indexed prefill product: the prefill expert matmul of the "llama.cpp-v100" README
 * (shadowgraph.io), kernels-and-runtime list, with qmv_id's routing (mul_mat_id, page
 * "ik_llama.cpp 老工作站多 GPU 部署 Qwen3-235B-A22B 实战指南" (nxmr.cn)):
 *     e = ids[t][s],  r = t * x_tok_rows + s * x_slot_rows,
 *     Y[t][s][n] = sum_b d_w[e][n][b] * dx[r][b] * sum_j qw[e][n][32b+j] * Xq[r][32b+j]
 * i.e. qmm_q8_0 / qmm_q4_0 of input row r with expert e's matrix, integer block sums exact,
 * the scaling as in qmm_q8_0.  The slots of each expert are gathered into row tiles (in
 * slot order), so each expert's rows are streamed once per 64 of its slots.
 * w_packed: expert tensor of format fmt packed as ONE matrix of E*N rows.  ids: int32
 * [T][top_k].  Xq, dx: quantized activations from bqm_quantize_q8_act, rows as indexed
 * above (x_tok_rows = 1, x_slot_rows = 0: one row per token; top_k, 1: one per slot).
 * Y: fp32 [T][top_k][N].  Padding slots (negative id) give zero rows, ids >= E NaN rows.
 * Limits: T <= BQM_QMM_ID_MAX_T, top_k <= 32, E <= 4096; the input rows the slots address,
 * and one expert's codes, below 2 GiB (else BQM_E_SHAPE). */
int qmm_id(int fmt, const void* w_packed, int E, int64_t N, int64_t K, const int32_t* ids, int T,
           int top_k, const int8_t* Xq, const float* dx, int64_t x_tok_rows, int64_t x_slot_rows,
           float* Y, hipStream_t stream);

/* Static English text for a status code. */
const char* bqm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* BQM_H */
