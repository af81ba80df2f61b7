// C ABI of the library (declared in include/bqm.h): argument checks on the host, then
// one asynchronous launch sequence on the caller's stream.  Nothing here allocates,
// frees or synchronizes.
#include "bqm_internal.h"

using namespace bqm;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }
bool valid_fmt(int fmt) { return fmt == BQM_Q4_0 || fmt == BQM_Q8_0; }

// Largest row count the kernels index with 32-bit row numbers.
constexpr int64_t kMaxRows = (int64_t)1 << 30;

int check_shape(int fmt, int64_t rows, int64_t K) {
  if (!valid_fmt(fmt)) return BQM_E_UNSUPPORTED;
  if (rows < 0 || K < 0 || K % kQK != 0 || rows > kMaxRows || K > ((int64_t)1 << 30))
    return BQM_E_SHAPE;
  return BQM_OK;
}

int check_ptr(const void* w) {
  if (!w) return BQM_E_NULL;
  if (!aligned16(w)) return BQM_E_ALIGN;
  return BQM_OK;
}


// Argument checks shared by qmv_id and qmv_id_gate_up (w2: the up tensor, or null).
int check_id(int fmt, const void* w, const void* w2, bool pair, int E, int64_t N, int64_t K,
             const int32_t* ids, int T, int top_k, const float* X, int64_t x_tok_stride,
             int64_t x_slot_stride, float* Y, bool* nothing) {
  *nothing = false;
  if (E < 0 || T < 0 || top_k < 0 || T > BQM_QMV_ID_MAX_T || top_k > BQM_QMV_ID_MAX_TOPK ||
      E > BQM_QMV_ID_MAX_E)
    return BQM_E_SHAPE;
  if (N < 0 || (int64_t)E * N > kMaxRows) return BQM_E_SHAPE;
  if (int st = check_shape(fmt, (int64_t)E * N, K)) return st;
  if (x_tok_stride < 0 || x_slot_stride < 0) return BQM_E_SHAPE;
  if (T == 0 || top_k == 0 || N == 0) {
    *nothing = true;
    return BQM_OK;
  }
  if (!Y || !ids) return BQM_E_NULL;
  if (!aligned16(Y) || !aligned16(ids)) return BQM_E_ALIGN;
  if (K > 0 && E > 0) {
    if (int st = check_ptr(w)) return st;
    if (pair)
      if (int st = check_ptr(w2)) return st;
    if (int st = check_ptr(X)) return st;
    // every (t, s) input row must start 16-byte aligned
    if ((x_tok_stride & 3) != 0 || (x_slot_stride & 3) != 0) return BQM_E_ALIGN;
  }
  return BQM_OK;
}
}  // namespace

extern "C" {

size_t bqm_packed_bytes(int fmt, int64_t rows, int64_t K) {
  Layout L;
  if (!layout_of(fmt, rows, K, &L)) return 0;
  return (size_t)L.total;
}

int bqm_repack(int fmt, const void* w_interchange, void* w_packed, int64_t rows, int64_t K,
               hipStream_t stream) {
  if (int st = check_shape(fmt, rows, K)) return st;
  if (rows == 0 || K == 0) return BQM_OK;
  if (int st = check_ptr(w_packed)) return st;
  if (!w_interchange) return BQM_E_NULL;
  if (!aligned2(w_interchange)) return BQM_E_ALIGN;
  return launch_repack(fmt, w_interchange, w_packed, rows, K, stream);
}

int bqm_unpack(int fmt, const void* w_packed, void* w_interchange, int64_t rows, int64_t K,
               hipStream_t stream) {
  if (int st = check_shape(fmt, rows, K)) return st;
  if (rows == 0 || K == 0) return BQM_OK;
  if (int st = check_ptr(w_packed)) return st;
  if (!w_interchange) return BQM_E_NULL;
  if (!aligned2(w_interchange)) return BQM_E_ALIGN;
  return launch_unpack(fmt, w_packed, w_interchange, rows, K, stream);
}

static int qmv_common(int fmt, const void* w, const float* X, float* Y, int M, int64_t N, int64_t K,
                      hipStream_t stream) {
  if (int st = check_shape(fmt, N, K)) return st;
  if (M < 0 || M > BQM_QMV_MAX_M) return BQM_E_SHAPE;
  if (M == 0 || N == 0) return BQM_OK;
  if (!Y) return BQM_E_NULL;
  if (!aligned16(Y)) return BQM_E_ALIGN;
  if (K > 0) {
    if (int st = check_ptr(w)) return st;
    if (int st = check_ptr(X)) return st;
  }
  return launch_qmv(fmt, w, X, Y, M, N, K, stream);
}

int qmv_q4_0(const void* w_packed, const float* X, float* Y, int M, int64_t N, int64_t K,
             hipStream_t stream) {
  return qmv_common(BQM_Q4_0, w_packed, X, Y, M, N, K, stream);
}

int qmv_q8_0(const void* w_packed, const float* X, float* Y, int M, int64_t N, int64_t K,
             hipStream_t stream) {
  return qmv_common(BQM_Q8_0, w_packed, X, Y, M, N, K, stream);
}

int qmv_id(int fmt, const void* w_packed, int E, int64_t N, int64_t K, const int32_t* ids, int T,
           int top_k, const float* X, int64_t x_tok_stride, int64_t x_slot_stride, float* Y,
           hipStream_t stream) {
  bool nothing = false;
  if (int st = check_id(fmt, w_packed, nullptr, false, E, N, K, ids, T, top_k, X, x_tok_stride,
                        x_slot_stride, Y, &nothing))
    return st;
  if (nothing) return BQM_OK;
  return launch_qmv_id(fmt, w_packed, E, N, K, ids, T, top_k, X, x_tok_stride, x_slot_stride, Y,
                       stream);
}

int qmv_id_gate_up(int fmt, const void* w_gate, const void* w_up, int E, int64_t N, int64_t K,
                   const int32_t* ids, int T, int top_k, const float* X, int64_t x_tok_stride,
                   int64_t x_slot_stride, float* Y, hipStream_t stream) {
  bool nothing = false;
  if (int st = check_id(fmt, w_gate, w_up, true, E, N, K, ids, T, top_k, X, x_tok_stride,
                        x_slot_stride, Y, &nothing))
    return st;
  if (nothing) return BQM_OK;
  return launch_qmv_id_gate_up(fmt, w_gate, w_up, E, N, K, ids, T, top_k, X, x_tok_stride,
                               x_slot_stride, Y, stream);
}

int qmv_id_sum(int fmt, const void* w_packed, int E, int64_t N, int64_t K, const int32_t* ids,
               const float* weights, int T, int top_k, const float* X, int64_t x_tok_stride,
               int64_t x_slot_stride, float* Y_slots, float* Y, hipStream_t stream) {
  bool nothing = false;
  if (int st = check_id(fmt, w_packed, nullptr, false, E, N, K, ids, T, top_k, X, x_tok_stride,
                        x_slot_stride, Y_slots, &nothing))
    return st;
  if (T == 0 || N == 0) return BQM_OK;
  if (!Y) return BQM_E_NULL;
  if (!aligned16(Y)) return BQM_E_ALIGN;
  if (top_k == 0) return launch_fill(Y, (int64_t)T * N, 0.0f, stream);  // empty sums
  if (!weights) return BQM_E_NULL;
  if ((reinterpret_cast<uintptr_t>(weights) & 3) != 0) return BQM_E_ALIGN;
  return launch_qmv_id_sum(fmt, w_packed, E, N, K, ids, weights, T, top_k, X, x_tok_stride,
                           x_slot_stride, Y_slots, Y, stream);
}

int qmv_id_sum_noalloc(int fmt, const void* w_packed, int E, int64_t N, int64_t K,
                       const int32_t* ids, const float* weights, int T, int top_k, const float* X,
                       int64_t x_tok_stride, int64_t x_slot_stride, float* Y, hipStream_t stream) {
  bool nothing = false;
  // the same checks as qmv_id_sum, Y standing in for the slot rows' pointer checks
  if (int st = check_id(fmt, w_packed, nullptr, false, E, N, K, ids, T, top_k, X, x_tok_stride,
                        x_slot_stride, Y, &nothing))
    return st;
  if (T == 0 || N == 0) return BQM_OK;
  if (!Y) return BQM_E_NULL;
  if (!aligned16(Y)) return BQM_E_ALIGN;
  if ((int64_t)T * top_k * N > BQM_NOALLOC_SLOT_FLOATS) return BQM_E_SHAPE;
  if (top_k == 0) return launch_fill(Y, (int64_t)T * N, 0.0f, stream);  // empty sums
  if (!weights) return BQM_E_NULL;
  if ((reinterpret_cast<uintptr_t>(weights) & 3) != 0) return BQM_E_ALIGN;
  return launch_qmv_id_sum_noalloc(fmt, w_packed, E, N, K, ids, weights, T, top_k, X, x_tok_stride,
                                   x_slot_stride, Y, stream);
}

int bqm_quantize_q8_act(const float* X, int8_t* Xq, float* dx, int64_t M, int64_t K,
                        hipStream_t stream) {
  if (M < 0 || K < 0 || K % kQK != 0 || M > kMaxRows || K > ((int64_t)1 << 30)) return BQM_E_SHAPE;
  if (M == 0 || K == 0) return BQM_OK;
  if (!X || !Xq || !dx) return BQM_E_NULL;
  if (!aligned16(X) || !aligned16(Xq) || !aligned16(dx)) return BQM_E_ALIGN;
  return launch_quantize_q8_act(X, Xq, dx, M, K, stream);
}

static int qmm_common(int fmt, const void* w_packed, const int8_t* Xq, const float* dx, float* Y,
                      int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (int st = check_shape(fmt, N, K)) return st;
  if (M < 0 || M > kMaxRows) return BQM_E_SHAPE;
  if (M == 0 || N == 0) return BQM_OK;
  if (!Y) return BQM_E_NULL;
  if (!aligned16(Y)) return BQM_E_ALIGN;
  if (K == 0) return launch_fill(Y, M * N, 0.0f, stream);
  if (int st = check_ptr(w_packed)) return st;
  if (int st = check_ptr(Xq)) return st;
  if (int st = check_ptr(dx)) return st;
  return fmt == BQM_Q4_0 ? launch_qmm_q4_0(w_packed, Xq, dx, Y, M, N, K, stream)
                         : launch_qmm_q8_0(w_packed, Xq, dx, Y, M, N, K, stream);
}

int qmm_q8_0(const void* w_packed, const int8_t* Xq, const float* dx, float* Y, int64_t M,
             int64_t N, int64_t K, hipStream_t stream) {
  return qmm_common(BQM_Q8_0, w_packed, Xq, dx, Y, M, N, K, stream);
}

int qmm_q4_0(const void* w_packed, const int8_t* Xq, const float* dx, float* Y, int64_t M,
             int64_t N, int64_t K, hipStream_t stream) {
  return qmm_common(BQM_Q4_0, w_packed, Xq, dx, Y, M, N, K, stream);
}

int qmm_id(int fmt, const void* w_packed, int E, int64_t N, int64_t K, const int32_t* ids, int T,
           int top_k, const int8_t* Xq, const float* dx, int64_t x_tok_rows, int64_t x_slot_rows,
           float* Y, hipStream_t stream) {
  if (E < 0 || T < 0 || top_k < 0 || T > BQM_QMM_ID_MAX_T || top_k > BQM_QMV_ID_MAX_TOPK ||
      E > BQM_QMV_ID_MAX_E)
    return BQM_E_SHAPE;
  if (N < 0 || (int64_t)E * N > kMaxRows) return BQM_E_SHAPE;
  if (int st = check_shape(fmt, (int64_t)E * N, K)) return st;
  if (x_tok_rows < 0 || x_slot_rows < 0) return BQM_E_SHAPE;
  if (T > 0 && top_k > 0 &&
      (int64_t)(T - 1) * x_tok_rows + (int64_t)(top_k - 1) * x_slot_rows >= ((int64_t)1 << 31))
    return BQM_E_SHAPE;
  if (T == 0 || top_k == 0 || N == 0) return BQM_OK;
  if (!Y || !ids) return BQM_E_NULL;
  if (!aligned16(Y) || !aligned16(ids)) return BQM_E_ALIGN;
  if (K > 0 && E > 0) {
    if (int st = check_ptr(w_packed)) return st;
    if (int st = check_ptr(Xq)) return st;
    if (int st = check_ptr(dx)) return st;
  }
  return launch_qmm_id(fmt, w_packed, E, N, K, ids, T, top_k, Xq, dx, x_tok_rows, x_slot_rows, Y,
                       stream);
}

size_t bqm_chain_workspace_bytes(int n) { return chain_workspace_bytes(n); }

int bqm_chain_prepare(const bqm_gemv* descs, int n, void* workspace, hipStream_t stream) {
  if (n < 1 || n > (1 << 20)) return BQM_E_SHAPE;
  if (!descs || !workspace) return BQM_E_NULL;
  if (!aligned16(workspace)) return BQM_E_ALIGN;
  return chain_prepare(descs, n, workspace, stream);
}

int qmv_chain(int fmt, int M, void* workspace, int n, hipStream_t stream) {
  if (!valid_fmt(fmt)) return BQM_E_UNSUPPORTED;
  if (n < 1 || n > (1 << 20) || M < 1 || M > BQM_QMV_MAX_M) return BQM_E_SHAPE;
  if (!workspace) return BQM_E_NULL;
  if (!aligned16(workspace)) return BQM_E_ALIGN;
  return chain_launch(fmt, M, workspace, n, stream);
}

int bqm_chain_status(const void* workspace, hipStream_t stream) {
  if (!workspace) return -1;
  return chain_status(workspace, stream);
}

const char* bqm_strerror(int status) {
  switch (status) {
    case BQM_OK: return "success";
    case BQM_E_NULL: return "a required pointer is NULL";
    case BQM_E_SHAPE: return "invalid size (negative, K not a multiple of 32, or over a limit)";
    case BQM_E_ALIGN: return "a pointer or stride is not suitably aligned (16 bytes)";
    case BQM_E_UNSUPPORTED: return "unknown block format";
    case BQM_E_LAUNCH: return "the HIP runtime refused a kernel launch";
    default: return "unknown status";
  }
}

}  // extern "C"
