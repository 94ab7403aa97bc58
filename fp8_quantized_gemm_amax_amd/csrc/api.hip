// api.hip - the C ABI declared in include/fp8amax.h: host-side validation, then kernel
// launches on the caller's stream.  Validation makes no HIP call, so every error path can
// be exercised on a machine without a GPU.
#include "fp8amax.h"

#include <hip/hip_runtime.h>

#include "gemm_plan.hpp"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;   // kernels index rows/cols with int
constexpr int64_t kMaxElems = int64_t{1} << 40;
constexpr int64_t kMaxExperts = int64_t{1} << 16;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool valid_dt(fp8_dtype_t dt) { return dt == FP8_BF16 || dt == FP8_F16; }

fp8_status_t check_2d(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return FP8_ERR_BAD_SHAPE;
  if (rows > kMaxDim || cols > kMaxDim) return FP8_ERR_TOO_LARGE;
  if (cols > 0 && rows > kMaxElems / cols) return FP8_ERR_TOO_LARGE;
  return FP8_OK;
}

bool group_shape_ok(int32_t gr, int32_t gc) { return gc == 128 && (gr == 1 || gr == 128); }

fp8_status_t finish_launch() {
  return hipGetLastError() == hipSuccess ? FP8_OK : FP8_ERR_LAUNCH;
}

// Shape rules of the scaled GEMMs, and the plan of their launches (FP8_OK only).
fp8_status_t gemm_shape(int mode, int64_t M, int64_t N, int64_t K, fp8_gemm_plan_t* plan) {
  const bool blockwise = fp8amax::slab_scaled(mode);
  if (M < 0 || N < 0 || K <= 0) return FP8_ERR_BAD_SHAPE;
  if (blockwise ? (K % 128 != 0) : (K % 16 != 0)) return FP8_ERR_BAD_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8_ERR_TOO_LARGE;
  if (M > kMaxElems / K || N > kMaxElems / K || (N > 0 && M > kMaxElems / N)) return FP8_ERR_TOO_LARGE;
  *plan = fp8amax::plan::plan_gemm(mode, M, N, K);
  if (!fp8amax::plan::plan_fits(*plan)) return FP8_ERR_TOO_LARGE;
  return FP8_OK;
}

fp8_status_t gemm_common(int mode, const uint8_t* qa, const void* sa, const uint8_t* qb,
                         const void* sb, int64_t M, int64_t N, int64_t K, void* c,
                         fp8_dtype_t out_dt, void* stream) {
  fp8_gemm_plan_t plan;
  const fp8_status_t st = gemm_shape(mode, M, N, K, &plan);
  if (st != FP8_OK) return st;
  if (!valid_dt(out_dt)) return FP8_ERR_BAD_DTYPE;
  if (M == 0 || N == 0) return FP8_OK;
  if (!qa || !sa || !qb || !sb || !c) return FP8_ERR_NULL_POINTER;
  if (!aligned16(qa) || !aligned16(qb) || !aligned16(c) || !aligned4(sa) || !aligned4(sb))
    return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();   // clear a stale error so FP8_ERR_LAUNCH reports this call only
  if (!fp8amax::launch_gemm(mode, static_cast<int>(out_dt), plan, qa, sa, qb, sb, static_cast<int>(M),
                            static_cast<int>(N), static_cast<int>(K), c, static_cast<hipStream_t>(stream)))
    return FP8_ERR_LAUNCH;
  return finish_launch();
}

fp8_status_t grouped_common(int mode, const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb,
                            const int32_t* offsets, int64_t E, int64_t T, int64_t N, int64_t K, void* c,
                            fp8_dtype_t out_dt, void* stream) {
  if (E < 1 || T < 0 || N < 0 || K <= 0 || K % 128 != 0) return FP8_ERR_BAD_SHAPE;
  if (E > kMaxExperts || T > kMaxDim || N > kMaxDim || K * 256 >= (int64_t{1} << 31)) return FP8_ERR_TOO_LARGE;
  if (E * N > kMaxDim || (N > 0 && E > kMaxElems / (N * K))) return FP8_ERR_TOO_LARGE;
  if (!valid_dt(out_dt)) return FP8_ERR_BAD_DTYPE;
  if (T == 0 || N == 0) return FP8_OK;
  if (!qa || !sa || !qb || !sb || !offsets || !c) return FP8_ERR_NULL_POINTER;
  if (!aligned16(qa) || !aligned16(qb) || !aligned16(c) || !aligned4(sa) || !aligned4(sb) || !aligned4(offsets))
    return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();
  if (!fp8amax::launch_grouped(mode, static_cast<int>(out_dt), qa, sa, qb, sb, offsets, static_cast<int>(E),
                               static_cast<int>(T), static_cast<int>(N), static_cast<int>(K), c,
                               static_cast<hipStream_t>(stream)))
    return FP8_ERR_TOO_LARGE;
  return finish_launch();
}

}  // namespace

extern "C" {

const char* fp8_status_string(fp8_status_t s) {
  switch (s) {
    case FP8_OK: return "FP8_OK";
    case FP8_ERR_NULL_POINTER: return "FP8_ERR_NULL_POINTER: a required pointer is NULL";
    case FP8_ERR_BAD_SHAPE: return "FP8_ERR_BAD_SHAPE: unsupported size or group/block shape";
    case FP8_ERR_BAD_DTYPE: return "FP8_ERR_BAD_DTYPE: unknown 16-bit dtype";
    case FP8_ERR_MISALIGNED: return "FP8_ERR_MISALIGNED: data pointers need 16-byte, float pointers 4-byte alignment";
    case FP8_ERR_LAUNCH: return "FP8_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case FP8_ERR_TOO_LARGE: return "FP8_ERR_TOO_LARGE: a dimension exceeds 2^31-1 or a tensor 2^40 elements";
  }
  return "unknown fp8_status_t";
}

fp8_status_t fp8_amax(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                      int32_t block_rows, int32_t block_cols, float* amax, void* stream) {
  fp8_status_t st = check_2d(rows, cols);
  if (st != FP8_OK) return st;
  const bool whole = block_rows == 0 && block_cols == 0;
  if (!whole && !group_shape_ok(block_rows, block_cols)) return FP8_ERR_BAD_SHAPE;
  if (!valid_dt(dt)) return FP8_ERR_BAD_DTYPE;
  const int64_t n = rows * cols;
  if (!whole && n == 0) return FP8_OK;                 // empty grid: nothing to write
  if (!amax || (n > 0 && !x)) return FP8_ERR_NULL_POINTER;
  if ((x && !aligned16(x)) || !aligned4(amax)) return FP8_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (whole) fp8amax::launch_tensor_amax(static_cast<int>(dt), x, n, amax, s);
  else fp8amax::launch_groups(static_cast<int>(dt), x, rows, cols, block_rows, nullptr, amax, false, s);
  return finish_launch();
}

fp8_status_t fp8_quantize_per_tensor(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                     uint8_t* q, float* scale, void* stream) {
  fp8_status_t st = check_2d(rows, cols);
  if (st != FP8_OK) return st;
  if (!valid_dt(dt)) return FP8_ERR_BAD_DTYPE;
  const int64_t n = rows * cols;
  if (!scale || (n > 0 && (!x || !q))) return FP8_ERR_NULL_POINTER;
  if ((x && !aligned16(x)) || (q && !aligned16(q)) || !aligned4(scale)) return FP8_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  fp8amax::launch_tensor_quantize(static_cast<int>(dt), x, n, scale, q, s);
  return finish_launch();
}

fp8_status_t fp8_quantize_rowwise(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols, uint8_t* q,
                                  float* scales, void* stream) {
  fp8_status_t st = check_2d(rows, cols);
  if (st != FP8_OK) return st;
  if (!valid_dt(dt)) return FP8_ERR_BAD_DTYPE;
  if (rows == 0) return FP8_OK;
  if (!scales || (cols > 0 && (!x || !q))) return FP8_ERR_NULL_POINTER;
  if ((x && !aligned16(x)) || (q && !aligned16(q)) || !aligned4(scales)) return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();
  fp8amax::launch_rows(static_cast<int>(dt), x, rows, cols, q, scales, static_cast<hipStream_t>(stream));
  return finish_launch();
}

fp8_status_t fp8_gemm_scaled_rowwise(const uint8_t* qa, const float* sa, const uint8_t* qb,
                                     const float* sb, int64_t M, int64_t N, int64_t K, void* c,
                                     fp8_dtype_t out_dt, void* stream) {
  return gemm_common(fp8amax::SM_ROW, qa, sa, qb, sb, M, N, K, c, out_dt, stream);
}

fp8_status_t fp8_gemm_grouped_blockwise(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                                       const int32_t* offsets, int64_t E, int64_t T, int64_t N, int64_t K,
                                       void* c, fp8_dtype_t out_dt, void* stream) {
  return grouped_common(fp8amax::SM_BLOCK, qa, sa, qb, sb, offsets, E, T, N, K, c, out_dt, stream);
}

fp8_status_t fp8_gemm_grouped_blockwise_ue8m0(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb,
                                             const uint8_t* sb, const int32_t* offsets, int64_t E, int64_t T,
                                             int64_t N, int64_t K, void* c, fp8_dtype_t out_dt, void* stream) {
  return grouped_common(fp8amax::SM_E8M0, qa, sa, qb, sb, offsets, E, T, N, K, c, out_dt, stream);
}

fp8_status_t fp8_quantize_per_token_group(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                          int32_t group_rows, int32_t group_cols, uint8_t* q,
                                          float* scales, void* stream) {
  fp8_status_t st = check_2d(rows, cols);
  if (st != FP8_OK) return st;
  if (!group_shape_ok(group_rows, group_cols)) return FP8_ERR_BAD_SHAPE;
  if (!valid_dt(dt)) return FP8_ERR_BAD_DTYPE;
  if (rows * cols == 0) return FP8_OK;
  if (!x || !q || !scales) return FP8_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(q) || !aligned4(scales)) return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();
  fp8amax::launch_groups(static_cast<int>(dt), x, rows, cols, group_rows, q, scales, true,
                         static_cast<hipStream_t>(stream));
  return finish_launch();
}

fp8_status_t fp8_gemm_scaled_tensorwise(const uint8_t* qa, const float* sa, const uint8_t* qb,
                                        const float* sb, int64_t M, int64_t N, int64_t K, void* c,
                                        fp8_dtype_t out_dt, void* stream) {
  return gemm_common(fp8amax::SM_TENSOR, qa, sa, qb, sb, M, N, K, c, out_dt, stream);
}

fp8_status_t fp8_gemm_scaled_blockwise(const uint8_t* qa, const float* sa, const uint8_t* qb,
                                       const float* sb, int64_t M, int64_t N, int64_t K, void* c,
                                       fp8_dtype_t out_dt, void* stream) {
  return gemm_common(fp8amax::SM_BLOCK, qa, sa, qb, sb, M, N, K, c, out_dt, stream);
}

fp8_status_t fp8_quantize_per_token_group_ue8m0(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                                int32_t group_rows, int32_t group_cols, uint8_t* q,
                                                uint8_t* scales, void* stream) {
  fp8_status_t st = check_2d(rows, cols);
  if (st != FP8_OK) return st;
  if (!group_shape_ok(group_rows, group_cols)) return FP8_ERR_BAD_SHAPE;
  if (!valid_dt(dt)) return FP8_ERR_BAD_DTYPE;
  if (rows * cols == 0) return FP8_OK;
  if (!x || !q || !scales) return FP8_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(q) || !aligned4(scales)) return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();
  fp8amax::launch_groups_e8m0(static_cast<int>(dt), x, rows, cols, group_rows, q, scales,
                              static_cast<hipStream_t>(stream));
  return finish_launch();
}

fp8_status_t fp8_gemm_scaled_blockwise_ue8m0(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb,
                                             const uint8_t* sb, int64_t M, int64_t N, int64_t K, void* c,
                                             fp8_dtype_t out_dt, void* stream) {
  return gemm_common(fp8amax::SM_E8M0, qa, sa, qb, sb, M, N, K, c, out_dt, stream);
}

fp8_status_t fp8_quantize_static(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                 const float* scale, uint8_t* q, uint32_t* amax_acc, void* stream) {
  fp8_status_t st = check_2d(rows, cols);
  if (st != FP8_OK) return st;
  if (!valid_dt(dt)) return FP8_ERR_BAD_DTYPE;
  const int64_t n = rows * cols;
  if (n == 0) return FP8_OK;
  if (!x || !q || !scale) return FP8_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(q) || !aligned4(scale) || (amax_acc && !aligned4(amax_acc)))
    return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();
  fp8amax::launch_tensor_static(static_cast<int>(dt), x, n, scale, q, amax_acc,
                                static_cast<hipStream_t>(stream));
  return finish_launch();
}

fp8_status_t fp8_delayed_scaling_update(float* history, int32_t len, uint32_t* amax_acc, int32_t* step,
                                        int32_t interval, int32_t margin, float* scale, void* stream) {
  if (len < 1 || interval < 1 || margin < -126 || margin > 126) return FP8_ERR_BAD_SHAPE;
  if (!history || !amax_acc || !step || !scale) return FP8_ERR_NULL_POINTER;
  if (!aligned4(history) || !aligned4(amax_acc) || !aligned4(step) || !aligned4(scale))
    return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();
  fp8amax::launch_delayed_update(history, len, amax_acc, step, interval, margin, scale,
                                 static_cast<hipStream_t>(stream));
  return finish_launch();
}

fp8_status_t fp8_quantize_delayed(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                  float* history, int32_t len, uint32_t* amax_acc, int32_t* step,
                                  int32_t interval, int32_t margin, float* scale, float* scale_used,
                                  uint8_t* q, void* stream) {
  fp8_status_t st = check_2d(rows, cols);
  if (st != FP8_OK) return st;
  if (!valid_dt(dt)) return FP8_ERR_BAD_DTYPE;
  if (len < 1 || interval < 1 || margin < -126 || margin > 126) return FP8_ERR_BAD_SHAPE;
  const int64_t n = rows * cols;
  if ((n > 0 && (!x || !q)) || !history || !amax_acc || !step || !scale || !scale_used)
    return FP8_ERR_NULL_POINTER;
  if ((n > 0 && (!aligned16(x) || !aligned16(q))) || !aligned4(history) || !aligned4(amax_acc) ||
      !aligned4(step) || !aligned4(scale) || !aligned4(scale_used))
    return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();
  fp8amax::launch_delayed_quantize(static_cast<int>(dt), x, n, history, len, amax_acc, step, interval,
                                   margin, scale, scale_used, q, static_cast<hipStream_t>(stream));
  return finish_launch();
}

fp8_status_t fp8_debug_cast_f32(const float* v, uint8_t* q, int64_t n, void* stream) {
  if (n < 0) return FP8_ERR_BAD_SHAPE;
  if (n > kMaxElems) return FP8_ERR_TOO_LARGE;
  if (n == 0) return FP8_OK;
  if (!v || !q) return FP8_ERR_NULL_POINTER;
  if (!aligned4(v)) return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();
  fp8amax::launch_debug_cast(v, n, q, static_cast<hipStream_t>(stream));
  return finish_launch();
}

fp8_status_t fp8_debug_gemm_plan(int32_t mode, int64_t M, int64_t N, int64_t K, fp8_gemm_plan_t* plan) {
  if (mode < FP8_SCALE_TENSOR || mode > FP8_SCALE_ROW) return FP8_ERR_BAD_SHAPE;
  if (!plan) return FP8_ERR_NULL_POINTER;
  return gemm_shape(mode, M, N, K, plan);
}

fp8_status_t fp8_gemv_dynamic(int32_t mode, const void* x, fp8_dtype_t in_dt, const uint8_t* qb, const void* sb,
                              int64_t N, int64_t K, uint8_t* qa, void* sa, void* c, fp8_dtype_t out_dt,
                              void* stream) {
  if (mode < FP8_SCALE_TENSOR || mode > FP8_SCALE_ROW) return FP8_ERR_BAD_SHAPE;
  fp8_gemm_plan_t plan;
  const fp8_status_t st = gemm_shape(mode, 1, N, K, &plan);
  if (st != FP8_OK) return st;
  if (!valid_dt(in_dt) || !valid_dt(out_dt)) return FP8_ERR_BAD_DTYPE;
  if (!x || !qa || !sa || (N > 0 && (!qb || !sb || !c))) return FP8_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(qa) || !aligned4(sa) ||
      (N > 0 && (!aligned16(qb) || !aligned4(sb) || !aligned16(c))))
    return FP8_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int idt = static_cast<int>(in_dt), odt = static_cast<int>(out_dt);
  (void)hipGetLastError();
  if (fp8amax::plan::dynamic_fits(N, K)) {
    fp8amax::launch_gemv_dynamic(mode, idt, odt, x, qb, sb, qa, sa, static_cast<int>(N), static_cast<int>(K), c, s);
    return finish_launch();
  }
  // the quantizer of the mode, then the one-token GEMM
  if (mode == FP8_SCALE_TENSOR) fp8amax::launch_tensor_quantize(idt, x, K, static_cast<float*>(sa), qa, s);
  else if (mode == FP8_SCALE_ROW) fp8amax::launch_rows(idt, x, 1, K, qa, static_cast<float*>(sa), s);
  else if (mode == FP8_SCALE_BLOCK) fp8amax::launch_groups(idt, x, 1, K, 1, qa, static_cast<float*>(sa), true, s);
  else fp8amax::launch_groups_e8m0(idt, x, 1, K, 1, qa, static_cast<uint8_t*>(sa), s);
  if (N > 0 && !fp8amax::launch_gemm(mode, odt, plan, qa, sa, qb, sb, 1, static_cast<int>(N), static_cast<int>(K), c, s))
    return FP8_ERR_LAUNCH;
  return finish_launch();
}

fp8_status_t fp8_debug_byte_mix(const void* x, uint8_t* q, int64_t n, void* stream) {
  if (n < 0) return FP8_ERR_BAD_SHAPE;
  if (n > kMaxElems) return FP8_ERR_TOO_LARGE;
  if (n == 0) return FP8_OK;
  if (!x || !q) return FP8_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(q)) return FP8_ERR_MISALIGNED;
  (void)hipGetLastError();
  fp8amax::launch_byte_mix(x, n, q, static_cast<hipStream_t>(stream));
  return finish_launch();
}

}  // extern "C"
