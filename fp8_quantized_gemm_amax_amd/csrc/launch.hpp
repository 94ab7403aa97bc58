// launch.hpp - host-side launchers behind the C ABI (internal; arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8amax {

// Fused amax + scale + cast per group (group_rows 1 or 128, group_cols 128).  With
// write_q = false only the amax grid is written to `out`.
void launch_groups(int dt, const void* x, int64_t rows, int64_t cols, int32_t group_rows,
                   uint8_t* q, float* out, bool write_q, hipStream_t s);

// Whole-tensor amax of n elements into the word `word`.  want_scale = false: the word ends
// as the float amax.  want_scale = true: the word holds a pending reduction key that
// launch_tensor_cast turns into the float scale amax / 448 (for n == 0 it is finished here).
void launch_tensor_reduce(int dt, const void* x, int64_t n, float* word, bool want_scale,
                          hipStream_t s);

// Whole-tensor quantize of n elements: the scale word and the codes.  Small tensors take
// one single-workgroup launch; larger ones launch_tensor_reduce + launch_tensor_cast.
void launch_tensor_quantize(int dt, const void* x, int64_t n, float* scale, uint8_t* q,
                            hipStream_t s);

// q[i] = e4m3(x[i] / scale) for n > 0 elements, with the scale taken from (and written
// back to) the word launch_tensor_reduce left.
void launch_tensor_cast(int dt, const void* x, int64_t n, float* scale, uint8_t* q,
                        hipStream_t s);

void launch_debug_cast(const float* v, int64_t n, uint8_t* q, hipStream_t s);

// Decode GEMV path: whether it takes this shape (1 <= M <= 16, 32 K below 2^31) and its
// launcher.
bool gemv_fits(int M, int K);
void launch_gemv(bool blockwise, int out_dt, const uint8_t* qa, const float* sa, const uint8_t* qb,
                 const float* sb, int M, int N, int K, void* c, hipStream_t s);

// Scaled FP8 GEMM, C [M, N] of out_dt (dispatches M <= 16 to the GEMV path).
void launch_gemm(bool blockwise, int out_dt, const uint8_t* qa, const float* sa, const uint8_t* qb,
                 const float* sb, int M, int N, int K, void* c, hipStream_t s);

}  // namespace fp8amax
