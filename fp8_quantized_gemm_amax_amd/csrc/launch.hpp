// launch.hpp - host-side launchers behind the C ABI (internal; arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8amax.h"

namespace fp8amax {

// How a GEMM is scaled (template argument of the GEMM kernels, argument of the launchers):
//   SM_TENSOR: one float32 scale per operand;
//   SM_BLOCK:  float32 scales per 1x128 activation group and 128x128 weight block;
//   SM_E8M0:   the same groups and blocks with UE8M0 scales, one e8m0fnu byte each,
//              every scale row padded to whole 32-bit words (e8m0_row_bytes);
//   SM_ROW:    one float32 scale per row of A (token) and per row of B (output channel).
enum ScaleMode { SM_TENSOR = 0, SM_BLOCK = 1, SM_E8M0 = 2, SM_ROW = 3 };

// Modes whose scales change every 128-wide K slab, applied inside the K loop; the others
// scale the finished float32 accumulator once in the epilogue.
__host__ __device__ constexpr bool slab_scaled(int sm) { return sm == SM_BLOCK || sm == SM_E8M0; }

// Bytes per row of a UE8M0 scale tensor with `groups` scales: four per 32-bit word.
__host__ __device__ constexpr int64_t e8m0_row_bytes(int64_t groups) { return (groups + 3) & ~int64_t{3}; }

// Fused amax + scale + cast per group (group_rows 1 or 128, group_cols 128).  With
// write_q = false only the amax grid is written to `out`.
void launch_groups(int dt, const void* x, int64_t rows, int64_t cols, int32_t group_rows,
                   uint8_t* q, float* out, bool write_q, hipStream_t s);

// The same groups and blocks with UE8M0 scales: the codes, and one e8m0fnu byte per group
// in rows of e8m0_row_bytes(groups per row) bytes whose padding is set to 127.
void launch_groups_e8m0(int dt, const void* x, int64_t rows, int64_t cols, int32_t group_rows,
                        uint8_t* q, uint8_t* codes, hipStream_t s);

// One float32 scale per row: amax of the row / 448, the row cast with it.
void launch_rows(int dt, const void* x, int64_t rows, int64_t cols, uint8_t* q, float* scales,
                 hipStream_t s);

// Whole-tensor amax of n elements into the float *amax (0 for n == 0).
void launch_tensor_amax(int dt, const void* x, int64_t n, float* amax, hipStream_t s);

// Whole-tensor quantize of n > 0 elements: the scale and the codes.  Small tensors take one
// single-workgroup launch; larger ones two launches, the first of which leaves partial
// maxima in q that the second reads before it overwrites them with codes.
void launch_tensor_quantize(int dt, const void* x, int64_t n, float* scale, uint8_t* q,
                            hipStream_t s);

// Static scaling: q[i] = e4m3(x[i] / *scale) for n > 0 elements in one pass; with amax_acc
// the tensor's amax is folded into *amax_acc (float bits, atomic max).
void launch_tensor_static(int dt, const void* x, int64_t n, const float* scale, uint8_t* q,
                          uint32_t* amax_acc, hipStream_t s);

// One delayed-scaling step on device-resident state (see fp8_delayed_scaling_update).
void launch_delayed_update(float* history, int len, uint32_t* amax_acc, int* step, int interval,
                           int margin, float* scale, hipStream_t s);
void launch_delayed_quantize(int dt, const void* x, int64_t n, float* history, int len,
                             uint32_t* amax_acc, int* step, int interval, int margin, float* scale,
                             float* scale_used, uint8_t* q, hipStream_t s);

void launch_debug_cast(const float* v, int64_t n, uint8_t* q, hipStream_t s);

// Measurement reference: q[i] = high byte of the 16-bit x[i] (the quantizers' byte mix).
void launch_byte_mix(const void* x, int64_t n, uint8_t* q, hipStream_t s);

// Grouped (mixture-of-experts) blockwise product, SM_BLOCK or SM_E8M0: expert e's rows
// [offsets[e], offsets[e + 1]) of A and C times qb[e] ([E][N][K]); offsets [E + 1] int32 on
// the device.  Returns false when the launch grid would be too large.
bool launch_grouped(int mode, int out_dt, const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb,
                    const int* offsets, int E, int T, int N, int K, void* c, hipStream_t s);

// One decode launch of a plan (kernels FP8_KERNEL_GEMV_*).  sa and sb point at float32
// scales, or at e8m0fnu bytes for SM_E8M0.  False for a launch it has no kernel for.
bool launch_gemv(int mode, int out_dt, const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa,
                 const uint8_t* qb, const void* sb, int M, int N, int K, void* c, hipStream_t s);

// The fused one-token step (plan::dynamic_fits(N, K)): x [K] quantized with the scheme of
// `mode` into qa [K] and sa, and C [N] = the one-token GEMM of that mode, in one launch.
void launch_gemv_dynamic(int mode, int in_dt, int out_dt, const void* x, const uint8_t* qb, const void* sb,
                         uint8_t* qa, void* sa, int N, int K, void* c, hipStream_t s);

// Scaled FP8 GEMM, C [M, N] of out_dt: the launches of plan_gemm(mode, M, N, K), in order.
// False (after the launches before it) for a launch it has no kernel for.
bool launch_gemm(int mode, int out_dt, const fp8_gemm_plan_t& p, const uint8_t* qa, const void* sa,
                 const uint8_t* qb, const void* sb, int M, int N, int K, void* c, hipStream_t s);

}  // namespace fp8amax
