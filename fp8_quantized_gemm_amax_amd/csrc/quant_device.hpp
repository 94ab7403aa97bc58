// quant_device.hpp - element-wise steps of the quantizers, shared by every kernel that
// writes e4m3 codes (the quantize kernels and the fused one-token decode step): 16-byte
// loads of eight 16-bit inputs, their magnitude keys, the cast of eight inputs with a
// group's scale (the fast quotient or the exact path), and a group's scale and its store.
//
// Steps: Transformer Engine page "Что такое FP8 инференс на H100 (Transformer Engine)?",
// section 3 steps 2-4 (amax, scale = amax / 448, x / scale rounded to e4m3); UE8M0
// scales from the fine-grained FP8 page ("FP8 chi tiết", UE8M0 scale format).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8_device.hpp"

namespace fp8amax {

struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 load16(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return {v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ uint32_t key8(const U4& v) {
  uint32_t m = key_max_pair(0u, v.x);
  m = key_max_pair(m, v.y);
  m = key_max_pair(m, v.z);
  return key_max_pair(m, v.w);
}

template <int DT>
__device__ __forceinline__ float lo16(uint32_t w) { return in_to_f32<DT>(w & 0xffffu); }
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w) { return in_to_f32<DT>(w >> 16); }

// Exact path: IEEE division and the software encoder, element by element.  Used for
// groups whose scale is NaN, infinite or below 2^-100.
template <int DT>
__device__ __forceinline__ uint32_t enc4_exact(uint32_t w0, uint32_t w1, float s) {
  return e4m3_encode(lo16<DT>(w0) / s) | (e4m3_encode(hi16<DT>(w0) / s) << 8) |
         (e4m3_encode(lo16<DT>(w1) / s) << 16) | (e4m3_encode(hi16<DT>(w1) / s) << 24);
}

template <int DT>
__device__ __forceinline__ uint32_t enc4_fast(uint32_t w0, uint32_t w1, float s, float r) {
  return cvt4(quot_fast(lo16<DT>(w0), s, r), quot_fast(hi16<DT>(w0), s, r),
              quot_fast(lo16<DT>(w1), s, r), quot_fast(hi16<DT>(w1), s, r));
}

// Eight 16-bit inputs -> eight e4m3 codes.  `fast` = fast_scale(s), r = 1/s.
template <int DT>
__device__ __forceinline__ uint2 enc8(const U4& v, float s, float r, bool fast) {
  if (fast) return make_uint2(enc4_fast<DT>(v.x, v.y, s, r), enc4_fast<DT>(v.z, v.w, s, r));
  return make_uint2(enc4_exact<DT>(v.x, v.y, s), enc4_exact<DT>(v.z, v.w, s));
}

// One element (ragged paths).
template <int DT>
__device__ __forceinline__ uint8_t enc1(uint32_t h, float s, float r, bool fast) {
  const float x = in_to_f32<DT>(h);
  if (fast) {
    const float q = quot_fast(x, s, r);
    return static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false) & 0xff);
  }
  return static_cast<uint8_t>(e4m3_encode(x / s));
}

// A group's scale from its amax, and the value stored for it: the float32 scale amax / 448,
// or (E8M0) the power-of-two scale and its e8m0fnu code.
template <bool E8M0>
struct GroupScale {
  float scale;
  uint32_t code;
  __device__ __forceinline__ explicit GroupScale(float amax) {
    if constexpr (E8M0) {
      code = e8m0_from_amax(amax);
      scale = e8m0_value(code);
    } else {
      scale = scale_from_amax(amax);
      code = 0;
    }
  }
  // Store the scale of group (row, col) of a grid with `ncols` groups per row: float32
  // rows are ncols long; UE8M0 rows are `stride` bytes (ncols rounded up to whole 32-bit
  // words), and the group that ends a row also sets the row's padding bytes to 127 (2^0).
  __device__ __forceinline__ void store(void* out, int64_t row, int64_t col, int64_t ncols,
                                        int64_t stride) const {
    if constexpr (E8M0) {
      uint8_t* o = static_cast<uint8_t*>(out) + row * stride;
      o[col] = static_cast<uint8_t>(code);
      if (col == ncols - 1)
        for (int64_t p = ncols; p < stride; ++p) o[p] = 127;
    } else {
      static_cast<float*>(out)[row * ncols + col] = scale;
    }
  }
};

}  // namespace fp8amax
