// fp8_device.hpp - device helpers shared by the gfx950 kernels: 16-bit input unpacking,
// magnitude keys for amax, the e4m3fn encoder and 16-lane DPP reductions.
//
// Format and rules: "Что такое FP8 инференс на H100 (Transformer Engine)?", sections 2-3
// (E4M3 for inference, largest value 448, scale = amax / 448, divide then round to FP8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace fp8amax {

enum : int { DT_BF16 = 0, DT_F16 = 1 };

// Cache policy of a buffer load (the builtins' aux operand) for weights read exactly once in
// whole 1 KB runs per load instruction, as the one-token kernels stream them: non-temporal (nt).
// Measured with cold weights, outputs bit-identical: the fused one-token step 5-10% faster and
// the one-token GEMVs 5-8% faster than with the default policy.  The MFMA-fed kernels (2-128
// tokens) read each 128-byte weight line as two half-line loads; there nt was 7-11% slower, so
// they, and every operand that other workgroups read again, keep the default.
constexpr int kStreamOnce = 2;

// The factor a GEMM epilogue multiplies the float32 accumulator of C[m, n] by: `alpha`
// = sa * sb with one scale per tensor; sa[m] * sb[n] with one scale per row of A (token)
// and of B (output channel; the Transformer Engine page's per-channel scaling); `alpha`
// = 1 in the slab-scaled modes, whose scales were applied inside the K loop.
// For the fragment layout of the 16x16 MFMA outputs (lane l holds token row 16 i + l % 16
// and output columns 16 j + 4 (l / 16) + r) the rowwise factors are loaded when a kernel
// starts, so that the loads overlap its K loop instead of following it.  Rows and columns
// past the ends read the last entry (their outputs are not stored).
template <int SM, int MI, int NJ>
struct FragFactors {
  static constexpr bool kRow = SM == SM_ROW;
  float a[kRow ? MI : 1];
  float b[kRow ? NJ : 1][4];
  __device__ __forceinline__ void load(const float* sa, const float* sb, int m0, int n0, int M, int N) {
    if constexpr (kRow) {
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < MI; ++i) a[i] = sa[min(m0 + 16 * i + (lane & 15), M - 1)];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) b[j][r] = sb[min(n0 + 16 * j + 4 * (lane >> 4) + r, N - 1)];
    }
  }
  __device__ __forceinline__ float operator()(float alpha, int i, int j, int r) const {
    if constexpr (kRow) return a[i] * b[j][r];
    else return alpha;
  }
};

// Exact float32 value of a 16-bit input pattern (low 16 bits of `h`).
template <int DT>
__device__ __forceinline__ float in_to_f32(uint32_t h) {
  if constexpr (DT == DT_BF16) {
    return __uint_as_float(h << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
  }
}

// Magnitude key of a 16-bit float pattern: the pattern with its sign bit cleared.  For
// bf16 and fp16 alike, key order equals |x| order on finite values, +inf sorts above every
// finite value and NaN patterns sort above +inf, so an unsigned max over keys is amax with
// NaN propagation.  No rounding is involved.
__device__ __forceinline__ uint32_t key_max_pair(uint32_t m, uint32_t word) {
  const uint32_t lo = word & 0x7fffu;
  const uint32_t hi = (word >> 16) & 0x7fffu;
  return max(m, max(lo, hi));
}

constexpr uint32_t kCanonicalNaN = 0x7fc00000u;

// amax value of a magnitude key; a NaN key gives the canonical quiet NaN (NaN payloads
// carry no information and would otherwise depend on which NaN won the reduction).
template <int DT>
__device__ __forceinline__ float amax_from_key(uint32_t key) {
  constexpr uint32_t kInfKey = DT == DT_BF16 ? 0x7f80u : 0x7c00u;
  return key > kInfKey ? __uint_as_float(kCanonicalNaN) : in_to_f32<DT>(key);
}

// scale = amax / 448 as one IEEE float32 division (round to nearest even, subnormals
// kept; hipcc's default division is the correctly rounded sequence).  amax == 0 -> 1;
// NaN -> the canonical quiet NaN.
__device__ __forceinline__ float scale_from_amax(float amax) {
  if (amax != amax) return __uint_as_float(kCanonicalNaN);
  return amax == 0.0f ? 1.0f : amax / 448.0f;
}

// UE8M0 scale code of a block (e8m0fnu byte: 2^(code - 127), 255 = NaN; fine-grained
// FP8 page, UE8M0 scale format): the smallest power of two not below amax / 448, clamped
// to 2^-127 .. 2^127.  amax 0 -> 2^0 (code 127); NaN or infinite amax -> 255.
// Exact integer work on amax's bits: with amax = (1 + f) 2^E and 448 = 1.75 * 2^8,
// 448 * 2^e >= amax holds first at e = E - 8 when 1 + f <= 1.75 (fraction bits
// <= 0x600000) and at e = E - 7 otherwise.  A subnormal amax (< 2^-126) lies far below
// 448 * 2^-127, so its code is the smallest one.
__device__ __forceinline__ uint32_t e8m0_from_amax(float amax) {
  const uint32_t b = __float_as_uint(amax) & 0x7fffffffu;
  const uint32_t ef = b >> 23;
  if (ef == 0xffu) return 0xffu;
  if (ef == 0u) return b == 0u ? 127u : 0u;
  const int e = static_cast<int>(ef) - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return static_cast<uint32_t>(min(max(e, -127), 127) + 127);
}

// The float32 value of an e8m0fnu code: 2^(code - 127) exactly (code 0 is the float32
// subnormal 2^-127), code 255 the canonical NaN.
__device__ __forceinline__ float e8m0_value(uint32_t code) {
  if (code == 0xffu) return __uint_as_float(kCanonicalNaN);
  return code == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(code << 23);
}

// Byte (slab & 3) of a 32-bit word holding the UE8M0 scales of four consecutive K slabs
// (the packed layout of the UE8M0 scale tensors).
__device__ __forceinline__ int e8m0_byte(uint32_t word, int slab) {
  return static_cast<int>((word >> (8 * (slab & 3))) & 0xffu);
}

// Saturating round-to-nearest-even encode of a float32 to an OCP e4m3fn code.
//   NaN -> 0x7F; |v| >= 448 (inf included) -> 0x7E with v's sign; the sign of zero and of
//   values that round to zero is kept.
// Normal range (|v| >= 2^-6): round the float32 significand to 3 bits with the usual
// add-half-minus-one-plus-lsb trick, then rebias the exponent from 127 to 7.
// Subnormal range (|v| < 2^-6): e4m3 subnormals are multiples of 2^-9; adding 2^14 (whose
// float32 ulp is 2^-9) rounds |v| to that grid with the FPU's round-to-nearest-even, and
// the low bits of the sum are the code (8 = 2^-6 when it rounds up to the first normal).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x3c800000u) {                              // |v| >= 2^-6
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = min((r >> 20) - (120u << 3), 0x7eu);        // saturate at 448 (covers inf)
  } else {
    const float t = __uint_as_float(a) + 16384.0f;     // 2^14
    code = __float_as_uint(t) - 0x46800000u;           // bits of 2^14
  }
  code |= sign;
  return a > 0x7f800000u ? 0x7fu : code;               // NaN
}

// ------------------------------------------------------------------------------------
// Fast quotient + encode, used when the scale s is finite and s >= 2^-100.
//   r = RN(1/s) once per group; per element q0 = RN(x*r), rem = x - q0*s (exact, one
//   FMA), q = RN(q0 + rem*r) is the correctly rounded x/s (Markstein's correction step;
//   a correctly rounded reciprocal and a quotient within one ulp give the correctly
//   rounded quotient when nothing under- or overflows, which s >= 2^-100 and
//   |x| <= 448*s guarantee for every value that can encode to a non-zero code).
//   copysign restores the sign of x when x = -0 (the FMA sum of +0 and -0 is +0).
//   The clamp to +-448 makes the hardware conversion saturate; v_cvt_pk_fp8_f32 then
//   rounds to nearest even exactly as e4m3_encode does (checked over every finite
//   float32 input), and no NaN reaches this path.
// The GPU tests check the codes of this path bit for bit against the oracle (IEEE division,
// then the value-search encoder) for every finite bf16 and fp16 amax, with x taken across
// each group's range, for all 65536 patterns of both formats at several scales, and for the
// conversion alone on every float32 input.
constexpr float kFastScaleMin = 0x1p-100f;

__device__ __forceinline__ bool fast_scale(float s) {
  return s >= kFastScaleMin && s <= 3.40282347e38f;   // false for NaN and inf
}

__device__ __forceinline__ float quot_fast(float x, float s, float r) {
  const float q0 = x * r;
  const float rem = __builtin_fmaf(-q0, s, x);
  const float q = __builtin_copysignf(__builtin_fmaf(rem, r, q0), x);
  return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
}

// Four quotients -> four e4m3 codes packed little-endian in one dword.
__device__ __forceinline__ uint32_t cvt4(float q0, float q1, float q2, float q3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, lo, true));
}

// DPP lane moves within rows of 16 lanes (bound_ctrl off, all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, false));
}

// Max over each aligned group of 16 lanes; every lane of the group gets the result.
// quad_perm(1,0,3,2) and quad_perm(2,3,0,1) reduce each quad, row_half_mirror joins the
// two quads of each half-row, row_mirror joins the two half-rows.
__device__ __forceinline__ uint32_t max16(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));   // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));   // row_mirror
  return v;
}

// Max over each aligned group of 8 lanes (the first three steps of max16).
__device__ __forceinline__ uint32_t max8(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));   // row_half_mirror
  return v;
}

// Sum of v over the 64 lanes of the wave, the same value in every lane (wave-uniform): DPP
// adds within each row of 16 lanes (quads, half-rows, rows), then the four row sums read
// with readlane.  No LDS crossbar (ds_bpermute) round trips, which a __shfl_xor butterfly
// would take at every step.
__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));    // quad_perm [1,0,3,2]
  v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));    // quad_perm [2,3,0,1]
  v += __uint_as_float(dpp_u32<0x141>(__float_as_uint(v)));   // row_half_mirror
  v += __uint_as_float(dpp_u32<0x140>(__float_as_uint(v)));   // row_mirror
  // readlane moves 32-bit integers: the float travels as its bits
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// Max over the whole wave (64 lanes); every lane gets the result.
__device__ __forceinline__ uint32_t max64(uint32_t v) {
  v = max16(v);
  v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 16)));
  v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 32)));
  return v;
}

}  // namespace fp8amax
