// gemm_common.hpp - pieces shared by the tiled FP8 GEMM kernels for gfx950: operand types,
// the FP8 MFMA wrappers, output conversion, the LDS slab swizzle and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8_device.hpp"
#include "launch.hpp"

namespace fp8amax {
namespace gemm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kSlab = 128;
constexpr uint32_t kOOB = 0x80000000u;     // buffer offset past any range: the load returns zeros

// LDS layout of a slab tile, [rows][128 B]: the 16-byte chunk c of row r is stored at chunk
// position c ^ swz(r), swz being linear (over GF(2)) in the row's low four bits.  A fragment
// read takes one 16-byte chunk from each of 16 consecutive rows per group of 16 lanes; with
// this swizzle no group of a ds_read_b128 hits an LDS bank twice.  Measured on gfx950 with
// the bank-conflict counter (SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE): 4 LDS cycles per
// fragment read, against 8 with the swizzle (r >> 1) & 7, r & 7 or a row rotation, and 16
// with none.  Each row keeps its own 128 bytes, so an LDS DMA instruction still writes eight
// whole rows.
__host__ __device__ constexpr int swz(int row) {
  return ((row & 1) ? 1 : 0) ^ ((row & 2) ? 4 : 0) ^ ((row & 4) ? 1 : 0) ^ ((row & 8) ? 3 : 0);
}

// The logical chunk lane `lane` of an LDS DMA instruction fetches: instruction g writes rows
// 8g .. 8g + 7 as one contiguous KB, lane i at row 8g + i / 8, chunk position i % 8.  swz
// depends on bit 3 of the row only through g's parity, so a lane has one chunk for even and
// one for odd instructions.
__host__ __device__ constexpr int dma_chunk(int lane, int odd) { return (lane & 7) ^ swz(8 * odd + (lane >> 3)); }

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz = blgp = 0: both operands e4m3; E8M0 scale 127 = 2^0 on both.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The same product with E8M0 block scales: each lane's 32 K positions of the first operand
// are scaled by 2^(ea - 127) and those of the second by 2^(eb - 127) (measured on gfx950:
// a lane's scale byte covers exactly the 32 K positions it holds, for both operands).
__device__ __forceinline__ v4f mfma_fp8_e8m0(const v8i& a, const v8i& b, const v4f& c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;                     // nearest even
}

template <int OUT>
__device__ __forceinline__ uint32_t f32_to_out_bits(float f) {
  if constexpr (OUT == DT_BF16) {
    return f32_to_bf16_bits(f);
  } else {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(f)));
  }
}

// Tile order: workgroup b runs on XCD b % 8; consecutive tiles of a grouped order
// (groups of kGroupM tile rows) are given to the same XCD so its L2 serves their shared
// A rows and B columns.
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total / kXcds, r = total % kXcds;
  const int x = b % kXcds, i = b / kXcds;
  const int logical = x * q + min(x, r) + i;
  const int per_group = kGroupM * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_g = logical - g * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

}  // namespace gemm
}  // namespace fp8amax
