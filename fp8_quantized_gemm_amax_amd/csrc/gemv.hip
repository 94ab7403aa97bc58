// gemv.hip - the decode regime (M <= 16 tokens) of the scaled FP8 GEMM, for gfx950.
//
// Same operation as gemm.hip (Transformer Engine page "Что такое FP8 инференс на H100
// (Transformer Engine)?", section 3 steps 5-6; per-slab scales from "FP8 chi tiết",
// opening bullets), in the regime the task page times (batch 1): the weights are read once
// and the product is bound by HBM bandwidth, so the kernel is built around streaming W.
//
// Design: a workgroup owns 16 * NB rows of W and its WAVES waves split the K slabs
// between them.  Nothing goes through LDS on the way in: each wave streams its W slabs
// straight from HBM into MFMA operand registers with 16-byte buffer loads, and fetches the
// matching activation fragment (at most 16 rows, L2-resident after the first workgroup)
// the same way.  The loads form a rolling pipeline: the registers of slab s are refilled
// with slab s + UNROLL as soon as slab s has been multiplied, so UNROLL slabs stay in
// flight per wave with no barrier in the loop.  Rows past M or N and bytes past K read as
// zero through the buffer range check.  One v_mfma_scale_f32_16x16x128_f8f6f4 per slab and
// row block (W as the first operand, A padded to 16 rows as the second) gives lane l the
// partial sums of C[m = l % 16][n = n0 + 16 j + 4 (l / 16) + r].  The waves' K shares are
// summed in LDS and the epilogue scales and stores.
#include "fp8_device.hpp"
#include "gemm_plan.hpp"
#include "launch.hpp"
#include "quant_device.hpp"

namespace fp8amax {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kSlab = 128;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOOB = 0x80000000u;     // offset past any range: the load returns zeros

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// With E8M0 block scales: a lane's 32 K positions of the first operand times 2^(ea - 127),
// of the second times 2^(eb - 127).
__device__ __forceinline__ v4f mfma_fp8_e8m0(const v8i& a, const v8i& b, const v4f& c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int OUT>
__device__ __forceinline__ uint32_t f32_to_out_bits(float f) {
  if constexpr (OUT == DT_BF16) return f32_to_bf16_bits(f);
  else return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(f)));
}

__device__ __forceinline__ v8i load32(const __amdgpu_buffer_rsrc_t& r, uint32_t off_lo, uint32_t off_hi) {
  const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(r, off_lo, 0, 0);
  const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(r, off_hi, 0, 0);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// WAVES waves split K; each holds UNROLL slabs in flight and multiplies NB row blocks of
// 16 weight rows by MB activation fragments of 16 tokens.  Slabs go to the waves in turn
// (slab s to wave s % WAVES), so at any moment a workgroup reads WAVES * 128 contiguous
// bytes of each of its rows.  A workgroup's rows may straddle a 128-row weight block; the
// blockwise scale of each row block is looked up on its own.
template <int SM, int OUT, int WAVES, int UNROLL, int NB, int MB>
__global__ __launch_bounds__(WAVES * 64) void gemv_fp8_kernel(
    const uint8_t* __restrict__ qa, const void* __restrict__ sa_, const uint8_t* __restrict__ qb,
    const void* __restrict__ sb_, int M, int N, int K, uint16_t* __restrict__ c) {
  constexpr bool BLOCKWISE = slab_scaled(SM);
  constexpr bool E8M0 = SM == SM_E8M0;
  const float* __restrict__ sa = static_cast<const float*>(sa_);
  const float* __restrict__ sb = static_cast<const float*>(sb_);
  __shared__ v4f red[WAVES > 1 ? (WAVES - 1) * NB * MB * 64 : 1];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int r16 = lane & 15, kq = lane >> 4;
  const int n0 = blockIdx.x * 16 * NB;
  const int nslabs = (K + kSlab - 1) / kSlab;
  FragFactors<SM, MB, NB> ff;                                 // rowwise epilogue scales, fetched now
  ff.load(sa, sb, 0, n0, M, N);
  const int KG = K / kSlab;                                   // blockwise: K % 128 == 0
  const int KG4 = static_cast<int>(e8m0_row_bytes(KG));      // UE8M0: bytes per scale row
  const int SR = E8M0 ? KG4 : KG * 4;                         // bytes per scale row
  const int count = (nslabs - w + WAVES - 1) / WAVES;         // this wave's slabs
  const int iters = (count + UNROLL - 1) / UNROLL;

  // W rows n0 .. n0 + 16 NB - 1 and the M activation rows as buffers; a lane reads the
  // 32 bytes of quarter kq of a slab in row r16 of a block.  plan_gemm keeps 16 NB K and
  // 16 K below 2^31, so every offset fits the 32-bit buffer offset.
  const int rows = min(16 * NB, N - n0);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qb + static_cast<int64_t>(n0) * K), static_cast<short>(0), rows * K,
      static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qa), static_cast<short>(0), M * K, static_cast<int>(kRsrcWord3));
  // blockwise scales: sa [M][KG] and the rows of sb [ceil(N/128)][KG] of the weight blocks
  // nb0 .. nb1 this workgroup touches (float32, or UE8M0 bytes in rows of KG4)
  const int nb0 = n0 / kSlab, nb1 = (n0 + rows - 1) / kSlab;
  const __amdgpu_buffer_rsrc_t sar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(sa_), static_cast<short>(0), BLOCKWISE ? M * SR : 0,
      static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t sbr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(sb_) + (BLOCKWISE ? static_cast<int64_t>(nb0) * SR : 0)),
      static_cast<short>(0), BLOCKWISE ? (nb1 - nb0 + 1) * SR : 0, static_cast<int>(kRsrcWord3));

  // operands of this wave's i-th slab; past the wave's share every load reads zeros (the
  // scales too, so such a slab adds 0 * 0 and a non-finite scale elsewhere cannot leak in)
  // UE8M0: sav / sbv hold the 32-bit words with the slab's scale bytes, slab[u] the slab
  v8i wf[UNROLL][NB], af[UNROLL][MB];
  float sav[UNROLL][MB], sbv[UNROLL][NB];
  int slab[UNROLL];
  auto fetch = [&](int i, int u) {
    const bool live = i < count;                              // wave-uniform
    const int s = w + i * WAVES;
    slab[u] = s;
    const int kk = s * kSlab + kq * 32;
    const bool lo_in = live && kk < K, hi_in = live && kk + 16 < K;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int row = 16 * j + r16;
      const uint32_t off = static_cast<uint32_t>(row * K + kk);
      wf[u][j] = load32(wr, (lo_in && row < rows) ? off : kOOB, (hi_in && row < rows) ? off + 16 : kOOB);
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int m = 16 * b + r16;
      const uint32_t aoff = static_cast<uint32_t>(m * K + kk);
      af[u][b] = load32(ar, (lo_in && m < M) ? aoff : kOOB, (hi_in && m < M) ? aoff + 16 : kOOB);
    }
    if constexpr (BLOCKWISE) {
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int m = 16 * b + r16;
        const uint32_t soff = static_cast<uint32_t>(m * SR + (E8M0 ? (s & ~3) : s * 4));
        sav[u][b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sar, (live && m < M) ? soff : kOOB, 0, 0));
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint32_t soff = static_cast<uint32_t>(((n0 + 16 * j) / kSlab - nb0) * SR + (E8M0 ? (s & ~3) : s * 4));
        sbv[u][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sbr, (live && 16 * j < rows) ? soff : kOOB, 0, 0));
      }
    }
  };

  // The first pass multiplies zero registers while the first UNROLL slabs load; from then
  // on pass p multiplies slabs (p - 1) UNROLL + u and refetches into the same registers.
  // Entering the loop with no load pending lets the compiler keep the steady-state wait
  // (only the oldest slab's loads) instead of draining every load at the loop head.
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
    for (int b = 0; b < MB; ++b) { af[u][b] = v8i{0, 0, 0, 0, 0, 0, 0, 0}; sav[u][b] = 0.0f; }
#pragma unroll
    for (int j = 0; j < NB; ++j) { wf[u][j] = v8i{0, 0, 0, 0, 0, 0, 0, 0}; sbv[u][j] = 0.0f; }
    slab[u] = 0;
  }
  v4f acc[NB][MB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[j][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  auto consume = [&](int u) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        if constexpr (E8M0) {
          acc[j][b] = mfma_fp8_e8m0(wf[u][j], af[u][b], acc[j][b], e8m0_byte(__float_as_uint(sbv[u][j]), slab[u]),
                                    e8m0_byte(__float_as_uint(sav[u][b]), slab[u]));
        } else if constexpr (BLOCKWISE) {
          const float scale = sav[u][b] * sbv[u][j];
          const v4f p = mfma_fp8(wf[u][j], af[u][b], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][b][r] = __builtin_fmaf(p[r], scale, acc[j][b][r]);
        } else {
          acc[j][b] = mfma_fp8(wf[u][j], af[u][b], acc[j][b]);
        }
      }
  };
  // pass `it` multiplies slabs (it - 1) UNROLL + u of this wave and refills with
  // it UNROLL + u; the last pass only multiplies
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      consume(u);
      fetch(it * UNROLL + u, u);
      __builtin_amdgcn_sched_barrier(0);   // refill slot u before the next slot's math
    }
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) consume(u);

  // sum the waves' K shares in LDS (wave 0 adds waves 1 .. WAVES-1 in order)
  if constexpr (WAVES > 1) {
    if (w > 0) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b) red[(((w - 1) * NB + j) * MB + b) * 64 + lane] = acc[j][b];
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int q = 1; q < WAVES; ++q)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          const v4f o = red[(((q - 1) * NB + j) * MB + b) * 64 + lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][b][r] += o[r];
        }
  }
  float alpha = 1.0f;
  if constexpr (SM == SM_TENSOR) alpha = sa[0] * sb[0];
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int m = 16 * b + r16;
    if (m >= M) continue;
    uint16_t* crow = c + static_cast<int64_t>(m) * N;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + 16 * j + 4 * kq;
      uint32_t h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = f32_to_out_bits<OUT>(acc[j][b][r] * ff(alpha, b, j, r));
      if ((N & 3) == 0 && n + 3 < N) {
        *reinterpret_cast<uint2*>(crow + n) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) crow[n + r] = static_cast<uint16_t>(h[r]);
      }
    }
  }
}

// Few-token kernel (M <= MT <= 4) on the vector ALUs.  A wave owns RPW whole weight rows
// and walks K in 1 KB chunks: each 16-byte load of a lane is bytes [1024 c + 16 l, +16) of
// one row, so every load instruction streams 1 KB of contiguous HBM (the access pattern that
// keeps HBM busiest) and no LDS is involved.  The 16 codes are widened exactly to f16
// (every e4m3 value is an f16 normal) and multiplied with v_dot2c_f32_f16, which forms the
// products exactly and accumulates in float32.  A lane's 16 K positions lie in one
// 128-wide slab, so the blockwise scale sa[m, g] * sb[n / 128, g] is applied to each
// lane's 16-term partial.  At the end the 64 lanes' partials of each (m, row) are summed
// with DPP within rows of 16 lanes and readlane across them (wave_sum).  The float32 sum is
// ordered differently from the MFMA path; both are within the product tolerance of the
// exact sum.
template <int SM, int OUT, int MT, int RPW, int UNROLL>
__global__ __launch_bounds__(256) void gemv_valu_kernel(
    const uint8_t* __restrict__ qa, const void* __restrict__ sa_, const uint8_t* __restrict__ qb,
    const void* __restrict__ sb_, int M, int N, int K, uint16_t* __restrict__ c) {
  constexpr bool BLOCKWISE = slab_scaled(SM);
  constexpr bool E8M0 = SM == SM_E8M0;
  const float* __restrict__ sa = static_cast<const float*>(sa_);
  const float* __restrict__ sb = static_cast<const float*>(sb_);
  static_assert(MT * RPW <= 64 && 128 % RPW == 0, "one output per lane; a wave's rows share a weight block");
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = (blockIdx.x * 4 + w) * RPW;
  if (row0 >= N) return;                                      // no barrier in this kernel
  const int rows = min(RPW, N - row0);
  // rowwise: the factor of the output this lane stores (lane m * RPW + r writes C[m, row0 + r]),
  // fetched now so that the load overlaps the K loop
  float row_factor = 1.0f;
  if constexpr (SM == SM_ROW)
    row_factor = sa[min(lane / RPW, M - 1)] * sb[row0 + min(lane % RPW, rows - 1)];
  const int KG = K / kSlab;                                   // blockwise: K % 128 == 0
  const int SR = E8M0 ? static_cast<int>(e8m0_row_bytes(KG)) : KG * 4;   // bytes per scale row
  const int nch = (K + 1023) / 1024;
  const int iters = (nch + UNROLL - 1) / UNROLL;

  // RPW K and M K stay below 2^31 (plan_gemm checks 32 K), so offsets fit 32 bits
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qb + static_cast<int64_t>(row0) * K), static_cast<short>(0), rows * K,
      static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qa), static_cast<short>(0), M * K, static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t sar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(sa_), static_cast<short>(0), BLOCKWISE ? M * SR : 0,
      static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t sbr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(sb_) + (BLOCKWISE ? static_cast<int64_t>(row0 / kSlab) * SR : 0)),
      static_cast<short>(0), BLOCKWISE ? SR : 0, static_cast<int>(kRsrcWord3));

  // operands of chunk i in slot u; past the last chunk every load reads zeros (the scales
  // too, so such a chunk adds 0 * 0).  UE8M0: sav / sbv hold the 32-bit words with the
  // scale bytes of this lane's slab, gsl[u] that slab.
  v4i wv[UNROLL][RPW], av[UNROLL][MT];
  float sav[UNROLL][MT], sbv[UNROLL];
  int gsl[UNROLL];
  auto fetch = [&](int i, int u) {
    const int col = i * 1024 + lane * 16;
    const bool in = (i < nch) & (col < K);                   // K % 16 == 0
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      wv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wr, (in & (r < rows)) ? static_cast<uint32_t>(r * K + col) : kOOB, 0,
                                                       kStreamOnce);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      av[u][m] = __builtin_amdgcn_raw_buffer_load_b128(ar, (in & (m < M)) ? static_cast<uint32_t>(m * K + col) : kOOB, 0, 0);
    if constexpr (BLOCKWISE) {
      const int g = col >> 7;
      const int goff = E8M0 ? (g & ~3) : g * 4;
      gsl[u] = g;
#pragma unroll
      for (int m = 0; m < MT; ++m)
        sav[u][m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            sar, (in & (m < M)) ? static_cast<uint32_t>(m * SR + goff) : kOOB, 0, 0));
      sbv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sbr, in ? static_cast<uint32_t>(goff) : kOOB, 0, 0));
    }
  };

  // Same rolling scheme as the MFMA kernel: pass 0 multiplies zero registers while the
  // first UNROLL chunks load, so the loop is entered with no load pending.
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) wv[u][r] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < MT; ++m) { av[u][m] = v4i{0, 0, 0, 0}; sav[u][m] = 0.0f; }
    sbv[u] = 0.0f;
    gsl[u] = 0;
  }
  float acc[MT][RPW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[m][r] = 0.0f;

  auto consume = [&](int u) {
    h2 ah[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        ah[m][2 * d] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(av[u][m][d], 1.0f, false);
        ah[m][2 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(av[u][m][d], 1.0f, true);
      }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      h2 wh[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        wh[2 * d] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wv[u][r][d], 1.0f, false);
        wh[2 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wv[u][r][d], 1.0f, true);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float d = BLOCKWISE ? 0.0f : acc[m][r];
#pragma unroll
        for (int p = 0; p < 8; ++p) d = __builtin_amdgcn_fdot2(wh[p], ah[m][p], d, false);
        if constexpr (E8M0) {
          // d * 2^(ea - 127) * 2^(eb - 127) in one exact step; a NaN code gives NaN
          const int ea = e8m0_byte(__float_as_uint(sav[u][m]), gsl[u]);
          const int eb = e8m0_byte(__float_as_uint(sbv[u]), gsl[u]);
          const float t = (ea == 0xff || eb == 0xff) ? __uint_as_float(kCanonicalNaN)
                                                     : __builtin_amdgcn_ldexpf(d, ea + eb - 254);
          acc[m][r] += t;
        } else if constexpr (BLOCKWISE) {
          acc[m][r] = __builtin_fmaf(d, sav[u][m] * sbv[u], acc[m][r]);
        } else {
          acc[m][r] = d;
        }
      }
    }
  };
  // pass `it` multiplies chunks (it - 1) UNROLL + u and refills with it UNROLL + u; the
  // last pass only multiplies (its refills would all be past the end)
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      consume(u);
      fetch(it * UNROLL + u, u);
      __builtin_amdgcn_sched_barrier(0);   // refill slot u before the next slot's math
    }
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) consume(u);

  // sum over the 64 lanes; every lane ends with every total
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[m][r] = wave_sum(acc[m][r]);

  float alpha = 1.0f;
  if constexpr (SM == SM_TENSOR) alpha = sa[0] * sb[0];
  // lane m * RPW + r writes C[m, row0 + r]
  float mine = 0.0f;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      if (lane == m * RPW + r) mine = acc[m][r];
  const int m = lane / RPW, r = lane % RPW;
  if (lane < MT * RPW && m < M && r < rows)
    c[static_cast<int64_t>(m) * N + row0 + r] =
        static_cast<uint16_t>(f32_to_out_bits<OUT>(mine * (SM == SM_ROW ? row_factor : alpha)));
}

// One token on the vector ALUs, persistent: a grid that fills the chip; wave gw takes rows
// gw, gw + waves, ...  The activation row (NCH 1 KB chunks, K <= 1024 NCH) and its scales
// are loaded into registers once and reused for every row.  The NCH chunk loads of the next
// row are issued as soon as the current row's chunks have been multiplied, so a whole row
// stays in flight while the current row's 64 lane partials are reduced and stored.  The
// arithmetic per chunk is that of gemv_valu_kernel.
template <int SM, int OUT, int NCH>
__global__ __launch_bounds__(256) void gemv1_stream_kernel(
    const uint8_t* __restrict__ qa, const void* __restrict__ sa_, const uint8_t* __restrict__ qb,
    const void* __restrict__ sb_, int N, int K, uint16_t* __restrict__ c, int waves) {
  constexpr bool BLOCKWISE = slab_scaled(SM);
  constexpr bool E8M0 = SM == SM_E8M0;
  const float* __restrict__ sa = static_cast<const float*>(sa_);
  const float* __restrict__ sb = static_cast<const float*>(sb_);
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= N) return;                                        // no barrier in this kernel
  const int KG = K / kSlab;                                   // blockwise: K % 128 == 0
  const int SR = E8M0 ? static_cast<int>(e8m0_row_bytes(KG)) : KG * 4;   // bytes per scale row

  // N K < 2^31 (plan_gemm checks), so every offset fits 32 bits
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qb), static_cast<short>(0), N * K, static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qa), static_cast<short>(0), K, static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t sar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(sa_), static_cast<short>(0), BLOCKWISE ? SR : 0, static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t sbr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(sb_), static_cast<short>(0), BLOCKWISE ? ((N + kSlab - 1) / kSlab) * SR : 0,
      static_cast<int>(kRsrcWord3));

  v4i av[NCH], wv[NCH];
  float sav[NCH], sbv[NCH];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int col = ch * 1024 + lane * 16;
    av[ch] = __builtin_amdgcn_raw_buffer_load_b128(ar, col < K ? static_cast<uint32_t>(col) : kOOB, 0, 0);
    if constexpr (BLOCKWISE) {
      const int g = min(col, K - 1) >> 7;
      sav[ch] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          sar, static_cast<uint32_t>(E8M0 ? (g & ~3) : g * 4), 0, 0));
    }
  }
  auto fetch = [&](int row, int ch) {                         // chunk ch of row (row >= N: zeros)
    const int col = ch * 1024 + lane * 16;
    const bool in = (row < N) & (col < K);                    // K % 16 == 0
    // unsigned: rows past N (their offsets are not used) would overflow int
    wv[ch] = __builtin_amdgcn_raw_buffer_load_b128(
        wr, in ? static_cast<uint32_t>(row) * static_cast<uint32_t>(K) + static_cast<uint32_t>(col) : kOOB, 0, kStreamOnce);
    if constexpr (BLOCKWISE) {
      const int g = min(col, K - 1) >> 7;
      sbv[ch] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          sbr, in ? static_cast<uint32_t>((row / kSlab) * SR + (E8M0 ? (g & ~3) : g * 4)) : kOOB, 0, 0));
    }
  };
  float alpha = 1.0f;
  if constexpr (SM == SM_TENSOR) alpha = sa[0] * sb[0];
  const float a_row = SM == SM_ROW ? sa[0] : 1.0f;

#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) fetch(gw, ch);
  for (int row = gw; row < N; row += waves) {
    float acc = 0.0f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      float d = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const h2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wv[ch][q], 1.0f, false);
        const h2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wv[ch][q], 1.0f, true);
        const h2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(av[ch][q], 1.0f, false);
        const h2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(av[ch][q], 1.0f, true);
        d = __builtin_amdgcn_fdot2(w0, a0, d, false);
        d = __builtin_amdgcn_fdot2(w1, a1, d, false);
      }
      if constexpr (E8M0) {
        const int g = min(ch * 1024 + lane * 16, K - 1) >> 7;
        const int ea = e8m0_byte(__float_as_uint(sav[ch]), g);
        const int eb = e8m0_byte(__float_as_uint(sbv[ch]), g);
        acc += (ea == 0xff || eb == 0xff) ? __uint_as_float(kCanonicalNaN) : __builtin_amdgcn_ldexpf(d, ea + eb - 254);
      } else if constexpr (BLOCKWISE) {
        acc = __builtin_fmaf(d, sav[ch] * sbv[ch], acc);
      } else {
        acc += d;
      }
      fetch(row + waves, ch);                                  // the same chunk of the next row
      __builtin_amdgcn_sched_barrier(0);
    }
    acc = wave_sum(acc);
    const float f = SM == SM_ROW ? a_row * sb[row] : alpha;
    if (lane == 0) c[row] = static_cast<uint16_t>(f32_to_out_bits<OUT>(acc * f));
  }
}

// The whole one-token step in one launch: quantize the activation row x[K] dynamically and
// multiply it with the weights.  Every workgroup first quantizes the whole activation row
// itself: wave w owns the row's 1 KB chunks w, w + WAVES, ... (sixteen elements per lane),
// reduces their amax (the row's, across the workgroup through LDS, for one scale per tensor or
// per row; eight lanes' worth for a 1x128 group), casts them with the quantizers' own element
// steps, and leaves the codes widened to f16 in LDS (exact: every e4m3 value is an f16 normal
// or zero) with the group scales beside them.  Every workgroup derives the same codes and
// scales from the same x; workgroup 0 stores them.  Each wave then multiplies weight rows as
// gemv_valu_kernel does: the same f16 dot products in the same order and the same scale
// arithmetic, so C is bit for bit what the quantize launch and the one-token GEMV give (a NaN
// output is a NaN in both; its sign and payload follow the compiler's operand order).
//   STREAM = false: workgroup b takes rows WAVES b .. WAVES b + WAVES - 1, one per wave.
//   STREAM = true: a grid of `waves` waves; wave gw takes rows gw, gw + waves, ..., each chunk
//     of the next row loaded as soon as the current row's chunk has been multiplied, so the
//     row is quantized once per workgroup instead of once per WAVES rows.
// The activation loads are issued first: x is L2-resident after the first workgroups, and
// loads return in order, so the weight loads issued after them do not hold them up while the
// first weight row streams in during the quantize.  Chunks past K (NCH is K / 1 KB rounded up
// to 2, 4 or 8) load nothing and add zero.
template <int SM, int DT, int OUT, int NCH, int WAVES, bool STREAM>
__global__ __launch_bounds__(WAVES * 64) void gemv1_dynamic_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ qb, const void* __restrict__ sb_,
    uint8_t* __restrict__ qa, void* __restrict__ sa_, int N, int K, uint16_t* __restrict__ c, int waves) {
  constexpr int CPW = (NCH + WAVES - 1) / WAVES;             // activation chunks per wave
  constexpr bool GROUPS = slab_scaled(SM);
  constexpr bool E8M0 = SM == SM_E8M0;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  __shared__ __attribute__((aligned(16))) v4i alo[NCH][64];   // f16 of a lane's codes 0..7
  __shared__ __attribute__((aligned(16))) v4i ahi[NCH][64];   // and 8..15
  __shared__ float gsc[GROUPS ? NCH * 8 : 1];                   // group scales (UE8M0: the codes' bits)
  __shared__ uint32_t wkey[WAVES];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = blockIdx.x * WAVES + w;                    // the wave's first (or only) row
  const int KG = K / kSlab;                                   // groups: K % 128 == 0
  const int SR = E8M0 ? static_cast<int>(e8m0_row_bytes(KG)) : KG * 4;   // bytes per scale row

  // the wave's activation chunks; K % 16 == 0, so a lane's sixteen elements are all in or out
  U4 v0[CPW], v1[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int xcol = (w + j * WAVES) * 1024 + lane * 16;
    v0[j] = U4{0u, 0u, 0u, 0u};
    v1[j] = U4{0u, 0u, 0u, 0u};
    if (xcol < K) {
      v0[j] = load16(x + xcol);
      v1[j] = load16(x + xcol + 8);
    }
  }
  // the first weight row (and its block scales), every chunk in flight during the quantize;
  // N K < 2^31 (plan::dynamic_fits), so every offset fits 32 bits
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qb), static_cast<short>(0), N * K, static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t sbr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(sb_), static_cast<short>(0), GROUPS ? ((N + kSlab - 1) / kSlab) * SR : 0,
      static_cast<int>(kRsrcWord3));
  v4i wv[NCH];
  float sbv[NCH];
  auto fetch = [&](int row, int ch) {                         // chunk ch of a row (row >= N: zeros)
    const int col = ch * 1024 + lane * 16;
    const bool in = (row < N) & (col < K);
    // unsigned: rows past N (their offsets are not used) would overflow int
    wv[ch] = __builtin_amdgcn_raw_buffer_load_b128(
        wr, in ? static_cast<uint32_t>(row) * static_cast<uint32_t>(K) + static_cast<uint32_t>(col) : kOOB, 0, kStreamOnce);
    if constexpr (GROUPS) {
      const int g = col >> 7;
      sbv[ch] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          sbr, in ? static_cast<uint32_t>((row / kSlab) * SR + (E8M0 ? (g & ~3) : g * 4)) : kOOB, 0, 0));
    }
  };
  // every load is issued unconditionally (a chunk past K reads zeros without touching memory),
  // so the compiler counts the loads in flight exactly: the quantize waits for x alone, and
  // each chunk's math only for its own chunk
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) fetch(row0, ch);

  // the quantize; lanes past K hold zeros, whose key 0 leaves every amax unchanged
  float tscale = 1.0f;                                        // one scale per tensor or per row
  uint2 ca[CPW], cb[CPW];
  if constexpr (GROUPS) {
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      // eight lanes hold one 1x128 group (K % 128 == 0: a group is all in or all out)
      const int ch = w + j * WAVES;
      const GroupScale<E8M0> gs(amax_from_key<DT>(max8(max(key8(v0[j]), key8(v1[j])))));
      const bool fast = fast_scale(gs.scale);
      const float r = 1.0f / gs.scale;
      ca[j] = enc8<DT>(v0[j], gs.scale, r, fast);
      cb[j] = enc8<DT>(v1[j], gs.scale, r, fast);
      const int xcol = ch * 1024 + lane * 16;
      if (ch < NCH && (lane & 7) == 0) {
        gsc[ch * 8 + (lane >> 3)] = E8M0 ? __uint_as_float(gs.code) : gs.scale;
        if (blockIdx.x == 0 && xcol < K) gs.store(sa_, 0, xcol >> 7, KG, SR);
      }
    }
  } else {
    uint32_t key = 0;
#pragma unroll
    for (int j = 0; j < CPW; ++j) key = max(key, max(key8(v0[j]), key8(v1[j])));
    const uint32_t wk = max64(key);
    if (lane == 0) wkey[w] = wk;
    __syncthreads();
    uint32_t k = 0;
#pragma unroll
    for (int i = 0; i < WAVES; ++i) k = max(k, wkey[i]);
    tscale = scale_from_amax(amax_from_key<DT>(k));
    const bool fast = fast_scale(tscale);
    const float r = 1.0f / tscale;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      ca[j] = enc8<DT>(v0[j], tscale, r, fast);
      cb[j] = enc8<DT>(v1[j], tscale, r, fast);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) static_cast<float*>(sa_)[0] = tscale;
  }
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int ch = w + j * WAVES;
    if (ch < NCH) {
      const uint32_t cw[4] = {ca[j].x, ca[j].y, cb[j].x, cb[j].y};
      h2 f[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        f[2 * d] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(cw[d]), 1.0f, false);
        f[2 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(cw[d]), 1.0f, true);
      }
      alo[ch][lane] = v4i{__builtin_bit_cast(int, f[0]), __builtin_bit_cast(int, f[1]), __builtin_bit_cast(int, f[2]),
                          __builtin_bit_cast(int, f[3])};
      ahi[ch][lane] = v4i{__builtin_bit_cast(int, f[4]), __builtin_bit_cast(int, f[5]), __builtin_bit_cast(int, f[6]),
                          __builtin_bit_cast(int, f[7])};
      const int xcol = ch * 1024 + lane * 16;
      if (blockIdx.x == 0 && xcol < K)
        *reinterpret_cast<uint4*>(qa + xcol) = make_uint4(ca[j].x, ca[j].y, cb[j].x, cb[j].y);
    }
  }
  __syncthreads();

  // weight rows: gemv_valu_kernel's arithmetic with one token and one row per wave at a time
  const float* __restrict__ sb = static_cast<const float*>(sb_);
  const int step = STREAM ? waves : N;                        // one pass without STREAM
  for (int row = row0; row < N; row += step) {
    float acc = 0.0f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      // a chunk past K holds zero codes and a zero weight row, so it adds zero: 0 * 1 * 0 with
      // block scales, ldexp(0) with UE8M0 codes 127 and 0 (skipping it with a branch was 4%
      // slower at W[18432, 7168])
      const v4i lo = alo[ch][lane], hi = ahi[ch][lane];
      const int aw[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      float d = GROUPS ? 0.0f : acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const h2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wv[ch][q], 1.0f, false);
        const h2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wv[ch][q], 1.0f, true);
        d = __builtin_amdgcn_fdot2(w0, __builtin_bit_cast(h2, aw[2 * q]), d, false);
        d = __builtin_amdgcn_fdot2(w1, __builtin_bit_cast(h2, aw[2 * q + 1]), d, false);
      }
      if constexpr (E8M0) {
        // d * 2^(ea - 127) * 2^(eb - 127) in one exact step; a NaN code gives NaN
        const int ea = static_cast<int>(__float_as_uint(gsc[ch * 8 + (lane >> 3)]));
        const int eb = e8m0_byte(__float_as_uint(sbv[ch]), (ch * 1024 + lane * 16) >> 7);
        acc += (ea == 0xff || eb == 0xff) ? __uint_as_float(kCanonicalNaN) : __builtin_amdgcn_ldexpf(d, ea + eb - 254);
      } else if constexpr (GROUPS) {
        acc = __builtin_fmaf(d, gsc[ch * 8 + (lane >> 3)] * sbv[ch], acc);
      } else {
        acc = d;
      }
      if constexpr (STREAM) {
        fetch(row + waves, ch);                               // the same chunk of the next row
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    acc = wave_sum(acc);
    float wfac = 1.0f;                                        // the weight side of the epilogue factor
    if constexpr (SM == SM_TENSOR) wfac = sb[0];
    else if constexpr (SM == SM_ROW) wfac = sb[row];
    if (lane == 0) c[row] = static_cast<uint16_t>(f32_to_out_bits<OUT>(acc * (tscale * wfac)));
  }
}

template <int BW, int OUT, int NCH>
void launch_stream1_t(const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa, const uint8_t* qb,
                      const void* sb, int N, int K, void* c, hipStream_t s) {
  const int waves = min(N, 256 * plan::kStreamPerCu);
  gemv1_stream_kernel<BW, OUT, NCH><<<static_cast<unsigned>(L.grid), 256, 0, s>>>(qa, sa, qb, sb, N, K,
                                                                                 static_cast<uint16_t*>(c), waves);
}

template <int BW, int OUT, int MT, int RPW, int UNROLL>
void launch_valu_t(const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa, const uint8_t* qb,
                   const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  gemv_valu_kernel<BW, OUT, MT, RPW, UNROLL><<<static_cast<unsigned>(L.grid), 256, 0, s>>>(
      qa, sa, qb, sb, M, N, K, static_cast<uint16_t*>(c));
}

template <int BW, int OUT, int WAVES, int UNROLL, int NB, int MB = 1>
void launch_t(const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb,
              int M, int N, int K, void* c, hipStream_t s) {
  gemv_fp8_kernel<BW, OUT, WAVES, UNROLL, NB, MB><<<static_cast<unsigned>(L.grid), WAVES * 64, 0, s>>>(
      qa, sa, qb, sb, M, N, K, static_cast<uint16_t*>(c));
}

// Carries out a decode launch of a plan (plan_gemm in gemm_plan.hpp picks the kernel and
// says why).  The persistent one-token kernel exists for float32 block scales only.
template <int BW, int OUT>
bool launch_m(const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb,
              int M, int N, int K, void* c, hipStream_t s) {
  switch (L.kernel) {
    case FP8_KERNEL_GEMV_STREAM:
      if constexpr (BW == SM_BLOCK) {
        switch (L.variant) {
          case 1: launch_stream1_t<BW, OUT, 1>(L, qa, sa, qb, sb, N, K, c, s); return true;
          case 2: launch_stream1_t<BW, OUT, 2>(L, qa, sa, qb, sb, N, K, c, s); return true;
          case 3: launch_stream1_t<BW, OUT, 3>(L, qa, sa, qb, sb, N, K, c, s); return true;
          case 4: launch_stream1_t<BW, OUT, 4>(L, qa, sa, qb, sb, N, K, c, s); return true;
          case 5: launch_stream1_t<BW, OUT, 5>(L, qa, sa, qb, sb, N, K, c, s); return true;
          case 6: launch_stream1_t<BW, OUT, 6>(L, qa, sa, qb, sb, N, K, c, s); return true;
          case 7: launch_stream1_t<BW, OUT, 7>(L, qa, sa, qb, sb, N, K, c, s); return true;
          case 8: launch_stream1_t<BW, OUT, 8>(L, qa, sa, qb, sb, N, K, c, s); return true;
          default: return false;
        }
      }
      return false;
    case FP8_KERNEL_GEMV_VALU:
      launch_valu_t<BW, OUT, 1, 1, 4>(L, qa, sa, qb, sb, M, N, K, c, s);
      return true;
    case FP8_KERNEL_GEMV_MFMA:
      if (L.variant == 1) launch_t<BW, OUT, 2, 4, 1>(L, qa, sa, qb, sb, M, N, K, c, s);
      else launch_t<BW, OUT, 4, 2, 2>(L, qa, sa, qb, sb, M, N, K, c, s);
      return true;
    default:
      return false;
  }
}

template <int SM>
bool launch_gemv_m(int out_dt, const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa, const uint8_t* qb,
                   const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  if (out_dt == DT_BF16) return launch_m<SM, DT_BF16>(L, qa, sa, qb, sb, M, N, K, c, s);
  return launch_m<SM, DT_F16>(L, qa, sa, qb, sb, M, N, K, c, s);
}


// Per tensor and per row the persistent form is faster (W[11008, 4096]: 9.3 against 10.1 us;
// W[5632, 2048]: 5.0 against 5.1 us); with float32 or UE8M0 block scales one row per wave is
// (W[18432, 7168]: 23.9 against 24.3 us; W[4096, 7168]: 7.5 against 8.7 us).  Sustained HIP-graph
// runs with cold operands on MI355X.
template <int SM, int DT, int OUT, int NCH>
void launch_dynamic_nch(const uint16_t* x, const uint8_t* qb, const void* sb, uint8_t* qa, void* sa, int N, int K,
                        uint16_t* c, hipStream_t s) {
  if constexpr (plan::dynamic_stream(SM)) {
    const int64_t grid = std::min<int64_t>((N + plan::kDynStreamWaves - 1) / plan::kDynStreamWaves,
                                           int64_t{plan::kCus} * plan::kDynStreamPerCu);
    gemv1_dynamic_kernel<SM, DT, OUT, NCH, plan::kDynStreamWaves, true>
        <<<static_cast<unsigned>(grid), plan::kDynStreamWaves * 64, 0, s>>>(
            x, qb, sb, qa, sa, N, K, c, static_cast<int>(grid) * plan::kDynStreamWaves);
  } else {
    const unsigned grid = static_cast<unsigned>((N + plan::kDynWaves - 1) / plan::kDynWaves);
    gemv1_dynamic_kernel<SM, DT, OUT, NCH, plan::kDynWaves, false><<<grid, plan::kDynWaves * 64, 0, s>>>(
        x, qb, sb, qa, sa, N, K, c, 0);
  }
}

template <int SM, int DT, int OUT>
void launch_dynamic_t(const void* x, const uint8_t* qb, const void* sb, uint8_t* qa, void* sa, int N, int K,
                      void* c, hipStream_t s) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint16_t* cp = static_cast<uint16_t*>(c);
  const int nch = (K + 1023) / 1024;                          // 1 KB activation chunks
  if (nch <= 2) launch_dynamic_nch<SM, DT, OUT, 2>(xp, qb, sb, qa, sa, N, K, cp, s);
  else if (nch <= 4) launch_dynamic_nch<SM, DT, OUT, 4>(xp, qb, sb, qa, sa, N, K, cp, s);
  else launch_dynamic_nch<SM, DT, OUT, 8>(xp, qb, sb, qa, sa, N, K, cp, s);
}

template <int SM>
void launch_dynamic_m(int in_dt, int out_dt, const void* x, const uint8_t* qb, const void* sb, uint8_t* qa, void* sa,
                      int N, int K, void* c, hipStream_t s) {
  if (in_dt == DT_BF16) {
    if (out_dt == DT_BF16) launch_dynamic_t<SM, DT_BF16, DT_BF16>(x, qb, sb, qa, sa, N, K, c, s);
    else launch_dynamic_t<SM, DT_BF16, DT_F16>(x, qb, sb, qa, sa, N, K, c, s);
  } else {
    if (out_dt == DT_BF16) launch_dynamic_t<SM, DT_F16, DT_BF16>(x, qb, sb, qa, sa, N, K, c, s);
    else launch_dynamic_t<SM, DT_F16, DT_F16>(x, qb, sb, qa, sa, N, K, c, s);
  }
}

}  // namespace

bool launch_gemv(int mode, int out_dt, const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa,
                 const uint8_t* qb, const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  if (mode == SM_ROW) return launch_gemv_m<SM_ROW>(out_dt, L, qa, sa, qb, sb, M, N, K, c, s);
  if (mode == SM_E8M0) return launch_gemv_m<SM_E8M0>(out_dt, L, qa, sa, qb, sb, M, N, K, c, s);
  if (mode == SM_BLOCK) return launch_gemv_m<SM_BLOCK>(out_dt, L, qa, sa, qb, sb, M, N, K, c, s);
  return launch_gemv_m<SM_TENSOR>(out_dt, L, qa, sa, qb, sb, M, N, K, c, s);
}

void launch_gemv_dynamic(int mode, int in_dt, int out_dt, const void* x, const uint8_t* qb, const void* sb,
                         uint8_t* qa, void* sa, int N, int K, void* c, hipStream_t s) {
  if (mode == SM_ROW) launch_dynamic_m<SM_ROW>(in_dt, out_dt, x, qb, sb, qa, sa, N, K, c, s);
  else if (mode == SM_E8M0) launch_dynamic_m<SM_E8M0>(in_dt, out_dt, x, qb, sb, qa, sa, N, K, c, s);
  else if (mode == SM_BLOCK) launch_dynamic_m<SM_BLOCK>(in_dt, out_dt, x, qb, sb, qa, sa, N, K, c, s);
  else launch_dynamic_m<SM_TENSOR>(in_dt, out_dt, x, qb, sb, qa, sa, N, K, c, s);
}

}  // namespace fp8amax
