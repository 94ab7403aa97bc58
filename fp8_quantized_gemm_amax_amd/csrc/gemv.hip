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
#include "launch.hpp"

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
  // 32 bytes of quarter kq of a slab in row r16 of a block.  The dispatcher keeps
  // 16 NB K and M K below 2^31, so every offset fits the 32-bit buffer offset.
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
// lane's 16-term partial.  At the end the 64 lanes' partials of each (m, row) are summed by
// a butterfly.  The float32 sum is ordered differently from the MFMA path; both are within
// the product tolerance of the exact sum.
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

  // RPW K and M K stay below 2^31 (the dispatcher checks 32 K), so offsets fit 32 bits
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
      wv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wr, (in & (r < rows)) ? static_cast<uint32_t>(r * K + col) : kOOB, 0, 0);
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

  // butterfly sum over the 64 lanes; every lane ends with every total
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc[m][r] += __shfl_xor(acc[m][r], o, 64);

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

template <int BW, int OUT, int MT, int RPW, int UNROLL>
void launch_valu_t(const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb, int M, int N,
                   int K, void* c, hipStream_t s) {
  const int waves = (N + RPW - 1) / RPW;
  gemv_valu_kernel<BW, OUT, MT, RPW, UNROLL><<<(waves + 3) / 4, 256, 0, s>>>(
      qa, sa, qb, sb, M, N, K, static_cast<uint16_t*>(c));
}

template <int BW, int OUT, int WAVES, int UNROLL, int NB, int MB = 1>
void launch_t(const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb, int M, int N,
              int K, void* c, hipStream_t s) {
  gemv_fp8_kernel<BW, OUT, WAVES, UNROLL, NB, MB><<<(N + 16 * NB - 1) / (16 * NB), WAVES * 64, 0, s>>>(
      qa, sa, qb, sb, M, N, K, static_cast<uint16_t*>(c));
}

// Measured on MI355X with cold weights: one token runs best on the vector-ALU kernel
// (1 KB row streams; one row per wave with four 1 KB loads in flight beat two or more rows
// per wave by 5% at W[11008, 4096] and tied at W[18432, 7168]); from two tokens on the MFMA
// kernel, with two row blocks per wave once the activation fragment is worth sharing (M > 4).
template <int BW, int OUT>
void launch_m(const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb, int M, int N,
              int K, void* c, hipStream_t s) {
  if (M == 1) launch_valu_t<BW, OUT, 1, 1, 4>(qa, sa, qb, sb, M, N, K, c, s);
  else if (M <= 4) launch_t<BW, OUT, 2, 4, 1>(qa, sa, qb, sb, M, N, K, c, s);
  else launch_t<BW, OUT, 4, 2, 2>(qa, sa, qb, sb, M, N, K, c, s);
}

template <int SM>
void launch_gemv_m(int out_dt, const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb, int M,
                   int N, int K, void* c, hipStream_t s) {
  if (out_dt == DT_BF16) launch_m<SM, DT_BF16>(qa, sa, qb, sb, M, N, K, c, s);
  else launch_m<SM, DT_F16>(qa, sa, qb, sb, M, N, K, c, s);
}

}  // namespace

bool gemv_fits(int M, int K) {
  return M >= 1 && M <= 16 && static_cast<int64_t>(K) * 32 < (int64_t{1} << 31);
}

void launch_gemv(int mode, int out_dt, const uint8_t* qa, const void* sa, const uint8_t* qb,
                 const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  if (mode == SM_ROW) launch_gemv_m<SM_ROW>(out_dt, qa, sa, qb, sb, M, N, K, c, s);
  else if (mode == SM_E8M0) launch_gemv_m<SM_E8M0>(out_dt, qa, sa, qb, sb, M, N, K, c, s);
  else if (mode == SM_BLOCK) launch_gemv_m<SM_BLOCK>(out_dt, qa, sa, qb, sb, M, N, K, c, s);
  else launch_gemv_m<SM_TENSOR>(out_dt, qa, sa, qb, sb, M, N, K, c, s);
}

}  // namespace fp8amax
