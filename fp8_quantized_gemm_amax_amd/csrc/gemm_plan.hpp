// gemm_plan.hpp - the scaled GEMM's dispatcher as plain host arithmetic: which kernel runs
// for a shape, on which grid and tile, over which columns of C, and how far the 32-bit
// buffer ranges and offsets of each launch reach.  The launchers in gemm.hip and gemv.hip
// carry out a plan as it stands; fp8_debug_gemm_plan hands the same plan to tests.
#pragma once

#include <stdint.h>

#include <algorithm>

#include "fp8amax.h"
#include "launch.hpp"

namespace fp8amax {
namespace plan {

static_assert(int{FP8_SCALE_TENSOR} == int{SM_TENSOR} && int{FP8_SCALE_BLOCK} == int{SM_BLOCK} &&
                  int{FP8_SCALE_BLOCK_UE8M0} == int{SM_E8M0} && int{FP8_SCALE_ROW} == int{SM_ROW},
              "the C ABI's scale modes are the kernels' template values");

constexpr int kCus = 256;              // compute units of one MI355X
constexpr int kSkinnyMaxCw = 7;        // compute waves of the few-token kernel, at most
constexpr int kStreamPerCu = 24;       // waves per CU of the persistent one-token kernel
constexpr int64_t kSlabK = 128;        // K positions per scale slab and per MFMA
constexpr int64_t kLimit32 = (int64_t{1} << 31) - 1;   // the kernels form these in int

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Bytes of one row of blockwise activation (or weight-block) scales: K/128 float32, or
// K/128 UE8M0 bytes padded to whole words; 0 for the modes without slab scales.
inline int64_t scale_row_bytes(int sm, int64_t K) {
  if (sm == SM_E8M0) return e8m0_row_bytes(K / kSlabK);
  return slab_scaled(sm) ? 4 * (K / kSlabK) : 0;
}

// Whether the decode kernels take M tokens: 1..16 tokens, and 32 rows of K bytes (a weight
// row block of the two-block MFMA variant) within 32-bit offsets.
inline bool gemv_fits(int64_t M, int64_t K) { return M >= 1 && M <= 16 && K * 32 <= kLimit32; }

// Whether the fused one-token step (the activation row quantized and multiplied in one
// launch) takes the shape: an eight-wave workgroup holds the row as one 1 KB chunk per wave,
// so K <= 8192, and the weight rows are addressed with 32-bit buffer offsets, so N K < 2^31.
constexpr int kDynWaves = 8;
inline bool dynamic_fits(int64_t N, int64_t K) {
  return N >= 1 && K >= 1 && K <= 1024 * kDynWaves && N * K <= kLimit32;
}
// Its persistent form (per tensor and per row): workgroups of four waves, three per CU, each
// wave taking every (grid waves)-th weight row; the block-scaled modes take one row per wave.
constexpr int kDynStreamWaves = 4;
constexpr int kDynStreamPerCu = 3;
constexpr bool dynamic_stream(int sm) { return sm == SM_TENSOR || sm == SM_ROW; }

// Whether the LDS-DMA kernels take K: whole slabs, and 256 rows of K bytes (the largest
// tile) within 32-bit offsets.  Other K go to the register-staged kernel.
inline bool dma_fits(int64_t K) { return K % kSlabK == 0 && K * 256 <= kLimit32; }

inline fp8_gemm_launch_t make_launch(int kernel, int64_t tile_m, int64_t tile_n, int variant, int waves,
                                     int64_t grid, int64_t threads, int64_t n_begin, int64_t n_end) {
  fp8_gemm_launch_t l{};
  l.kernel = kernel;
  l.tile_m = static_cast<int32_t>(tile_m);
  l.tile_n = static_cast<int32_t>(tile_n);
  l.variant = variant;
  l.waves = waves;
  l.paired = 0;
  l.grid = grid;
  l.threads = threads;
  l.n_begin = n_begin;
  l.n_end = n_end;
  return l;
}

// One launch of the tiled LDS-DMA kernel over columns [n0, n1): BM x BN tiles, waves of
// WM x WN, NS stages.  Per workgroup it builds descriptors over its min(BM, M) A rows,
// min(BN, n) B rows and, with slab scales, each wave's min(WM, M) rows of activation
// scales; lanes address rows of the whole tile (rows past the end read zeros).
inline fp8_gemm_launch_t tile_launch(int sm, int64_t M, int64_t n0, int64_t n1, int64_t K, int BM, int BN,
                                     int WM, int WN, int NS, bool paired) {
  const int waves = (BM / WM) * (BN / WN);
  const int64_t n = n1 - n0;
  fp8_gemm_launch_t l = make_launch(FP8_KERNEL_TILE, BM, BN, NS, waves, cdiv(M, BM) * cdiv(n, BN),
                                    64 * waves, n0, n1);
  l.paired = paired ? 1 : 0;
  const int64_t SR = scale_row_bytes(sm, K);
  l.max_range = std::max({std::min<int64_t>(BM, M) * K, std::min<int64_t>(BN, n) * K, std::min<int64_t>(WM, M) * SR});
  l.max_offset = std::max({int64_t{BM} * K, int64_t{BN} * K, int64_t{WM} * SR});
  return l;
}

// The plan of C[M, N] = A[M, K] B[N, K]^T in scale mode sm (shape already validated).
inline fp8_gemm_plan_t plan_gemm(int sm, int64_t M, int64_t N, int64_t K) {
  fp8_gemm_plan_t p{};
  if (M <= 0 || N <= 0) return p;
  const int64_t SR = scale_row_bytes(sm, K);
  p.launches = 1;
  fp8_gemm_launch_t& l = p.launch[0];

  if (gemv_fits(M, K)) {
    // Measured on MI355X with cold weights: one token runs best on the vector-ALU kernels
    // (1 KB row streams; one row per wave with four 1 KB loads in flight beat two or more
    // rows per wave by 5% at W[11008, 4096] and tied at W[18432, 7168]).  With float32
    // block scales the persistent kernel with the activation row in registers is 10-12%
    // faster on both shapes (24 waves per CU led 16 and 32); per tensor and with UE8M0
    // scales the one-wave-per-row kernel stays ahead.  From two tokens on the MFMA kernel,
    // with two row blocks per wave once the activation fragment is worth sharing (M > 4).
    if (sm == SM_BLOCK && M == 1 && K <= 8192 && N * K <= kLimit32) {
      const int64_t waves = std::min<int64_t>(N, int64_t{kCus} * kStreamPerCu);
      l = make_launch(FP8_KERNEL_GEMV_STREAM, 1, 1, static_cast<int>(cdiv(K, 1024)), 4, cdiv(waves, 4), 256, 0, N);
      l.max_range = std::max({N * K, cdiv(N, kSlabK) * SR});
      l.max_offset = l.max_range;
    } else if (M == 1) {
      l = make_launch(FP8_KERNEL_GEMV_VALU, 1, 1, 4, 4, cdiv(N, 4), 256, 0, N);
      l.max_range = std::max(K, SR);
      l.max_offset = l.max_range;
    } else {
      const int NB = M <= 4 ? 1 : 2;                // 16-row weight blocks per wave
      const int waves = M <= 4 ? 2 : 4;             // waves splitting the K slabs
      l = make_launch(FP8_KERNEL_GEMV_MFMA, M, 16 * NB, NB, waves, cdiv(N, 16 * NB), 64 * waves, 0, N);
      l.max_range = std::max({std::min<int64_t>(16 * NB, N) * K, M * K, M * SR, 2 * SR});
      l.max_offset = std::max<int64_t>(16 * NB, 16) * K + kSlabK;   // incl. the slab past a K tail
    }
    return p;
  }

  // K tail: the register-staged kernel zero-fills it.  It also takes K so large that 256
  // rows of K bytes overflow the 32-bit buffer offsets of the DMA kernels.  It addresses
  // its operands with 64-bit pointers and forms no buffer descriptors.
  if (!dma_fits(K)) {
    const int BM = M <= 16 ? 16 : 128, BN = M <= 16 ? 256 : 128;
    l = make_launch(FP8_KERNEL_STAGED, BM, BN, 2, 4, cdiv(M, BM) * cdiv(N, BN), 256, 0, N);
    return p;
  }

  // Tile choice, measured on MI355X with cold operands:
  //  - up to 128 rows (weights streamed once): the few-token kernel, with as few compute
  //    waves (16 weight rows each) as keep the workgroups within one round on 256 CUs,
  //    since every workgroup also reads all of A;
  //  - at least one 256x256 tile per CU: 256x256, eight waves of 64x128, two stages;
  //  - more than one 128x128 tile per CU: 128x128 tiles of four 64x64 waves with two
  //    stages, so that two workgroups share a CU;
  //  - otherwise (one partial round): without per-slab scales, 128x96 tiles of four 64x48
  //    waves and three stages while they still fit one round (7-9% faster than 128x128 at
  //    512 x 5632 x 2048, 256 x 5632 x 2048 and 384 x 4096 x 4096: 30% fewer LDS bytes per
  //    slab, more CUs busy); else 128x128 tiles of eight 64x32 waves, three stages.  A
  //    48-column wave can straddle two 128-column weight blocks, so block-scaled modes keep
  //    the 128x128 tile.
  if (M <= 128) {
    const int MB = M <= 32 ? 2 : M <= 64 ? 4 : 8;   // 16-token blocks staged per slab
    const int cw = static_cast<int>(std::min<int64_t>(kSkinnyMaxCw, std::max<int64_t>(2, cdiv(N, 16 * 256))));
    const int64_t rows = 16 * int64_t{cw};          // weight rows per workgroup (one block per wave)
    l = make_launch(FP8_KERNEL_SKINNY, M, rows, MB, cw, cdiv(N, rows), 64 * (cw + 1), 0, N);
    const int64_t scale_dma = slab_scaled(sm) ? cdiv(16 * MB, 64) * 64 * SR : 0;   // 64 rows per scale DMA
    l.max_range = std::max({M * K, M * SR, std::min<int64_t>(16, N) * K, SR});
    l.max_offset = std::max({16 * int64_t{MB} * K, 16 * K, scale_dma, cdiv(M * SR, 256) * 256});
    return p;
  }
  const int64_t big_tiles = cdiv(M, 256) * cdiv(N, 256);
  const int64_t tiles = cdiv(M, 128) * cdiv(N, 128);
  if (big_tiles >= kCus) {
    // whole rounds of 256x256 tiles (one per CU), and when the tile columns left over make
    // at most half a round, those columns as smaller tiles in a second launch, so that the
    // last round is not half empty.  Columns split on whole tiles, so the second launch's
    // weight rows, block scales and C columns are plain offsets.  Paired DMA issue (one
    // wave of each SIMD pair issues the slab's DMA for both) measured faster where no
    // per-slab FMAs compete with the MFMAs, slower with float32 slab scales.
    const int64_t tiles_m = cdiv(M, 256), tiles_n = cdiv(N, 256);
    int64_t cols_main = tiles_n;
    if (big_tiles % kCus != 0) {
      const int64_t cand = (big_tiles / kCus) * kCus / tiles_m;   // whole columns in whole rounds
      if (cand > 0 && tiles_m * (tiles_n - cand) * 2 <= kCus) cols_main = cand;
    }
    const int64_t n_main = std::min(N, cols_main * 256);
    l = tile_launch(sm, M, 0, n_main, K, 256, 256, 64, 128, 2, sm != SM_BLOCK);
    if (n_main < N) {
      // At most half a round of 256x128 tiles leaves half the CUs idle: such a tail runs as
      // 128x128 tiles (eight 64x32 waves, three stages), at most one round of them; measured
      // 6-16% faster over the whole GEMM (DeepSeek-V3 up-projection at 1024 and 2048
      // tokens, 4096 x 4352 x 7168; float32 block, UE8M0 and per-tensor scales).  A larger
      // tail keeps 256x128 tiles, with a third stage where they fill a whole round and K
      // spans 48 slabs or more: measured 8-19% faster there alone (DeepSeek-V3
      // up-projection, 4096 tokens, every scale mode), 2-4% slower over 32 slabs or with
      // half a round.
      const int64_t tail_tiles = tiles_m * cdiv(N - n_main, 128);
      p.launches = 2;
      if (2 * tail_tiles <= kCus) {
        p.launch[1] = tile_launch(sm, M, n_main, N, K, 128, 128, 64, 32, 3, false);
      } else {
        const int ns = (tail_tiles >= kCus && K / kSlabK >= 48) ? 3 : 2;
        p.launch[1] = tile_launch(sm, M, n_main, N, K, 256, 128, 64, 64, ns, false);
      }
    }
  } else if (tiles > kCus) {
    // 128x128 tiles, two workgroups per CU.  Without float32 slab scales, a leftover of 64
    // to 256 tiles after whole rounds runs as a second launch of eight-wave three-stage
    // tiles (one per CU): measured 10-13% faster over the whole GEMM per tensor, per row
    // and with UE8M0 scales (DeepSeek-V3 up-projection at 512 tokens, 1024 x 11008 x 4096;
    // UE8M0 level at 512 tokens), 2-3% slower with float32 block scales, level with a
    // leftover of 32 tiles.
    const int64_t tiles_m = cdiv(M, 128), tiles_n = cdiv(N, 128), slots = 2 * int64_t{kCus};
    int64_t cols_main = tiles_n;
    if (sm != SM_BLOCK && tiles % slots != 0) {
      const int64_t cand = (tiles / slots) * slots / tiles_m;   // whole columns in whole rounds
      const int64_t left = tiles_m * (tiles_n - cand);
      if (cand > 0 && left >= 64 && left <= kCus) cols_main = cand;
    }
    const int64_t n_main = std::min(N, cols_main * 128);
    l = tile_launch(sm, M, 0, n_main, K, 128, 128, 64, 64, 2, false);
    if (n_main < N) {
      p.launches = 2;
      p.launch[1] = tile_launch(sm, M, n_main, N, K, 128, 128, 64, 32, 3, false);
    }
  } else if (!slab_scaled(sm) && cdiv(M, 128) * cdiv(N, 96) <= kCus) {
    l = tile_launch(sm, M, 0, N, K, 128, 96, 64, 48, 3, false);
  } else {
    l = tile_launch(sm, M, 0, N, K, 128, 128, 64, 32, 3, false);
  }
  return p;
}

// Whether every launch of a plan stays within what its kernel indexes with 32-bit int.
inline bool plan_fits(const fp8_gemm_plan_t& p) {
  for (int i = 0; i < p.launches; ++i) {
    const fp8_gemm_launch_t& l = p.launch[i];
    if (l.grid < 1 || l.grid > kLimit32 || l.max_range > kLimit32 || l.max_offset > kLimit32) return false;
  }
  return true;
}

}  // namespace plan
}  // namespace fp8amax
