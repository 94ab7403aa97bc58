// gemm.hip - FP8 x FP8 GEMM with float32 accumulation and a scale epilogue, for gfx950.
//
// C[m, n] = out( sum_k qa[m, k] * qb[n, k] * scale ), A = qa [M, K], B = qb [N, K], both
// K-contiguous (C = A @ B^T).
//   tensorwise: scale = sa * sb, applied once to the float32 accumulator (Transformer
//     Engine page "Что такое FP8 инференс на H100 (Transformer Engine)?", section 3 steps
//     5-6 and the pseudocode);
//   blockwise: each 128-wide K slab g has its own sa[m, g] * sb[n / 128, g] ("FP8 chi
//     tiết", opening bullets), applied in registers to that slab's float32 partial sum;
//   rowwise: scale = sa[m] * sb[n], one scale per token and per output channel (the
//     Transformer Engine page §5, per-channel scaling), applied once like tensorwise.
//
// Kernels (CDNA4).  Every kernel walks K in 128-byte slabs and multiplies with
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit E8M0 scales, i.e. a plain FP8 product, or the
// UE8M0 block scales themselves); one instruction covers exactly one slab, so the float32
// blockwise epilogue is one FMA per accumulator per slab.
//   gemm_dma_kernel: the tiled product for 129+ tokens.  A and B slabs move global -> LDS
//     by LDS DMA into an NS-stage ring, eight (or four) waves multiply fragments read from
//     LDS.  256x256 tiles when there is at least one per CU, launched as whole rounds plus
//     a second launch of 256x128 tiles for a leftover half round; 128x128 (or, without
//     per-slab scales, 128x96) tiles otherwise.
//   gemm_skinny_kernel / gemm_grouped_kernel: 17-128 tokens (and the mixture-of-experts
//     chunks), weight rows streamed into registers, the tokens staged in LDS by one wave.
//   gemm_fp8_kernel: K not a multiple of 128 (or too large for 32-bit buffer offsets),
//     slabs staged global -> VGPR -> LDS with a zero-filled K tail.
// 1-16 tokens go to the decode kernels of gemv.hip.  The LDS slab layout and the tile order
// are in gemm_common.hpp; which kernel, tile and grid a shape gets is plan_gemm in
// gemm_plan.hpp, whose 32-bit range and offset figures bound the buffer arithmetic here.
//
// MFMA operand roles: the first operand is the B (weight) sub-tile, the second the A
// sub-tile, so lane l holds C[m = l % 16][n = 4 * (l / 16) + r] for r = 0..3: four
// consecutive output columns, stored as one 8-byte write.  Each lane supplies the same
// 32-byte K quarter of its row for both operands, so the product is independent of the
// order in which the hardware walks K inside the instruction.
#include <type_traits>

#include "dma.hpp"
#include "fp8_device.hpp"
#include "gemm_common.hpp"
#include "gemm_plan.hpp"
#include "launch.hpp"

namespace fp8amax {

namespace {

using namespace gemm;

constexpr int kThreads = 256;      // the register-staged kernel

template <int BM, int BN, int WM, int WN, int SM, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_fp8_kernel(
    const uint8_t* __restrict__ qa, const void* __restrict__ sa_, const uint8_t* __restrict__ qb,
    const void* __restrict__ sb_, int M, int N, int K, uint16_t* __restrict__ c, int tiles_m) {
  constexpr bool BLOCKWISE = slab_scaled(SM);
  constexpr bool E8M0 = SM == SM_E8M0;
  const float* __restrict__ sa = static_cast<const float*>(sa_);
  const float* __restrict__ sb = static_cast<const float*>(sb_);
  const uint8_t* __restrict__ ea_ = static_cast<const uint8_t*>(sa_);
  const uint8_t* __restrict__ eb_ = static_cast<const uint8_t*>(sb_);
  constexpr int WAVES_N = BN / WN;
  constexpr int WAVES_M = BM / WM;
  static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
  static_assert(!BLOCKWISE || (WN <= 128 && 128 % WN == 0), "a wave's columns share one weight block");
  constexpr int TM = WM / 16;
  constexpr int TN = WN / 16;
  constexpr int A_IT = (BM * 8 + kThreads - 1) / kThreads;   // 16-byte chunks per thread
  constexpr int B_IT = (BN * 8 + kThreads - 1) / kThreads;
  constexpr int STAGE = (BM + BN) * kSlab;

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  const int tile = blockIdx.x;
  const int tm = tile % tiles_m;
  const int tn = tile / tiles_m;
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wm = w / WAVES_N;
  const int wn = w % WAVES_N;
  const int r16 = lane & 15;
  const int kq = lane >> 4;      // 32-byte quarter of the slab this lane feeds to the MFMA
  const int KG = K / kSlab;      // blockwise only (K % 128 == 0 there)
  const int64_t KG4 = e8m0_row_bytes(KG);

  uint4 ra[A_IT], rb[B_IT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < A_IT; ++j) {
      const int id = t + kThreads * j;
      const int row = id >> 3, ch = id & 7;
      const int gm = m0 + row, kk = k0 + ch * 16;
      ra[j] = make_uint4(0u, 0u, 0u, 0u);
      if ((BM * 8 % kThreads == 0 || id < BM * 8) && gm < M && kk < K)
        ra[j] = *reinterpret_cast<const uint4*>(qa + static_cast<int64_t>(gm) * K + kk);
    }
#pragma unroll
    for (int j = 0; j < B_IT; ++j) {
      const int id = t + kThreads * j;
      const int row = id >> 3, ch = id & 7;
      const int gn = n0 + row, kk = k0 + ch * 16;
      rb[j] = make_uint4(0u, 0u, 0u, 0u);
      if ((BN * 8 % kThreads == 0 || id < BN * 8) && gn < N && kk < K)
        rb[j] = *reinterpret_cast<const uint4*>(qb + static_cast<int64_t>(gn) * K + kk);
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* As = lds + stage * STAGE;
    uint8_t* Bs = As + BM * kSlab;
#pragma unroll
    for (int j = 0; j < A_IT; ++j) {
      const int id = t + kThreads * j;
      if (BM * 8 % kThreads == 0 || id < BM * 8) {
        const int row = id >> 3, ch = id & 7;
        *reinterpret_cast<uint4*>(As + row * kSlab + ((ch ^ swz(row)) << 4)) = ra[j];
      }
    }
#pragma unroll
    for (int j = 0; j < B_IT; ++j) {
      const int id = t + kThreads * j;
      if (BN * 8 % kThreads == 0 || id < BN * 8) {
        const int row = id >> 3, ch = id & 7;
        *reinterpret_cast<uint4*>(Bs + row * kSlab + ((ch ^ swz(row)) << 4)) = rb[j];
      }
    }
  };
  auto frag = [&](const uint8_t* base, int row) -> v8i {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row * kSlab + (((2 * kq) ^ swz(row)) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + row * kSlab + (((2 * kq + 1) ^ swz(row)) << 4));
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
  };

  // blockwise scales: sa for this lane's row in each M sub-tile, sb for the wave's block
  const int wave_n0 = n0 + wn * WN;
  FragFactors<SM, TM, TN> ff;                        // rowwise epilogue scales, fetched now
  ff.load(sa, sb, m0 + wm * WM, wave_n0, M, N);
  const int nb = wave_n0 / kSlab;
  const int NB = (N + kSlab - 1) / kSlab;
  auto load_scales = [&](int g, float* out, int* ea, int& eb) {
    if constexpr (E8M0) {
      eb = (nb < NB) ? eb_[nb * KG4 + g] : 127;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm * WM + 16 * i + r16;
        ea[i] = (m < M) ? ea_[m * KG4 + g] : 127;             // rows past M multiply zeros
      }
    } else {
      const float sbv = (nb < NB) ? sb[static_cast<int64_t>(nb) * KG + g] : 0.0f;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm * WM + 16 * i + r16;
        out[i] = (m < M) ? sa[static_cast<int64_t>(m) * KG + g] * sbv : 0.0f;
      }
    }
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  float scl[TM], scl_next[TM];
  int ea[TM], ea_next[TM], eb = 127, eb_next = 127;
  if constexpr (BLOCKWISE) load_scales(0, scl, ea, eb);

  const int nslabs = (K + kSlab - 1) / kSlab;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nslabs; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nslabs;
    if (more) gload((s + 1) * kSlab);
    if constexpr (BLOCKWISE) {
      if (more) load_scales(s + 1, scl_next, ea_next, eb_next);
    }
    const uint8_t* As = lds + cur * STAGE;
    const uint8_t* Bs = As + BM * kSlab;
    v8i af[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = frag(As, wm * WM + 16 * i + r16);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const v8i bf = frag(Bs, wn * WN + 16 * j + r16);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (E8M0) {
          acc[i][j] = mfma_fp8_e8m0(bf, af[i], acc[i][j], eb, ea[i]);
        } else if constexpr (BLOCKWISE) {
          const v4f p = mfma_fp8(bf, af[i], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], scl[i], acc[i][j][r]);
        } else {
          acc[i][j] = mfma_fp8(bf, af[i], acc[i][j]);
        }
      }
    }
    if (more) lstore(cur ^ 1);
    if constexpr (BLOCKWISE) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        scl[i] = scl_next[i];
        ea[i] = ea_next[i];
      }
      eb = eb_next;
    }
    __syncthreads();
  }

  float alpha = 1.0f;
  if constexpr (SM == SM_TENSOR) alpha = sa[0] * sb[0];
  const bool vec_store = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WM + 16 * i + r16;
    if (m >= M) continue;
    uint16_t* crow = c + static_cast<int64_t>(m) * N;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wave_n0 + 16 * j + 4 * kq;
      uint32_t h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        h[r] = f32_to_out_bits<OUT>(acc[i][j][r] * ff(alpha, i, j, r));
      if (vec_store && n + 3 < N) {
        *reinterpret_cast<uint2*>(crow + n) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) crow[n + r] = static_cast<uint16_t>(h[r]);
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Large-tile kernel: slabs move global -> LDS by buffer_load ... lds (LDS DMA), so no VGPRs
// stage them and no masked branches guard them: the buffer range check returns zeros for
// rows past M or N; K must be a multiple of 128.
// The DMA is inline asm, so the compiler does not wait for it before the fragment reads;
// the kernel orders them itself (wait_vmcnt for its own DMA of the slab, then a barrier),
// and the next slabs' DMA stays in flight across the current slab's MFMAs.
//
// DMA layout: each wave instruction g writes 64 consecutive 16-byte chunks, rows 8g .. 8g+7;
// lane i of the instruction fetches logical chunk dma_chunk(i, g & 1) = (i % 8) ^
// swz(8g + i / 8) of its row, which puts chunk c of row r at position c ^ swz(r) - the
// swizzle the fragment reads use (gemm_common.hpp).
//
// Tile order: workgroup b runs on XCD b % 8; consecutive tiles of a grouped order
// (groups of kGroupM tile rows) are given to the same XCD so its L2 serves their shared
// A rows and B columns.
// Wait until at most `ahead` slabs of PER vector-memory operations each are still in flight
// (A = the most the pipeline ever leaves outstanding).
template <int PER, int A>
__device__ __forceinline__ void wait_slabs_ahead(int ahead) {
  if constexpr (A > 0) {
    if (ahead >= A) {
      wait_vmcnt<A * PER>();
      return;
    }
    wait_slabs_ahead<PER, A - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
}

template <int BM, int BN, int WM, int WN>
constexpr int dma_threads() { return 64 * (BM / WM) * (BN / WN); }

template <int BM, int BN, int WM, int WN, int SM, int OUT, int NS, bool PAIR = false>
__global__ __launch_bounds__((dma_threads<BM, BN, WM, WN>())) void gemm_dma_kernel(
    const uint8_t* __restrict__ qa, const void* __restrict__ sa_, const uint8_t* __restrict__ qb,
    const void* __restrict__ sb_, int M, int N, int K, uint16_t* __restrict__ c, int tiles_m,
    int tiles_n, int ldc) {
  constexpr bool BLOCKWISE = slab_scaled(SM);
  constexpr bool E8M0 = SM == SM_E8M0;
  const float* __restrict__ sa = static_cast<const float*>(sa_);
  const float* __restrict__ sb = static_cast<const float*>(sb_);
  constexpr int WAVES_N = BN / WN;
  constexpr int WAVES_M = BM / WM;
  constexpr int WAVES = WAVES_M * WAVES_N;
  static_assert(WAVES == 4 || WAVES == 8, "four or eight waves per workgroup");
  static_assert(!BLOCKWISE || (WN <= 128 && 128 % WN == 0), "a wave's columns share one weight block");
  static_assert(!BLOCKWISE || WM % 64 == 0, "one scale DMA instruction per 64 rows");
  constexpr int TM = WM / 16;
  constexpr int TN = WN / 16;
  constexpr int IA = BM * 8 / (WAVES * 64);   // DMA instructions per wave per slab
  constexpr int IB = BN * 8 / (WAVES * 64);
  static_assert(IA * WAVES * 64 == BM * 8 && IB * WAVES * 64 == BN * 8, "whole DMA instructions");
  constexpr int IS = BLOCKWISE ? WM / 64 : 0;
  constexpr int PER_SLAB = IA + IB + IS;          // vector-memory ops per wave per slab
  static_assert(NS >= 2 && NS <= 6, "two to six stages");
  static_assert((NS - 2) * PER_SLAB < 64, "stages in flight fit vmcnt");

  __shared__ __attribute__((aligned(1024))) uint8_t Abuf[NS][BM * kSlab];
  __shared__ __attribute__((aligned(1024))) uint8_t Bbuf[NS][BN * kSlab];
  __shared__ __attribute__((aligned(16))) float Sbuf[NS][BLOCKWISE ? WAVES * WM : 1];

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, uniform (SGPR)
  const int wm = w / WAVES_N, wn = w % WAVES_N;
  const int r16 = lane & 15, kq = lane >> 4;
  const int KG = K / kSlab;
  const int KG4 = static_cast<int>(e8m0_row_bytes(KG));   // UE8M0: bytes per scale row

  const v4i ra = make_rsrc(qa + static_cast<int64_t>(m0) * K, static_cast<uint32_t>(min(BM, M - m0) * K));
  const v4i rb = make_rsrc(qb + static_cast<int64_t>(n0) * K, static_cast<uint32_t>(min(BN, N - n0) * K));
  // logical chunk this lane fetches in even and in odd DMA instructions
  const int lc0 = dma_chunk(lane, 0), lc1 = dma_chunk(lane, 1);
  const uint32_t row_off = static_cast<uint32_t>(((w * IA) * 8 + (lane >> 3)) * K);
  const uint32_t row_off_b = static_cast<uint32_t>(((w * IB) * 8 + (lane >> 3)) * K);
  const uint32_t c_even = static_cast<uint32_t>(lc0 * 16), c_odd = static_cast<uint32_t>(lc1 * 16);
  (void)TN;
  // blockwise: this wave's WM activation scales of a slab, one 32-bit word per lane per
  // instruction (a float32 scale, or for UE8M0 the word holding the slab's scale byte)
  const int srow0 = m0 + wm * WM;
  v4i rs = {0, 0, 0, 0};
  if constexpr (E8M0)
    rs = make_rsrc(static_cast<const uint8_t*>(sa_) + static_cast<int64_t>(srow0) * KG4,
                   static_cast<uint32_t>(max(0, min(WM, M - srow0)) * KG4));
  else if constexpr (BLOCKWISE)
    rs = make_rsrc(sa + static_cast<int64_t>(srow0) * KG,
                   static_cast<uint32_t>(max(0, min(WM, M - srow0)) * KG * 4));

  // PAIR (eight waves): waves w and w + 4 share a SIMD; the first of the pair issues the
  // slab's DMA for both, so the second keeps the SIMD's matrix unit busy while the first
  // waits for room in the memory queue
  static_assert(!PAIR || WAVES == 8, "pairs of waves on one SIMD");
  const bool lead = !PAIR || w < 4;
  const int wp = PAIR ? w + 4 : w;                         // the partner's wave index
  const int srow0p = m0 + (wp / WAVES_N) * WM;
  v4i rsp = {0, 0, 0, 0};
  if constexpr (PAIR && E8M0)
    rsp = make_rsrc(static_cast<const uint8_t*>(sa_) + static_cast<int64_t>(srow0p) * KG4,
                    static_cast<uint32_t>(max(0, min(WM, M - srow0p)) * KG4));
  else if constexpr (PAIR && BLOCKWISE)
    rsp = make_rsrc(sa + static_cast<int64_t>(srow0p) * KG,
                    static_cast<uint32_t>(max(0, min(WM, M - srow0p)) * KG * 4));
  const uint32_t row_off_p = static_cast<uint32_t>(((wp * IA) * 8 + (lane >> 3)) * K);
  const uint32_t row_off_bp = static_cast<uint32_t>(((wp * IB) * 8 + (lane >> 3)) * K);

  // K % 128 == 0 here (plan_gemm sends other K to the staged kernel), so every
  // offset is plain arithmetic and only the row range check can zero a chunk
  auto issue_pair = [&](int s, int st) {
    const uint32_t k0 = static_cast<uint32_t>(s * kSlab);
#pragma unroll
    for (int j = 0; j < IA; ++j)
      dma16(ra, lds_addr(Abuf[st] + (wp * IA + j) * 1024),
            row_off_p + static_cast<uint32_t>(j * 8 * K) + k0 + (((wp * IA + j) & 1) ? c_odd : c_even));
#pragma unroll
    for (int j = 0; j < IB; ++j)
      dma16(rb, lds_addr(Bbuf[st] + (wp * IB + j) * 1024),
            row_off_bp + static_cast<uint32_t>(j * 8 * K) + k0 + (((wp * IB + j) & 1) ? c_odd : c_even));
    if constexpr (BLOCKWISE) {
#pragma unroll
      for (int j = 0; j < IS; ++j)
        dma4(rsp, lds_addr(Sbuf[st] + wp * WM + j * 64),
             E8M0 ? static_cast<uint32_t>((j * 64 + lane) * KG4 + (s & ~3))
                  : static_cast<uint32_t>(((j * 64 + lane) * KG + s) * 4));
    }
  };
  auto issue = [&](int s, int st) {
    if constexpr (PAIR) {
      if (!lead) return;
      issue_pair(s, st);
    }
    const uint32_t k0 = static_cast<uint32_t>(s * kSlab);
    uint8_t* As = Abuf[st];
    uint8_t* Bs = Bbuf[st];
#pragma unroll
    for (int j = 0; j < IA; ++j)
      dma16(ra, lds_addr(As + (w * IA + j) * 1024),
            row_off + static_cast<uint32_t>(j * 8 * K) + k0 + (((w * IA + j) & 1) ? c_odd : c_even));
#pragma unroll
    for (int j = 0; j < IB; ++j)
      dma16(rb, lds_addr(Bs + (w * IB + j) * 1024),
            row_off_b + static_cast<uint32_t>(j * 8 * K) + k0 + (((w * IB + j) & 1) ? c_odd : c_even));
    if constexpr (BLOCKWISE) {
      float* Ss = Sbuf[st];
#pragma unroll
      for (int j = 0; j < IS; ++j)
        dma4(rs, lds_addr(Ss + w * WM + j * 64),
             E8M0 ? static_cast<uint32_t>((j * 64 + lane) * KG4 + (s & ~3))
                  : static_cast<uint32_t>(((j * 64 + lane) * KG + s) * 4));
    }
  };
  const int nslabs = K / kSlab;
  auto frag = [&](const uint8_t* base, int row) -> v8i {
    const int sw = swz(row);
    const v4i lo = *reinterpret_cast<const v4i*>(base + row * kSlab + (((2 * kq) ^ sw) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(base + row * kSlab + (((2 * kq + 1) ^ sw) << 4));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  const int wave_n0 = n0 + wn * WN;
  const int nb = min(wave_n0, N - 1) / kSlab;
  // rowwise epilogue factors, fetched now: loaded after the K loop, their latency was
  // exposed load by load between the bf16 roundings (rowwise bf16 was 25% slower than fp16)
  FragFactors<SM, TM, TN> ff;
  ff.load(sa, sb, m0 + wm * WM, wave_n0, M, N);

  // Weight-block scales of this wave's block row nb: a window of 64 slabs (float32) or of
  // 64 words of four UE8M0 bytes (256 slabs), lane l holding entry l, read per slab with
  // readlane.  A per-slab scalar load would be waited for with lgkmcnt, the counter the
  // slab's LDS fragment reads use, so every fragment wait after it would wait for it too.
  // The window is loaded before the tile's first DMA and waited for there (vmcnt 0, which
  // also tells the compiler's own wait insertion that it has arrived); a K of more than
  // one window reloads it the same way at the window's first slab.
  constexpr int kWin = E8M0 ? 256 : 64;
  auto load_window = [&](int s0) -> uint32_t {
    if constexpr (E8M0) {
      const int word = s0 / 4 + lane;
      return word < KG4 / 4 ? *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(sb_) +
                                                                 static_cast<int64_t>(nb) * KG4 + 4 * word)
                            : 0u;
    } else {
      const int g = s0 + lane;
      return g < KG ? __float_as_uint(sb[static_cast<int64_t>(nb) * KG + g]) : 0u;
    }
  };
  uint32_t sbw = 0;
  if constexpr (BLOCKWISE) sbw = load_window(0);

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (BLOCKWISE) wait_vmcnt<0>();

  auto compute = [&](int s, int st) {
    const uint8_t* As = Abuf[st];
    const uint8_t* Bs = Bbuf[st];
    float scl[TM];
    int ea[TM], eb = 127;
    if constexpr (E8M0) {
      // the weight block's word from the window; each lane's activation word came with
      // the slab's DMA
      eb = e8m0_byte(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(sbw), (s % kWin) / 4)), s);
      const float* Ss = Sbuf[st];
#pragma unroll
      for (int i = 0; i < TM; ++i) ea[i] = e8m0_byte(__float_as_uint(Ss[w * WM + 16 * i + r16]), s);
    } else if constexpr (BLOCKWISE) {
      const float sbv = __int_as_float(__builtin_amdgcn_readlane(static_cast<int>(sbw), s % kWin));
      const float* Ss = Sbuf[st];
#pragma unroll
      for (int i = 0; i < TM; ++i) scl[i] = Ss[w * WM + 16 * i + r16] * sbv;
    }
    v8i af[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = frag(As, wm * WM + 16 * i + r16);
    v8i bfb[2];
    bfb[0] = frag(Bs, wn * WN + r16);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if (j + 1 < TN) bfb[(j + 1) & 1] = frag(Bs, wn * WN + 16 * (j + 1) + r16);
      const v8i bf = bfb[j & 1];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (E8M0) {
          acc[i][j] = mfma_fp8_e8m0(bf, af[i], acc[i][j], eb, ea[i]);
        } else if constexpr (BLOCKWISE) {
          const v4f p = mfma_fp8(bf, af[i], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], scl[i], acc[i][j][r]);
        } else {
          acc[i][j] = mfma_fp8(bf, af[i], acc[i][j]);
        }
      }
    }
    if constexpr (!BLOCKWISE && WN == 128) {
      // Without per-slab scales, on the 64x128 waves of the 256x256 tiles: one MFMA, then at
      // most four VALU instructions, through the slab.  Measured per tensor and per row: 3-4%
      // faster than the compiler's own order in the whole-round launch of the DeepSeek-V3 and
      // Llama-3-8B shapes; with slab scales (float32 FMAs, or UE8M0 scale operands) every fixed
      // order tried was slower or level, and on the 128x96 tiles it gained nothing.
#pragma unroll
      for (int k = 0; k < TM * TN; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
      }
    }
  };

  // Pipeline: slabs s+1 .. s+NS-2 stay in flight while slab s is multiplied.  Step s waits
  // until its own DMA for slab s has landed (everything issued later may still be
  // outstanding), then a barrier makes every wave's part visible and tells every wave
  // that slab s-1's stage is free again; that stage receives slab s+NS-1.
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < nslabs) issue(p, p);
  for (int s = 0; s < nslabs; ++s) {
    if constexpr (BLOCKWISE) {
      if (s > 0 && s % kWin == 0) {                    // the next window of weight-block scales
        sbw = load_window(s);
        wait_vmcnt<0>();
      }
    }
    const int ahead = min(NS - 2, nslabs - 1 - s);    // later slabs allowed to stay in flight
    if constexpr (PAIR) {
      if (lead) wait_slabs_ahead<2 * PER_SLAB, NS - 2>(ahead);
    } else {
      wait_slabs_ahead<PER_SLAB, NS - 2>(ahead);
    }
    stage_barrier();
    if (s + NS - 1 < nslabs) issue(s + NS - 1, (s + NS - 1) % NS);
    compute(s, s % NS);
  }

  float alpha = 1.0f;
  if constexpr (SM == SM_TENSOR) alpha = sa[0] * sb[0];
  const bool vec_store = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WM + 16 * i + r16;
    if (m >= M) continue;
    uint16_t* crow = c + static_cast<int64_t>(m) * ldc;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wave_n0 + 16 * j + 4 * kq;
      uint32_t h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        h[r] = f32_to_out_bits<OUT>(acc[i][j][r] * ff(alpha, i, j, r));
      if (vec_store && n + 3 < N) {
        *reinterpret_cast<uint2*>(crow + n) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) crow[n + r] = static_cast<uint16_t>(h[r]);
      }
    }
  }
}

// Few-token GEMM (16 < M <= 16 MB), bound by streaming W from HBM.  Every workgroup needs
// all of A, so the cost per CU is its share of W plus one pass over A: the tile spans all
// M rows and as few W rows as fill the chip, and no A byte is fetched twice per
// workgroup.  The roles are split between waves so that each keeps its own in-order
// vector-memory queue:
//  - the last wave (the loader) stages each A slab (16 MB rows x 128 B, plus the blockwise
//    activation scales) into an NS-deep LDS ring with LDS DMA, in the swizzled layout of
//    the tiled kernel above;
//  - the cw waves before it each own 16 NB weight rows and stream them from HBM straight into
//    MFMA operand registers (UNROLL slabs in flight, refilled as soon as consumed), and
//    multiply them by the A fragments read from LDS.
// One barrier per slab: the loader passes it once A(s) has landed, and by reaching it the
// compute waves have finished with slab s - 1, whose stage the loader refills next.
// The launch has cw + 1 waves (cw <= kSkinnyMaxCw): the number of compute waves sets how
// many weight rows a workgroup covers, and is chosen so one round of workgroups spans N.
constexpr int kSkinnyMaxCw = plan::kSkinnyMaxCw;

template <int SM, int MB>
struct SkinnyShape {
  static constexpr bool BLOCKWISE = slab_scaled(SM);
  static constexpr int IA = 2 * MB;                          // A DMA instructions per slab (8 rows each)
  static constexpr int IS = BLOCKWISE ? (16 * MB + 63) / 64 : 0;   // scale DMA instructions (64 rows each)
  static constexpr int PER = IA + IS;
  static constexpr int A_BYTES = 16 * MB * kSlab;            // one stage of the A ring
  static constexpr int S_FLOATS = BLOCKWISE ? IS * 64 : 1;   // one stage of the scale ring
  // blockwise: the workgroup's whole activation-scale block (16 MB rows of K/128 float32
  // scales, or of padded UE8M0 byte rows), staged once when it fits here
  static constexpr int PRE_BYTES = BLOCKWISE ? 65536 : 16;
};

// The few-token product of one workgroup: A rows [0, M) (M <= 16 MB) times the 16 cw NB
// weight rows of block `nblk`, written to C rows [0, M).  Abuf and Sbuf are the workgroup's
// LDS rings; every wave of the workgroup calls this once per tile, and each call passes
// exactly K / 128 barriers in every wave.
template <int SM, int OUT, int NB, int MB, int NS, int UNROLL>
__device__ __forceinline__ void skinny_body(
    const uint8_t* __restrict__ qa, const void* __restrict__ sa_, const uint8_t* __restrict__ qb,
    const void* __restrict__ sb_, int M, int N, int K, int cw, uint16_t* __restrict__ c, int nblk,
    uint8_t (*Abuf)[SkinnyShape<SM, MB>::A_BYTES], float (*Sbuf)[SkinnyShape<SM, MB>::S_FLOATS],
    uint8_t* Spre) {
  constexpr bool BLOCKWISE = slab_scaled(SM);
  constexpr bool E8M0 = SM == SM_E8M0;
  const float* __restrict__ sa = static_cast<const float*>(sa_);
  const float* __restrict__ sb = static_cast<const float*>(sb_);
  constexpr int IA = SkinnyShape<SM, MB>::IA;
  constexpr int IS = SkinnyShape<SM, MB>::IS;
  constexpr int PER = SkinnyShape<SM, MB>::PER;
  static_assert(NS >= 2 && (NS - 2) * PER < 64, "slabs in flight fit vmcnt");
  static_assert(kSlab % (16 * NB) == 0, "a wave's rows share one weight block");

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nslabs = K / kSlab;                      // K % 128 == 0 on this path
  const int KG = nslabs;
  const int KG4 = static_cast<int>(e8m0_row_bytes(KG));   // UE8M0: bytes per scale row
  // Activation scales of a slab lie a scale row apart, one cache line per token, so fetching
  // them slab by slab costs as many L2 requests as the A slab itself.  From 64 tokens on,
  // when the block fits, the loader stages it once (measured at 128 tokens, W[18432, 7168]:
  // 53.7 -> 50.0 us); below that it gained nothing (MoE chunks of up to 17 tokens).  UE8M0
  // stages only with one weight fragment per wave: with two (the grouped launch) the
  // staged path made the kernel spill registers.
  const int srow_bytes = E8M0 ? KG4 : 4 * KG;
  constexpr bool kCanStage = SM == SM_BLOCK || (E8M0 && NB == 1);
  const bool pre = kCanStage && M >= 64 && 16 * MB * srow_bytes <= SkinnyShape<SM, MB>::PRE_BYTES;

  if (w == cw) {
    // ---- loader wave ----
    const v4i ra = make_rsrc(qa, static_cast<uint32_t>(M * K));
    v4i rs = {0, 0, 0, 0};
    if constexpr (E8M0) rs = make_rsrc(sa_, static_cast<uint32_t>(M * KG4));
    else if constexpr (BLOCKWISE) rs = make_rsrc(sa, static_cast<uint32_t>(M * KG * 4));
    // instruction j fetches rows 8j .. 8j + 7; lane i takes logical chunk (i % 8) ^ swz(row)
    const int lc0 = dma_chunk(lane, 0), lc1 = dma_chunk(lane, 1);
    const uint32_t c_even = static_cast<uint32_t>(lc0 * 16), c_odd = static_cast<uint32_t>(lc1 * 16);
    const uint32_t row_off = static_cast<uint32_t>((lane >> 3) * K);
    auto issue = [&](int s, int st, bool scales) {
      const uint32_t k0 = static_cast<uint32_t>(s * kSlab);
#pragma unroll
      for (int j = 0; j < IA; ++j)
        dma16(ra, lds_addr(Abuf[st] + j * 1024),
              row_off + static_cast<uint32_t>(j * 8 * K) + k0 + ((j & 1) ? c_odd : c_even));
      if constexpr (BLOCKWISE) {
        if (scales) {
#pragma unroll
          for (int j = 0; j < IS; ++j)
            dma4(rs, lds_addr(Sbuf[st] + j * 64),
                 E8M0 ? static_cast<uint32_t>((j * 64 + lane) * KG4 + (s & ~3))
                      : static_cast<uint32_t>(((j * 64 + lane) * KG + s) * 4));
        }
      }
    };
    if (pre) {
      // the M scale rows in 256-byte pieces (scale pointers are only 4-byte aligned), at
      // most 48 in flight.  Slab 0's wait covers them all.  Rows M .. 16 MB are not staged:
      // their A rows are zero and their outputs are not stored.
      const int pieces = (M * srow_bytes + 255) / 256;
      for (int j = 0; j < pieces; ++j) {
        if (j >= 48) wait_vmcnt<47>();
        dma4(rs, lds_addr(Spre + j * 256), static_cast<uint32_t>(j * 256 + lane * 4));
      }
#pragma unroll
      for (int p = 0; p < NS - 1; ++p)
        if (p < nslabs) issue(p, p, false);
      for (int s = 0; s < nslabs; ++s) {
        wait_slabs_ahead<IA, NS - 2>(min(NS - 2, nslabs - 1 - s));
        stage_barrier();
        if (s + NS - 1 < nslabs) issue(s + NS - 1, (s + NS - 1) % NS, false);
      }
    } else {
#pragma unroll
      for (int p = 0; p < NS - 1; ++p)
        if (p < nslabs) issue(p, p, true);
      for (int s = 0; s < nslabs; ++s) {
        wait_slabs_ahead<PER, NS - 2>(min(NS - 2, nslabs - 1 - s));
        stage_barrier();
        if (s + NS - 1 < nslabs) issue(s + NS - 1, (s + NS - 1) % NS, true);
      }
    }
    return;
  }

  // ---- compute waves ----
  const int r16 = lane & 15, kq = lane >> 4;
  const int n0 = (nblk * cw + w) * 16 * NB;          // this wave's first weight row
  FragFactors<SM, MB, NB> ff;                        // rowwise epilogue scales, fetched now
  ff.load(sa, sb, 0, n0, M, N);
  // (readfirstlane keeps the clamp on the scalar unit: a VGPR range would make every
  // buffer load a waterfall loop)
  const int rows = __builtin_amdgcn_readfirstlane(max(0, min(16 * NB, N - n0)));
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qb + static_cast<int64_t>(min(n0, N)) * K), static_cast<short>(0), rows * K,
      static_cast<int>(kRsrcWord3));
  // this wave's weight-block row of sb: KG float32 scales, or KG4 UE8M0 bytes
  const int64_t sb_row = static_cast<int64_t>(min(n0, N - 1) / kSlab);
  const __amdgpu_buffer_rsrc_t sbr = __builtin_amdgcn_make_buffer_rsrc(
      E8M0 ? const_cast<uint8_t*>(static_cast<const uint8_t*>(sb_) + sb_row * KG4)
           : static_cast<void*>(const_cast<float*>(sb + (BLOCKWISE ? sb_row * KG : 0))),
      static_cast<short>(0), BLOCKWISE && rows > 0 ? (E8M0 ? KG4 : KG * 4) : 0, static_cast<int>(kRsrcWord3));

  // operands of slab i in slot u; past the last slab every load reads zeros
  v8i wf[UNROLL][NB];
  float sbv[UNROLL];
  auto fetch = [&](int i, int u) {
    const bool live = i < nslabs;                    // wave-uniform
    const uint32_t kk = static_cast<uint32_t>(i * kSlab + kq * 32);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int row = 16 * j + r16;
      const uint32_t off = static_cast<uint32_t>(row * K) + kk;
      const bool in = live && row < rows;
      const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(wr, in ? off : kOOB, 0, 0);
      const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(wr, in ? off + 16 : kOOB, 0, 0);
      wf[u][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    if constexpr (BLOCKWISE)   // UE8M0: the 32-bit word holding slab i's byte, kept as bits
      sbv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          sbr, live ? static_cast<uint32_t>(E8M0 ? (i & ~3) : i * 4) : kOOB, 0, 0));
  };
  auto frag = [&](const uint8_t* base, int row) -> v8i {
    const int sw = swz(row);
    const v4i lo = *reinterpret_cast<const v4i*>(base + row * kSlab + (((2 * kq) ^ sw) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(base + row * kSlab + (((2 * kq + 1) ^ sw) << 4));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  v4f acc[NB][MB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[j][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  auto consume = [&](int s, int u) {
    const int st = s % NS;
    const uint8_t* As = Abuf[st];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const v8i af = frag(As, 16 * b + r16);
      float scl = 0.0f;
      int ea = 127, eb = 127;
      if constexpr (E8M0) {
        ea = pre ? static_cast<int>(Spre[(16 * b + r16) * KG4 + s])
                 : e8m0_byte(__float_as_uint(Sbuf[st][16 * b + r16]), s);
        eb = e8m0_byte(__float_as_uint(sbv[u]), s);
      } else if constexpr (BLOCKWISE) {
        scl = (pre ? reinterpret_cast<const float*>(Spre)[(16 * b + r16) * KG + s] : Sbuf[st][16 * b + r16]) * sbv[u];
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if constexpr (E8M0) {
          acc[j][b] = mfma_fp8_e8m0(wf[u][j], af, acc[j][b], eb, ea);
        } else if constexpr (BLOCKWISE) {
          const v4f p = mfma_fp8(wf[u][j], af, v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][b][r] = __builtin_fmaf(p[r], scl, acc[j][b][r]);
        } else {
          acc[j][b] = mfma_fp8(wf[u][j], af, acc[j][b]);
        }
      }
    }
  };

  // Rolling W pipeline as in the decode kernel: the first pass only loads, pass `it`
  // multiplies slabs (it - 1) UNROLL + u and refills their registers with it UNROLL + u,
  // and the last pass only multiplies.  Every multiplied slab is preceded by its barrier.
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
    for (int j = 0; j < NB; ++j) wf[u][j] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    sbv[u] = 0.0f;
  }
  const int iters = (nslabs + UNROLL - 1) / UNROLL;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (it > 0) {
        stage_barrier();
        consume((it - 1) * UNROLL + u, u);
      }
      fetch(it * UNROLL + u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int s = (iters - 1) * UNROLL + u;
    if (s < nslabs) {
      stage_barrier();
      consume(s, u);
    }
  }

  float alpha = 1.0f;
  if constexpr (SM == SM_TENSOR) alpha = sa[0] * sb[0];
  const bool vec_store = (N & 3) == 0;
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
      if (vec_store && n + 3 < N) {
        *reinterpret_cast<uint2*>(crow + n) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) crow[n + r] = static_cast<uint16_t>(h[r]);
      }
    }
  }
}

template <int SM, int OUT, int NB, int MB, int NS, int UNROLL>
__global__ __launch_bounds__((kSkinnyMaxCw + 1) * 64) void gemm_skinny_kernel(
    const uint8_t* __restrict__ qa, const void* __restrict__ sa, const uint8_t* __restrict__ qb,
    const void* __restrict__ sb, int M, int N, int K, int cw, uint16_t* __restrict__ c) {
  using Shape = SkinnyShape<SM, MB>;
  __shared__ __attribute__((aligned(1024))) uint8_t Abuf[NS][Shape::A_BYTES];
  __shared__ __attribute__((aligned(16))) float Sbuf[NS][Shape::S_FLOATS];
  __shared__ __attribute__((aligned(16))) uint8_t Spre[Shape::PRE_BYTES];
  skinny_body<SM, OUT, NB, MB, NS, UNROLL>(qa, sa, qb, sb, M, N, K, cw, c, blockIdx.x, Abuf, Sbuf, Spre);
}

// Grouped (mixture-of-experts) product: expert e's tokens are the rows
// [offsets[e], offsets[e + 1]) of A and C, multiplied by its weight qb[e] with its block
// scales (the fine-grained FP8 page's expert products).  Each workgroup takes one tile:
// chunk j of 16 MB consecutive tokens of one expert, times weight block `nblk` of that
// expert (16 cw NB rows).  Its first wave finds the tile from the offsets alone - the
// number of chunks of each expert, prefix-summed 64 experts at a time - so the group sizes
// never go to the host and the launch can be captured in a graph.  The grid is sized for
// the worst case (sum_e ceil(m_e / chunk) <= T / chunk + E); workgroups past the last tile
// return before their first barrier.  Offsets are clamped to [0, T] and an expert whose end
// lies before its start is empty, so any offsets give in-bounds accesses.
template <int SM, int OUT, int NB, int MB, int NS, int UNROLL>
__global__ __launch_bounds__((kSkinnyMaxCw + 1) * 64) void gemm_grouped_kernel(
    const uint8_t* __restrict__ qa, const void* __restrict__ sa, const uint8_t* __restrict__ qb,
    const void* __restrict__ sb, const int* __restrict__ offsets, int E, int T, int N, int K, int cw,
    int nblks, uint16_t* __restrict__ c) {
  using Shape = SkinnyShape<SM, MB>;
  __shared__ __attribute__((aligned(1024))) uint8_t Abuf[NS][Shape::A_BYTES];
  __shared__ __attribute__((aligned(16))) float Sbuf[NS][Shape::S_FLOATS];
  __shared__ __attribute__((aligned(16))) uint8_t Spre[Shape::PRE_BYTES];
  __shared__ int tile[3];                           // expert (-1: none), first row, rows
  constexpr int CH = 16 * MB;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int chunk = blockIdx.x / nblks;
    int base = 0, found = -1, row0 = 0, rows = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {            // uniform loop
      const int e = e0 + lane;
      int lo = 0, m = 0;
      if (e < E) {
        lo = min(max(offsets[e], 0), T);
        m = min(max(offsets[e + 1], lo), T) - lo;
      }
      const int n_ch = (m + CH - 1) / CH;
      int incl = n_ch;                              // inclusive prefix over the 64 experts
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      const int first = base + incl - n_ch;         // this expert's first chunk
      const bool mine = chunk >= first && chunk < base + incl;
      const uint64_t hit = __ballot(mine);
      if (hit) {
        const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        const int j = chunk - first;                // chunk within the expert
        found = __shfl(e, src, 64);
        row0 = __shfl(lo + j * CH, src, 64);
        rows = __shfl(min(CH, m - j * CH), src, 64);
        break;
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      tile[0] = found;
      tile[1] = row0;
      tile[2] = rows;
    }
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(tile[0]);
  if (e < 0) return;                                // every wave alike, before any barrier
  const int row0 = __builtin_amdgcn_readfirstlane(tile[1]);
  const int rows = __builtin_amdgcn_readfirstlane(tile[2]);
  const int KG = K / kSlab;
  const int64_t sa_row = SM == SM_E8M0 ? e8m0_row_bytes(KG) : int64_t{4} * KG;   // bytes per scale row
  const int64_t sb_rows = (N + kSlab - 1) / kSlab;
  skinny_body<SM, OUT, NB, MB, NS, UNROLL>(
      qa + static_cast<int64_t>(row0) * K, static_cast<const uint8_t*>(sa) + row0 * sa_row,
      qb + static_cast<int64_t>(e) * N * K, static_cast<const uint8_t*>(sb) + e * sb_rows * sa_row,
      rows, N, K, cw, c + static_cast<int64_t>(row0) * N, blockIdx.x % nblks, Abuf, Sbuf, Spre);
}

template <int SM, int OUT, int NB, int MB, int NS, int UNROLL>
void launch_skinny(const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa, const uint8_t* qb,
                   const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  gemm_skinny_kernel<SM, OUT, NB, MB, NS, UNROLL><<<static_cast<unsigned>(L.grid), static_cast<unsigned>(L.threads), 0, s>>>(
      qa, sa, qb, sb, M, N, K, L.waves, static_cast<uint16_t*>(c));
}

// Weight-block scales of the columns from n_off on (n_off a multiple of 128).
template <int SM>
const void* scale_cols(const void* sb, int64_t n_off, int K) {
  if constexpr (SM == SM_BLOCK) return static_cast<const float*>(sb) + (n_off / kSlab) * (K / kSlab);
  else if constexpr (SM == SM_E8M0) return static_cast<const uint8_t*>(sb) + (n_off / kSlab) * e8m0_row_bytes(K / kSlab);
  else if constexpr (SM == SM_ROW) return static_cast<const float*>(sb) + n_off;
  else return sb;
}

// One launch of the tiled DMA kernel over the plan's columns [n_begin, n_end): the weight
// rows, block scales and C columns of that range are plain offsets (it starts on a whole
// weight block), and C keeps its full row pitch N.
template <int BM, int BN, int WM, int WN, int SM, int OUT, int NS, bool PAIR>
void launch_tile(const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa, const uint8_t* qb,
                 const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  const int n = static_cast<int>(L.n_end - L.n_begin);
  gemm_dma_kernel<BM, BN, WM, WN, SM, OUT, NS, PAIR><<<static_cast<unsigned>(L.grid), (dma_threads<BM, BN, WM, WN>()), 0, s>>>(
      qa, sa, qb + L.n_begin * K, scale_cols<SM>(sb, L.n_begin, K), M, n, K,
      static_cast<uint16_t*>(c) + L.n_begin, (M + BM - 1) / BM, (n + BN - 1) / BN, N);
}

template <int BM, int BN, int WM, int WN, int SM, int OUT>
void launch_cfg(const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa, const uint8_t* qb,
                const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  gemm_fp8_kernel<BM, BN, WM, WN, SM, OUT><<<static_cast<unsigned>(L.grid), kThreads, 0, s>>>(
      qa, sa, qb, sb, M, N, K, static_cast<uint16_t*>(c), (M + BM - 1) / BM);
}

// Carries out one launch of a plan (plan_gemm in gemm_plan.hpp chooses the kernel, tile,
// grid and columns, and measures why).  Returns false for a launch no kernel here matches.
template <int SM, int OUT>
bool run_launch(const fp8_gemm_launch_t& L, const uint8_t* qa, const void* sa, const uint8_t* qb,
                const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  constexpr bool BW = slab_scaled(SM);
  constexpr bool PAIR = SM != SM_BLOCK;            // the 256x256 kernel's DMA issue, per mode
  switch (L.kernel) {
    case FP8_KERNEL_GEMV_STREAM:
    case FP8_KERNEL_GEMV_VALU:
    case FP8_KERNEL_GEMV_MFMA:
      return launch_gemv(SM, OUT, L, qa, sa, qb, sb, M, N, K, c, s);
    case FP8_KERNEL_STAGED:
      if (L.tile_m == 16) launch_cfg<16, 256, 16, 64, SM, OUT>(L, qa, sa, qb, sb, M, N, K, c, s);
      else launch_cfg<128, 128, 64, 64, SM, OUT>(L, qa, sa, qb, sb, M, N, K, c, s);
      return true;
    case FP8_KERNEL_SKINNY:
      if (L.variant == 2) launch_skinny<SM, OUT, 1, 2, 4, 4>(L, qa, sa, qb, sb, M, N, K, c, s);
      else if (L.variant == 4) launch_skinny<SM, OUT, 1, 4, 4, 4>(L, qa, sa, qb, sb, M, N, K, c, s);
      else if constexpr (BW) launch_skinny<SM, OUT, 1, 8, 5, 2>(L, qa, sa, qb, sb, M, N, K, c, s);
      else launch_skinny<SM, OUT, 1, 8, 5, 4>(L, qa, sa, qb, sb, M, N, K, c, s);
      return true;
    case FP8_KERNEL_TILE:
      if (L.tile_m == 256 && L.tile_n == 256) {
        if (L.paired != (PAIR ? 1 : 0)) return false;
        launch_tile<256, 256, 64, 128, SM, OUT, 2, PAIR>(L, qa, sa, qb, sb, M, N, K, c, s);
      } else if (L.tile_m == 256) {
        if (L.variant == 3) launch_tile<256, 128, 64, 64, SM, OUT, 3, false>(L, qa, sa, qb, sb, M, N, K, c, s);
        else launch_tile<256, 128, 64, 64, SM, OUT, 2, false>(L, qa, sa, qb, sb, M, N, K, c, s);
      } else if (L.tile_n == 96) {
        if constexpr (slab_scaled(SM)) return false;   // 48-column waves: no per-block scales
        else launch_tile<128, 96, 64, 48, SM, OUT, 3, false>(L, qa, sa, qb, sb, M, N, K, c, s);
      } else if (L.waves == 4) {
        launch_tile<128, 128, 64, 64, SM, OUT, 2, false>(L, qa, sa, qb, sb, M, N, K, c, s);
      } else {
        launch_tile<128, 128, 64, 32, SM, OUT, 3, false>(L, qa, sa, qb, sb, M, N, K, c, s);
      }
      return true;
    default:
      return false;
  }
}

template <int SM, int OUT>
bool launch_gemm_t(const fp8_gemm_plan_t& p, const uint8_t* qa, const void* sa, const uint8_t* qb,
                   const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  for (int i = 0; i < p.launches; ++i)
    if (!run_launch<SM, OUT>(p.launch[i], qa, sa, qb, sb, M, N, K, c, s)) return false;
  return true;
}

// Grouped launch: 16 MB tokens per chunk, cw compute waves of NB weight-row blocks each.
// Returns false when the worst-case grid does not fit a launch.
template <int SM, int OUT, int NB, int MB, int NS, int UNROLL>
bool launch_grouped_t(const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb, const int* offsets,
                      int E, int T, int N, int K, int cw, void* c, hipStream_t s) {
  const int rows = 16 * cw * NB;
  const int64_t nblks = (N + rows - 1) / rows;
  const int64_t chunks = (static_cast<int64_t>(T) + 16 * MB - 1) / (16 * MB) + E;
  if (chunks * nblks > (int64_t{1} << 31) - 1) return false;
  gemm_grouped_kernel<SM, OUT, NB, MB, NS, UNROLL><<<static_cast<unsigned>(chunks * nblks), (cw + 1) * 64, 0, s>>>(
      qa, sa, qb, sb, offsets, E, T, N, K, cw, static_cast<int>(nblks), static_cast<uint16_t*>(c));
  return true;
}

// Measured on MI355X (32 experts of W[4096, 7168], cold weights): two 16-row weight
// fragments per compute wave and six compute waves (192 weight rows per workgroup against a
// chunk of 128 tokens) lead at both 256 and 4096 routed rows; one fragment per wave streams
// the token chunk more often per weight byte (13% slower at 4096 rows), and chunks of 16 or
// 32 tokens gain nothing at 256 rows and multiply the weight reads at 4096.
template <int SM, int OUT>
bool launch_grouped_m(const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb, const int* offsets,
                      int E, int T, int N, int K, void* c, hipStream_t s) {
  return launch_grouped_t<SM, OUT, 2, 8, 5, 2>(qa, sa, qb, sb, offsets, E, T, N, K, 6, c, s);
}

template <int SM>
bool launch_gemm_m(const fp8_gemm_plan_t& p, int out_dt, const uint8_t* qa, const void* sa, const uint8_t* qb,
                   const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  if (out_dt == DT_BF16) return launch_gemm_t<SM, DT_BF16>(p, qa, sa, qb, sb, M, N, K, c, s);
  return launch_gemm_t<SM, DT_F16>(p, qa, sa, qb, sb, M, N, K, c, s);
}

}  // namespace

bool launch_grouped(int mode, int out_dt, const uint8_t* qa, const void* sa, const uint8_t* qb, const void* sb,
                    const int* offsets, int E, int T, int N, int K, void* c, hipStream_t s) {
  if (mode == SM_E8M0)
    return out_dt == DT_BF16 ? launch_grouped_m<SM_E8M0, DT_BF16>(qa, sa, qb, sb, offsets, E, T, N, K, c, s)
                             : launch_grouped_m<SM_E8M0, DT_F16>(qa, sa, qb, sb, offsets, E, T, N, K, c, s);
  return out_dt == DT_BF16 ? launch_grouped_m<SM_BLOCK, DT_BF16>(qa, sa, qb, sb, offsets, E, T, N, K, c, s)
                           : launch_grouped_m<SM_BLOCK, DT_F16>(qa, sa, qb, sb, offsets, E, T, N, K, c, s);
}

bool launch_gemm(int mode, int out_dt, const fp8_gemm_plan_t& p, const uint8_t* qa, const void* sa,
                 const uint8_t* qb, const void* sb, int M, int N, int K, void* c, hipStream_t s) {
  if (mode == SM_ROW) return launch_gemm_m<SM_ROW>(p, out_dt, qa, sa, qb, sb, M, N, K, c, s);
  if (mode == SM_E8M0) return launch_gemm_m<SM_E8M0>(p, out_dt, qa, sa, qb, sb, M, N, K, c, s);
  if (mode == SM_BLOCK) return launch_gemm_m<SM_BLOCK>(p, out_dt, qa, sa, qb, sb, M, N, K, c, s);
  return launch_gemm_m<SM_TENSOR>(p, out_dt, qa, sa, qb, sb, M, N, K, c, s);
}

}  // namespace fp8amax
