// gemv.hip - the decode regime (M <= 16 tokens) of the scaled FP8 GEMM, for gfx950.
//
// Same operation as gemm.hip (Transformer Engine page "Что такое FP8 инференс на H100
// (Transformer Engine)?", section 3 steps 5-6; per-slab scales from "FP8 chi tiết",
// opening bullets), in the regime the task page times (batch 1): the weights are read once
// and the product is bound by HBM bandwidth, so the kernel is built around streaming W.
//
// Design: one workgroup per 16 rows of W.  The activations (at most 16 rows) are staged
// once in LDS.  Each of the four waves takes a quarter of the K slabs and streams its W
// slabs straight from HBM into MFMA operand registers with 16-byte buffer loads (no LDS
// round trip, no barriers in the loop), keeping kUnroll slabs in flight; rows past N read
// as zero through the buffer range check.  One v_mfma_scale_f32_16x16x128_f8f6f4 per slab
// (W as the first operand, A padded to 16 rows as the second) gives lane l the partial
// sums of C[m = l % 16][n = n0 + 4 * (l / 16) + r].  The four K quarters are summed in LDS
// and the epilogue scales and stores.
#include "fp8_device.hpp"
#include "launch.hpp"

namespace fp8amax {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kSlab = 128;
constexpr int kUnroll = 4;                 // W slabs in flight per wave
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOOB = 0x80000000u;     // offset past any range: the load returns zeros
constexpr int kMaxLds = 160 * 1024;

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
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

// A row stride in LDS: K plus 16 bytes, so the 16 rows a fragment read touches fall in
// different banks.
__host__ __device__ constexpr int a_stride(int K) { return K + 16; }

template <bool BLOCKWISE, int OUT>
__global__ __launch_bounds__(kThreads) void gemv_fp8_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa, const uint8_t* __restrict__ qb,
    const float* __restrict__ sb, int M, int N, int K, uint16_t* __restrict__ c) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* a_lds = smem;                                       // [M][K + 16]
  float* red = reinterpret_cast<float*>(smem + M * a_stride(K));  // [kWaves][64][4]

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int nslabs = (K + kSlab - 1) / kSlab;
  const int KG = K / kSlab;                                   // blockwise: K % 128 == 0

  // stage A (M rows of K bytes) in LDS, 16 bytes per thread per step
  for (int i = t; i < M * (K / 16); i += kThreads) {
    const int m = i / (K / 16), k16 = i - m * (K / 16);
    *reinterpret_cast<uint4*>(a_lds + m * a_stride(K) + k16 * 16) =
        *reinterpret_cast<const uint4*>(qa + static_cast<int64_t>(m) * K + k16 * 16);
  }

  // this wave's slabs: an even share of [0, nslabs)
  const int per = (nslabs + kWaves - 1) / kWaves;
  const int s_begin = min(w * per, nslabs), s_end = min(s_begin + per, nslabs);

  // W rows n0..n0+15 as one buffer; lane reads 32 bytes of row n0 + r16 per slab
  const int rows = min(16, N - n0);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qb + static_cast<int64_t>(n0) * K), static_cast<short>(0),
      rows * K, static_cast<int>(kRsrcWord3));
  const uint32_t lane_off = static_cast<uint32_t>(r16 * K + kq * 32);
  // each 16-byte half is checked on its own: with K % 128 != 0 a lane's 32 bytes can
  // straddle the end of the row
  auto load_w = [&](int s) -> v8i {
    const int kk = s * kSlab + kq * 32;
    const uint32_t off = lane_off + s * kSlab;
    const uint32_t off_lo = (r16 < rows && kk < K) ? off : kOOB;
    const uint32_t off_hi = (r16 < rows && kk + 16 < K) ? off + 16 : kOOB;
    const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(wr, off_lo, 0, 0);
    const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(wr, off_hi, 0, 0);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto a_frag = [&](int s) -> v8i {
    const int kk = s * kSlab + kq * 32;
    v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (r16 < M) {
      const uint8_t* p = a_lds + r16 * a_stride(K) + kk;
      if (kk < K) lo = *reinterpret_cast<const v4i*>(p);
      if (kk + 16 < K) hi = *reinterpret_cast<const v4i*>(p + 16);
    }
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  __syncthreads();

  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int nb = n0 / kSlab;
  for (int s0 = s_begin; s0 < s_end; s0 += kUnroll) {
    v8i wf[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) wf[u] = load_w(min(s0 + u, s_end - 1));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = s0 + u;
      if (s >= s_end) break;
      const v8i af = a_frag(s);
      if constexpr (BLOCKWISE) {
        const float scale = (r16 < M) ? sa[static_cast<int64_t>(r16) * KG + s] * sb[static_cast<int64_t>(nb) * KG + s] : 0.0f;
        const v4f p = mfma_fp8(wf[u], af, v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(p[r], scale, acc[r]);
      } else {
        acc = mfma_fp8(wf[u], af, acc);
      }
    }
  }

  // sum the four K quarters in LDS
  *reinterpret_cast<v4f*>(red + (w * 64 + lane) * 4) = acc;
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int q = 1; q < kWaves; ++q) {
    const v4f o = *reinterpret_cast<const v4f*>(red + (q * 64 + lane) * 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += o[r];
  }
  float alpha = 1.0f;
  if constexpr (!BLOCKWISE) alpha = sa[0] * sb[0];
  const int m = r16;
  if (m >= M) return;
  const int n = n0 + 4 * kq;
  uint32_t h[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) h[r] = f32_to_out_bits<OUT>(acc[r] * alpha);
  uint16_t* crow = c + static_cast<int64_t>(m) * N;
  if ((N & 3) == 0 && n + 3 < N) {
    *reinterpret_cast<uint2*>(crow + n) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) crow[n + r] = static_cast<uint16_t>(h[r]);
  }
}

template <bool BW, int OUT>
void launch_t(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb, int M, int N,
              int K, void* c, hipStream_t s) {
  const size_t lds = static_cast<size_t>(M) * a_stride(K) + kWaves * 64 * 4 * sizeof(float);
  static bool attr_set = false;      // allow the full LDS of a CU for dynamic shared memory
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_fp8_kernel<BW, OUT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    attr_set = true;
  }
  gemv_fp8_kernel<BW, OUT><<<(N + 15) / 16, kThreads, lds, s>>>(qa, sa, qb, sb, M, N, K,
                                                                static_cast<uint16_t*>(c));
}

}  // namespace

size_t gemv_lds_bytes(int M, int K) {
  return static_cast<size_t>(M) * a_stride(K) + kWaves * 64 * 4 * sizeof(float);
}

void launch_gemv(bool blockwise, int out_dt, const uint8_t* qa, const float* sa, const uint8_t* qb,
                 const float* sb, int M, int N, int K, void* c, hipStream_t s) {
  if (blockwise) {
    if (out_dt == DT_BF16) launch_t<true, DT_BF16>(qa, sa, qb, sb, M, N, K, c, s);
    else launch_t<true, DT_F16>(qa, sa, qb, sb, M, N, K, c, s);
  } else {
    if (out_dt == DT_BF16) launch_t<false, DT_BF16>(qa, sa, qb, sb, M, N, K, c, s);
    else launch_t<false, DT_F16>(qa, sa, qb, sb, M, N, K, c, s);
  }
}

}  // namespace fp8amax
