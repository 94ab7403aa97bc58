// quantize.hip - amax, scale and e4m3 cast kernels for gfx950.
//
// Steps (Transformer Engine page "Что такое FP8 инференс на H100 (Transformer Engine)?",
// section 3 steps 2-4): amax of the operand, scale = amax / 448, x / scale rounded to
// e4m3.  Block shapes ("FP8 chi tiết", opening bullets): per token in groups of 128 input
// channels, and 128x128 weight blocks.
//
// All kernels are HBM-bound streaming passes: 16-byte loads of eight 16-bit inputs per
// lane, 8-byte stores of eight codes.  For groups and blocks the amax, scale and cast are
// fused in one pass that keeps the block's inputs in registers between the reduction and
// the cast.
//
// Kernels: 1x128 groups and 128x128 blocks (float32 or UE8M0 scales); the whole tensor
// (amax, then cast; one workgroup for small tensors); one scale per row (per output
// channel or per token, the same page's per-channel scaling, section 5); the static cast
// with a scale fixed in advance and the delayed-scaling update (the task page's
// DelayedScaling recipe).
#include "fp8_device.hpp"
#include "launch.hpp"
#include "quant_device.hpp"

namespace fp8amax {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------------------------
// Per-token 1x128 groups.  Sixteen lanes (one DPP row) own one group, 8 elements each.
// Each 16-lane set takes one (row, chunk) pair: `cg` consecutive groups of one row,
// walked UNROLL groups at a time with all loads issued before the reductions.
// Vector path: cols % 8 == 0 (a lane's eight elements are all inside or all outside).
// WRITE_Q = false computes only the amax grid (fp8_amax with 1x128 blocks).  E8M0: the
// scales are UE8M0 codes (bytes) instead of float32.
template <int DT, bool WRITE_Q, int UNROLL, bool E8M0 = false>
__global__ __launch_bounds__(kThreads) void group_1x128_vec_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t nch, int64_t cg,
    uint8_t* __restrict__ q, void* __restrict__ out, int64_t sstride) {
  const int64_t gcols = (cols + 127) >> 7;
  const int sub = threadIdx.x & 15;
  const int64_t nsets = rows * nch;
  const int64_t set_stride = (static_cast<int64_t>(gridDim.x) * kThreads) >> 4;
  for (int64_t set = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 4; set < nsets;
       set += set_stride) {                        // whole 16-lane sets iterate together
  const int64_t row = set / nch;
  const int64_t g_begin = (set - row * nch) * cg;
  const int64_t g_end = min(g_begin + cg, gcols);
  const uint16_t* xrow = x + row * cols;
  for (int64_t g0 = g_begin; g0 < g_end; g0 += UNROLL) {
    U4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t col = ((g0 + u) << 7) + (sub << 3);
      v[u] = {0u, 0u, 0u, 0u};
      if (g0 + u < g_end && col < cols) v[u] = load16(xrow + col);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t g = g0 + u;
      if (g >= g_end) break;                       // uniform within the set
      const int64_t col = (g << 7) + (sub << 3);
      const uint32_t key = max16(key8(v[u]));
      const float amax = amax_from_key<DT>(key);
      if constexpr (WRITE_Q) {
        const GroupScale<E8M0> gs(amax);
        const float scale = gs.scale;
        const bool fast = fast_scale(scale);
        const float r = 1.0f / scale;
        if (col < cols) *reinterpret_cast<uint2*>(q + row * cols + col) = enc8<DT>(v[u], scale, r, fast);
        if (sub == 0) gs.store(out, row, g, gcols, sstride);
      } else {
        if (sub == 0) static_cast<float*>(out)[row * gcols + g] = amax;
      }
    }
  }
  }
}

// Rows of whole groups (cols % 128 == 0): the groups are contiguous in memory, group g at
// x + 128 g, so the tensor is one flat run of groups.  Eight lanes own a group, sixteen
// elements (two 16-byte loads, one 16-byte store) each, and a wave takes eight consecutive
// groups per step: its two load instructions cover one contiguous 2 KB piece and its store
// 1 KB.  Against sixteen lanes of eight elements, the group's scale, reciprocal and lane
// reduction are paid once per sixteen elements of a lane instead of eight.  Measured on
// MI355X (A[4096, 7168] and A[4096, 4096], cold): 17.2 and 11.6 us against 19.0 and
// 12.1 us for sixteen lanes per group, and 17.1 and 11.7 us for the byte-mix reference
// (the same bytes moved with no arithmetic); two steps in flight per wave were no faster.
template <int DT, bool WRITE_Q, bool E8M0 = false>
__global__ __launch_bounds__(kThreads) void group_1x128_flat_kernel(
    const uint16_t* __restrict__ x, int64_t ngroups, int64_t gcols, uint8_t* __restrict__ q,
    void* __restrict__ out, int64_t sstride) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 7;                                   // lane within the group
  const int gw = lane >> 3;                                   // group within the wave's step
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 6;
  const int64_t waves = (static_cast<int64_t>(gridDim.x) * kThreads) >> 6;
  const int64_t wsteps = (ngroups + 7) >> 3;                  // steps of eight groups
  for (int64_t i = wave; i < wsteps; i += waves) {
    const int64_t g = (i << 3) + gw;
    if (g >= ngroups) continue;                               // uniform within the group's lanes
    const uint16_t* xg = x + (g << 7) + (sub << 4);
    const U4 v0 = load16(xg), v1 = load16(xg + 8);
    const float amax = amax_from_key<DT>(max8(max(key8(v0), key8(v1))));
    if constexpr (WRITE_Q) {
      const GroupScale<E8M0> gs(amax);
      const float scale = gs.scale;
      const bool fast = fast_scale(scale);
      const float r = 1.0f / scale;
      const uint2 a = enc8<DT>(v0, scale, r, fast), b = enc8<DT>(v1, scale, r, fast);
      *reinterpret_cast<uint4*>(q + (g << 7) + (sub << 4)) = make_uint4(a.x, a.y, b.x, b.y);
      if (sub == 0) {
        const int64_t row = g / gcols;
        gs.store(out, row, g - row * gcols, gcols, sstride);
      }
    } else {
      if (sub == 0) static_cast<float*>(out)[g] = amax;
    }
  }
}

// Scalar path for rows whose length is not a multiple of 8: one group per 16-lane set.
template <int DT, bool WRITE_Q, bool E8M0 = false>
__global__ __launch_bounds__(kThreads) void group_1x128_scalar_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
    void* __restrict__ out, int64_t sstride) {
  const int64_t gcols = (cols + 127) >> 7;
  const int64_t ngroups = rows * gcols;
  const int sub = threadIdx.x & 15;
  const int64_t g_stride = (static_cast<int64_t>(gridDim.x) * kThreads) >> 4;
  for (int64_t g = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 4; g < ngroups;
       g += g_stride) {
  const int64_t row = g / gcols;
  const int64_t gc = g - row * gcols;
  const int64_t col0 = (gc << 7) + (sub << 3);
  uint32_t h[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = (col0 + i < cols) ? x[row * cols + col0 + i] : 0u;
    m = max(m, h[i] & 0x7fffu);
  }
  const uint32_t key = max16(m);
  const float amax = amax_from_key<DT>(key);
  if constexpr (WRITE_Q) {
    const GroupScale<E8M0> gs(amax);
    const float scale = gs.scale;
    const bool fast = fast_scale(scale);
    const float r = 1.0f / scale;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (col0 + i < cols) q[row * cols + col0 + i] = enc1<DT>(h[i], scale, r, fast);
    if (sub == 0) gs.store(out, row, gc, gcols, sstride);
  } else {
    if (sub == 0) static_cast<float*>(out)[g] = amax;
  }
  }
}

// ------------------------------------------------------------------------------------
// Per-row scales (per output channel of the weights, per token of the activations; the
// Transformer Engine page's per-channel scaling): scale = amax of the row / 448, the row
// cast with it.  Rows of up to 16384 elements stay in registers between the reduction and
// the cast: WPR = 1 gives a row to one wave (VEC 16-byte pieces per lane, up to 4096
// elements), WPR = 4 to the whole workgroup (up to 16384).  Each row is read through a
// buffer resource of exactly its bytes, so pieces past its end load as zeros and every load
// is issued without a branch.  cols % 8 == 0 (every row starts 16-byte aligned).
template <int DT, int WPR, int VEC>
__global__ __launch_bounds__(kThreads) void rows_vec_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ q,
                                                            float* __restrict__ scales) {
  static_assert(WPR == 1 || WPR == kThreads / 64, "a row per wave or per workgroup");
  constexpr int T = 64 * WPR;                  // threads per row
  constexpr int RPB = kThreads / T;            // rows per workgroup and pass
  __shared__ uint32_t part[kThreads / 64];
  const int lt = threadIdx.x % T;
  const int grp = threadIdx.x / T;
  const int64_t nv = cols >> 3;
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * RPB; row0 < rows;
       row0 += static_cast<int64_t>(gridDim.x) * RPB) {
    // the row is uniform over its wave(s): keep it, and the resource, in scalar registers
    const int64_t row = row0 + __builtin_amdgcn_readfirstlane(grp);
    const bool live = row < rows;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x + (live ? row : 0) * cols), static_cast<short>(0),
        live ? static_cast<int>(2 * cols) : 0, static_cast<int>(0x00020000));
    U4 v[VEC];
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
      v[u] = __builtin_bit_cast(U4, __builtin_amdgcn_raw_buffer_load_b128(xr, 16 * (lt + u * T), 0, 0));
      m = max(m, key8(v[u]));
    }
    m = max64(m);
    if constexpr (WPR > 1) {
      if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) m = max(m, part[w]);
      __syncthreads();                          // part is rewritten for the next row
    }
    if (live) {
      const float scale = scale_from_amax(amax_from_key<DT>(m));
      const bool fast = fast_scale(scale);
      const float r = 1.0f / scale;
      uint8_t* qr = q + row * cols;
#pragma unroll
      for (int u = 0; u < VEC; ++u) {
        const int64_t i = lt + u * T;
        if (i < nv) *reinterpret_cast<uint2*>(qr + (i << 3)) = enc8<DT>(v[u], scale, r, fast);
      }
      if (lt == 0) scales[row] = scale;
    }
  }
}

// Rows longer than 16384 elements (VEC) or of any length (!VEC, rows not 16-byte aligned):
// one workgroup per row, two passes - the amax, then the cast re-reading the row, which the
// first pass has just brought into the caches.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void rows_two_pass_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                 int64_t cols, uint8_t* __restrict__ q,
                                                                 float* __restrict__ scales) {
  __shared__ uint32_t part[kThreads / 64];
  const int t = threadIdx.x;
  const int64_t nv = VEC ? cols >> 3 : 0;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const uint16_t* xr = x + row * cols;
    uint32_t m = 0;
    int64_t i = t;
    for (; i + 3 * kThreads < nv; i += 4 * kThreads) {   // four loads in flight per lane
      const U4 v0 = load16(xr + (i << 3)), v1 = load16(xr + ((i + kThreads) << 3));
      const U4 v2 = load16(xr + ((i + 2 * kThreads) << 3)), v3 = load16(xr + ((i + 3 * kThreads) << 3));
      m = max(max(m, max(key8(v0), key8(v1))), max(key8(v2), key8(v3)));
    }
    for (; i < nv; i += kThreads) m = max(m, key8(load16(xr + (i << 3))));
    for (int64_t j = (nv << 3) + t; j < cols; j += kThreads) m = max(m, xr[j] & 0x7fffu);
    m = max64(m);
    if ((t & 63) == 0) part[t >> 6] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) m = max(m, part[w]);
    __syncthreads();
    const float scale = scale_from_amax(amax_from_key<DT>(m));
    const bool fast = fast_scale(scale);
    const float r = 1.0f / scale;
    uint8_t* qr = q + row * cols;
    for (int64_t v = t; v < nv; v += kThreads)
      *reinterpret_cast<uint2*>(qr + (v << 3)) = enc8<DT>(load16(xr + (v << 3)), scale, r, fast);
    for (int64_t j = (nv << 3) + t; j < cols; j += kThreads) qr[j] = enc1<DT>(xr[j], scale, r, fast);
    if (t == 0) scales[row] = scale;
  }
}

// ------------------------------------------------------------------------------------
// 128x128 weight blocks: one workgroup per block.  Thread t owns columns
// [8*(t%16), +8) of rows t/16 + 16*i, i = 0..7: eight 16-byte loads held in registers
// through the block-wide reduction, then cast and stored.  VEC: cols % 8 == 0.
template <int DT, bool WRITE_Q, bool VEC, bool E8M0 = false>
__global__ __launch_bounds__(kThreads) void block_128x128_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
    void* __restrict__ out, int64_t sstride) {
  __shared__ uint32_t wave_max[kThreads / 64];
  const int64_t bcols = (cols + 127) >> 7;
  const int64_t nblocks = ((rows + 127) >> 7) * bcols;
  const int t = threadIdx.x;
  for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
  const int64_t br = blk / bcols;
  const int64_t bc = blk - br * bcols;
  const int64_t col = (bc << 7) + ((t & 15) << 3);
  const int64_t row0 = (br << 7) + (t >> 4);
  U4 v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = row0 + 16 * i;
    v[i] = {0u, 0u, 0u, 0u};
    if constexpr (VEC) {
      if (row < rows && col < cols) v[i] = load16(x + row * cols + col);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        h[e] = (row < rows && col + e < cols) ? x[row * cols + col + e] : 0u;
      v[i] = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
    m = max(m, key8(v[i]));
  }
  m = max64(m);
  if ((t & 63) == 0) wave_max[t >> 6] = m;
  __syncthreads();
  m = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  __syncthreads();                                 // wave_max is rewritten next iteration
  const float amax = amax_from_key<DT>(m);
  if constexpr (WRITE_Q) {
    const GroupScale<E8M0> gs(amax);
    const float scale = gs.scale;
    const bool fast = fast_scale(scale);
    const float r = 1.0f / scale;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = row0 + 16 * i;
      if (row >= rows) continue;
      const uint2 o = enc8<DT>(v[i], scale, r, fast);
      if constexpr (VEC) {
        if (col < cols) *reinterpret_cast<uint2*>(q + row * cols + col) = o;
      } else {
        const uint32_t b[2] = {o.x, o.y};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < cols) q[row * cols + col + e] = static_cast<uint8_t>(b[e >> 2] >> (8 * (e & 3)));
      }
    }
    if (t == 0) gs.store(out, br, bc, bcols, sstride);
  } else {
    if (t == 0) static_cast<float*>(out)[blk] = amax;
  }
  }
}

// ------------------------------------------------------------------------------------
// Whole-tensor amax (fp8_amax).  The 32-bit result word is cleared to kKeyTag, each
// workgroup folds its max key in with a single atomicMax (no compare-and-swap retries), and
// a last one-thread launch turns the key into the float amax.
constexpr uint32_t kKeyTag = 0x80000000u;

__global__ void init_word_kernel(uint32_t* word) { *word = kKeyTag; }

// This thread's share of the whole-tensor max key: 16-byte pieces at a grid stride, four
// loads in flight per lane, then the scalar tail.
__device__ __forceinline__ uint32_t tensor_key_share(const uint16_t* __restrict__ x, int64_t n) {
  const int64_t nvec = n >> 3;
  uint32_t m = 0;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = tid;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const U4 v0 = load16(x + (i << 3)), v1 = load16(x + ((i + stride) << 3));
    const U4 v2 = load16(x + ((i + 2 * stride) << 3)), v3 = load16(x + ((i + 3 * stride) << 3));
    m = max(max(m, max(key8(v0), key8(v1))), max(key8(v2), key8(v3)));
  }
  for (; i < nvec; i += stride) m = max(m, key8(load16(x + (i << 3))));
  for (int64_t j = (nvec << 3) + tid; j < n; j += stride) m = max(m, x[j] & 0x7fffu);
  return m;
}

// Max key of a workgroup of WAVES waves, returned to every thread.
template <int WAVES>
__device__ __forceinline__ uint32_t block_key_max(uint32_t m, uint32_t* wave_max) {
  m = max64(m);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  m = wave_max[0];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) m = max(m, wave_max[w]);
  return m;
}

__global__ __launch_bounds__(kThreads) void tensor_amax_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                               uint32_t* word) {
  __shared__ uint32_t wave_max[kThreads / 64];
  const uint32_t m = block_key_max<kThreads / 64>(tensor_key_share(x, n), wave_max);
  if (threadIdx.x == 0) atomicMax(word, kKeyTag | m);
}

// Turns the finished reduction key into the float amax.
template <int DT>
__global__ void finalize_word_kernel(uint32_t* word) {
  *word = __float_as_uint(amax_from_key<DT>(*word & 0x7fffu));
}

// Whole-tensor quantize of more than kSmallTensor elements in two launches, with no atomics
// and no word to clear beforehand.
//  - The cast launch (tensor_cast_slots_kernel) runs B workgroups of 1024 threads over x
//    at a grid stride of 8192-element chunks, so that in its first round workgroup b writes
//    the codes of chunk b, q[b * 8192, (b + 1) * 8192), and no other workgroup writes there.
//  - The launch before it (tensor_partial_kernel, P <= 128 workgroups of 8192 elements,
//    looping over further ones for large x) reduces its share of x to a max key and stores
//    that key in slot p, the p-th 32-bit word of every chunk b < B.
//  - Cast workgroup b folds the P slots of its own chunk into the tensor's max key, so every
//    workgroup derives the same scale, and only after a barrier overwrites the chunk with
//    codes.
// The slots cost P * B scattered 4-byte stores, written back as 32-byte pieces: at most
// 1/10 of the pass's own traffic (128 x 128 of them, 0.5 MB, for 2^20 elements).
// Measured against three launches (clear a word, atomic amax, cast) in HIP graphs: 1.8 us
// less per step for A[512, 2048] and 0.7 us for A[128, 4096]; 256-thread cast workgroups
// (four times the slots) and fewer partial workgroups were slower.
constexpr int kPartialThreads = 1024;
constexpr int kCastThreads = 1024;
constexpr int64_t kCastChunk = int64_t{kCastThreads} * 8;
constexpr int kMaxPartials = 128;
constexpr int64_t kMaxCastBlocks = 1024;
static_assert(kMaxPartials * 4 <= kCastChunk && kMaxPartials <= kCastThreads, "slots fit a chunk");

__global__ __launch_bounds__(kPartialThreads) void tensor_partial_kernel(const uint16_t* __restrict__ x,
                                                                         int64_t n, int chunks,
                                                                         uint8_t* __restrict__ q) {
  __shared__ uint32_t wave_max[kPartialThreads / 64];
  const uint32_t m = block_key_max<kPartialThreads / 64>(tensor_key_share(x, n), wave_max);
  uint8_t* slot = q + 4 * static_cast<int64_t>(blockIdx.x);
  for (int b = threadIdx.x; b < chunks; b += kPartialThreads)
    *reinterpret_cast<uint32_t*>(slot + static_cast<int64_t>(b) * kCastChunk) = m;
}

template <int DT>
__global__ __launch_bounds__(kCastThreads) void tensor_cast_slots_kernel(const uint16_t* __restrict__ x,
                                                                     int64_t n, int partials,
                                                                     uint8_t* __restrict__ q,
                                                                     float* __restrict__ scale_out) {
  __shared__ uint32_t wave_max[kCastThreads / 64];
  const uint32_t* slots = reinterpret_cast<const uint32_t*>(q + static_cast<int64_t>(blockIdx.x) * kCastChunk);
  const uint32_t key = block_key_max<kCastThreads / 64>(threadIdx.x < partials ? slots[threadIdx.x] : 0u, wave_max);
  const float scale = scale_from_amax(amax_from_key<DT>(key));
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = scale;
  const bool fast = fast_scale(scale);
  const float r = 1.0f / scale;
  const int64_t nvec = n >> 3;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kCastThreads + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCastThreads;
  int64_t i = tid;
  for (; i + stride < nvec; i += 2 * stride) {      // two loads in flight per lane
    const U4 v0 = load16(x + (i << 3));
    const U4 v1 = load16(x + ((i + stride) << 3));
    *reinterpret_cast<uint2*>(q + (i << 3)) = enc8<DT>(v0, scale, r, fast);
    *reinterpret_cast<uint2*>(q + ((i + stride) << 3)) = enc8<DT>(v1, scale, r, fast);
  }
  if (i < nvec) *reinterpret_cast<uint2*>(q + (i << 3)) = enc8<DT>(load16(x + (i << 3)), scale, r, fast);
  for (int64_t j = (nvec << 3) + tid; j < n; j += stride) q[j] = enc1<DT>(x[j], scale, r, fast);
}

// ------------------------------------------------------------------------------------
// Static scaling (task page: the DelayedScaling recipe and the calibration step).  The
// scale is known before the pass - fixed by calibration, or left by the delayed-scaling
// update - so the cast needs no reduction first: one grid-stride pass casts with it
// (saturating above 448 * scale).  RECORD: each workgroup also folds the tensor's amax into
// *acc with one atomicMax on its float bits (non-negative floats, inf and the canonical NaN
// order as unsigned integers), for the next delayed-scaling update.
//
// A fixed scale does not bound the input the way a scale taken from the tensor's own amax
// does, so the cast differs from the dynamic one in three ways:
// * x is clamped to +-c, c = RN(448 s), before the division.  Every |x| >= c has a quotient
//   that encodes to 448 either way (within one float32 ulp of 448 or above it), so the
//   codes do not change, and the fast quotient keeps |x| <= ~448 s, its precondition: no
//   overflow of x*r and no infinite input reaches it.
// * NaN inputs are picked out from their bits and get code 0x7f (the exact encoder's
//   answer), since the clamp would turn them into numbers.
// * the fast quotient is used for 2^-80 <= s <= 2^119 only: above 2^119, c overflows to
//   inf (and past 2^126 the reciprocal 1/s is subnormal and loses bits); below 2^-80 the FMA
//   residual of a quotient near the smallest code (2^-10) could underflow.  Scales outside the range (and NaN, inf, zero
//   or negative ones) take the exact path: IEEE division and the software encoder.
constexpr float kStaticFastMin = 0x1p-80f;
constexpr float kStaticFastMax = 0x1p119f;

template <int DT>
__device__ __forceinline__ bool is_nan16(uint32_t h) {
  return (h & 0x7fffu) > (DT == DT_BF16 ? 0x7f80u : 0x7c00u);
}

template <int DT>
__device__ __forceinline__ float quot_static(uint32_t h, float s, float r, float c) {
  return quot_fast(__builtin_amdgcn_fmed3f(in_to_f32<DT>(h), -c, c), s, r);
}

// Four 16-bit inputs (two dwords) -> four codes, fast path of the static cast.
template <int DT>
__device__ __forceinline__ uint32_t enc4_static(uint32_t w0, uint32_t w1, float s, float r, float c) {
  const uint32_t h[4] = {w0 & 0xffffu, w0 >> 16, w1 & 0xffffu, w1 >> 16};
  uint32_t code = cvt4(quot_static<DT>(h[0], s, r, c), quot_static<DT>(h[1], s, r, c),
                       quot_static<DT>(h[2], s, r, c), quot_static<DT>(h[3], s, r, c));
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (is_nan16<DT>(h[k])) code = (code & ~(0xffu << (8 * k))) | (0x7fu << (8 * k));
  return code;
}

template <int DT>
__device__ __forceinline__ uint2 enc8_static(const U4& v, float s, float r, float c, bool fast) {
  if (fast) return make_uint2(enc4_static<DT>(v.x, v.y, s, r, c), enc4_static<DT>(v.z, v.w, s, r, c));
  return make_uint2(enc4_exact<DT>(v.x, v.y, s), enc4_exact<DT>(v.z, v.w, s));
}

template <int DT>
__device__ __forceinline__ uint8_t enc1_static(uint32_t h, float s, float r, float c, bool fast) {
  if (!fast) return static_cast<uint8_t>(e4m3_encode(in_to_f32<DT>(h) / s));
  if (is_nan16<DT>(h)) return 0x7fu;
  const float q = quot_static<DT>(h, s, r, c);
  return static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false) & 0xff);
}

// The static cast pass of one lane over a grid-strided range (four 16-byte loads in flight):
// q = e4m3(x / scale) for its elements; returns the lane's largest magnitude key when RECORD.
template <int DT, bool RECORD>
__device__ __forceinline__ uint32_t static_cast_pass(const uint16_t* __restrict__ x, int64_t n, float scale,
                                                     uint8_t* __restrict__ q, int64_t tid, int64_t stride) {
  const bool fast = scale >= kStaticFastMin && scale <= kStaticFastMax;   // false for NaN
  const float r = 1.0f / scale;
  const float c = 448.0f * scale;
  const int64_t nvec = n >> 3;
  uint32_t m = 0;
  int64_t i = tid;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    U4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = load16(x + ((i + u * stride) << 3));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (RECORD) m = max(m, key8(v[u]));
      *reinterpret_cast<uint2*>(q + ((i + u * stride) << 3)) = enc8_static<DT>(v[u], scale, r, c, fast);
    }
  }
  for (; i < nvec; i += stride) {
    const U4 v = load16(x + (i << 3));
    if constexpr (RECORD) m = max(m, key8(v));
    *reinterpret_cast<uint2*>(q + (i << 3)) = enc8_static<DT>(v, scale, r, c, fast);
  }
  for (int64_t j = (nvec << 3) + tid; j < n; j += stride) {
    if constexpr (RECORD) m = max(m, x[j] & 0x7fffu);
    q[j] = enc1_static<DT>(x[j], scale, r, c, fast);
  }
  return m;
}

// Largest key over a workgroup of WAVES waves; the result is valid in every lane of wave 0.
template <int WAVES>
__device__ __forceinline__ uint32_t block_max_key(uint32_t m, uint32_t* wave_max) {
  m = max64(m);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t k = 0;
  if (threadIdx.x < 64) {
    k = threadIdx.x < WAVES ? wave_max[threadIdx.x] : 0u;
    k = max64(k);
  }
  return k;
}

template <int DT, bool RECORD>
__global__ __launch_bounds__(kThreads) void tensor_static_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                 const float* __restrict__ scale_p,
                                                                 uint8_t* __restrict__ q, uint32_t* acc) {
  __shared__ uint32_t wave_max[kThreads / 64];
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  const uint32_t m = static_cast_pass<DT, RECORD>(x, n, *scale_p, q, tid, stride);
  if constexpr (RECORD) {
    const uint32_t k = block_max_key<kThreads / 64>(m, wave_max);
    if (threadIdx.x == 0) atomicMax(acc, __float_as_uint(amax_from_key<DT>(k)));
  }
}

// One delayed-scaling step, carried out by one wave, in two parts.  window_max takes the
// maximum (and whether a NaN occurs) over the history entries that stay, every slot but
// st % len, which this step overwrites; push_and_refresh then stores `recorded` (the amax of
// step st, float bits ordered as integers) in that slot, counts the step and, after every
// interval-th step, sets *scale = max(window) * 2^margin / 448 (all-zero window -> 1, a NaN
// in the window -> the canonical NaN).  The ring needs no head pointer: the step count says
// where the most recent amax is.  Splitting the two lets the window be read before the
// step's amax is known.
struct WindowMax {
  float m;
  bool nan;
};

__device__ __forceinline__ WindowMax wave_window_max(WindowMax w) {
  for (int o = 32; o >= 1; o >>= 1) {
    w.m = fmaxf(w.m, __shfl_xor(w.m, o, 64));
    w.nan |= __shfl_xor(static_cast<int>(w.nan), o, 64) != 0;
  }
  return w;
}

// The entry `first` of lane (the history's element lane, when lane < len) may have been
// loaded ahead of time; the loads do not depend on the slot.
__device__ __forceinline__ WindowMax window_max(const float* history, int len, int slot, float first) {
  const int lane = threadIdx.x & 63;
  WindowMax w{0.0f, false};
  for (int i = lane; i < len; i += 64) {
    const float h = i == lane ? first : history[i];
    if (i == slot) continue;
    w.nan |= h != h;
    w.m = fmaxf(w.m, h);
  }
  return wave_window_max(w);
}

__device__ __forceinline__ float history_first(const float* history, int len) {
  const int lane = threadIdx.x & 63;
  return lane < len ? history[lane] : 0.0f;
}

// Lane 0 of the wave stores.
__device__ __forceinline__ void push_and_refresh(float* history, int len, WindowMax w, float recorded,
                                                 int st, int* step, int interval, int margin,
                                                 float* scale) {
  if ((threadIdx.x & 63) != 0) return;
  history[st % len] = recorded;
  *step = st + 1;
  if ((st + 1) % interval == 0) {
    const bool nan = w.nan || recorded != recorded;
    const float m = fmaxf(w.m, recorded);
    *scale = nan ? __uint_as_float(kCanonicalNaN)
                 : (m == 0.0f ? 1.0f : __builtin_amdgcn_ldexpf(m, margin) / 448.0f);
  }
}

// The update alone: the amax recorded in *acc since the last update is pushed and *acc
// cleared.  scale_used (may be null) receives the scale before the update: the one the
// casts since the last update were made with.
__global__ __launch_bounds__(64) void delayed_update_kernel(float* history, int len, uint32_t* acc,
                                                            int* step, int interval, int margin,
                                                            float* scale, float* scale_used) {
  const int st = *step;
  const float recorded = __uint_as_float(*acc);
  const float before = *scale;
  const WindowMax w = window_max(history, len, st % len, history_first(history, len));
  push_and_refresh(history, len, w, recorded, st, step, interval, margin, scale);
  if (threadIdx.x == 0) {
    *acc = 0u;
    if (scale_used) *scale_used = before;
  }
}

// Static cast + update in one launch, for tensors of up to kSmallTensor elements: one
// workgroup casts with *scale, reduces the tensor's amax in LDS (folding in whatever *acc
// holds), and its first wave then does the update.  Every wave has read *scale before the
// barrier that precedes the update, so the scale may be rewritten.  No atomics.  (Larger
// tensors take the static cast and the update as two launches: with many workgroups the
// update could only start once all of them have recorded their amax, which inside one
// launch takes a device-scope release per workgroup - an L2 write-back on this chip - and
// that costs more than the second launch.)
constexpr int kSmallThreads = 1024;
constexpr int64_t kSmallTensor = int64_t{1} << 15;   // whole-tensor paths in one workgroup up to here

// The static cast of a tensor of at most kSmallTensor elements by one workgroup of
// kSmallThreads: each thread's (at most four) 16-byte pieces and tail element are loaded
// before the scale is needed, so the scale's load overlaps theirs instead of preceding them.
// Returns the thread's largest magnitude key; *scale_out receives the scale.
template <int DT>
__device__ __forceinline__ uint32_t static_cast_small(const uint16_t* __restrict__ x, int64_t n,
                                                      const float* scale_p, float* scale_out,
                                                      uint8_t* __restrict__ q) {
  static_assert(kSmallTensor == int64_t{4} * 8 * kSmallThreads, "four pieces per thread");
  const float scale = *scale_p;                     // issued first; waited for after x's loads
  const int t = threadIdx.x;
  const int64_t nvec = n >> 3;
  // x as a range-checked buffer of 2n bytes: loads past it read zeros, so every load is
  // issued unconditionally (no branch, no wait between them)
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), static_cast<short>(0), static_cast<int>(2 * n), static_cast<int>(0x00020000));
  U4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    v[u] = __builtin_bit_cast(U4, __builtin_amdgcn_raw_buffer_load_b128(xr, 16 * (t + u * kSmallThreads), 0, 0));
  const int64_t j = (nvec << 3) + t;                // n - 8 * nvec < 8 tail elements
  const uint32_t tail = __builtin_amdgcn_raw_buffer_load_b16(xr, static_cast<int>(2 * j), 0, 0);
  const bool fast = scale >= kStaticFastMin && scale <= kStaticFastMax;
  const float r = 1.0f / scale;
  const float c = 448.0f * scale;
  // the keys are selected, not branched on, so that no load is sunk past the scale's
  uint32_t m = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) m = max(m, t + u * kSmallThreads < nvec ? key8(v[u]) : 0u);
  m = max(m, j < n ? (tail & 0x7fffu) : 0u);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = t + u * kSmallThreads;
    if (i < nvec) *reinterpret_cast<uint2*>(q + (i << 3)) = enc8_static<DT>(v[u], scale, r, c, fast);
  }
  if (j < n) q[j] = enc1_static<DT>(tail, scale, r, c, fast);
  *scale_out = scale;
  return m;
}

template <int DT>
__global__ __launch_bounds__(kSmallThreads) void delayed_small_kernel(
    const uint16_t* __restrict__ x, int64_t n, float* history, int len, uint32_t* acc, int* step,
    int interval, int margin, float* scale, float* scale_used, uint8_t* __restrict__ q) {
  __shared__ uint32_t wave_max[kSmallThreads / 64];
  // the state the update reads is loaded with x, not after the cast: nothing writes it
  // before the update
  const int st = *step;
  const uint32_t acc0 = *acc;
  const float first = history_first(history, len);
  float s;
  const uint32_t m = static_cast_small<DT>(x, n, scale, &s, q);
  const uint32_t k = block_max_key<kSmallThreads / 64>(m, wave_max);
  if (threadIdx.x >= 64) return;
  const uint32_t recorded = max(acc0, __float_as_uint(amax_from_key<DT>(k)));
  const WindowMax w = window_max(history, len, st % len, first);
  push_and_refresh(history, len, w, __uint_as_float(recorded), st, step, interval, margin, scale);
  if (threadIdx.x == 0) {
    *acc = 0u;
    *scale_used = s;
  }
}

// Whole-tensor amax, scale and cast in one workgroup, for tensors small enough that one
// CU streams them in less time than the two-launch path spends on launches (the
// activations of decode steps).  No atomics and no result word to clear: the workgroup
// reduces in LDS, writes the finished float, and casts from the same scale.  The second
// pass re-reads x, which the first pass has just brought into the caches.
template <int DT, bool WANT_SCALE, bool WRITE_Q>
__global__ __launch_bounds__(kSmallThreads) void tensor_small_kernel(const uint16_t* __restrict__ x,
                                                                     int64_t n, uint32_t* word,
                                                                     uint8_t* __restrict__ q) {
  __shared__ uint32_t wave_max[kSmallThreads / 64];
  __shared__ float result;
  const int t = threadIdx.x;
  const int64_t nvec = n >> 3;
  uint32_t m = 0;
  int64_t i = t;
  for (; i + 3 * kSmallThreads < nvec; i += 4 * kSmallThreads) {   // four loads in flight per lane
    const U4 v0 = load16(x + (i << 3)), v1 = load16(x + ((i + kSmallThreads) << 3));
    const U4 v2 = load16(x + ((i + 2 * kSmallThreads) << 3)), v3 = load16(x + ((i + 3 * kSmallThreads) << 3));
    m = max(max(m, max(key8(v0), key8(v1))), max(key8(v2), key8(v3)));
  }
  for (; i < nvec; i += kSmallThreads) m = max(m, key8(load16(x + (i << 3))));
  for (int64_t j = (nvec << 3) + t; j < n; j += kSmallThreads) m = max(m, x[j] & 0x7fffu);
  m = max64(m);
  if ((t & 63) == 0) wave_max[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    uint32_t k = 0;
#pragma unroll
    for (int w = 0; w < kSmallThreads / 64; ++w) k = max(k, wave_max[w]);
    const float amax = amax_from_key<DT>(k);
    const float r = WANT_SCALE ? scale_from_amax(amax) : amax;
    result = r;
    *word = __float_as_uint(r);
  }
  if constexpr (WRITE_Q) {
    __syncthreads();
    const float scale = result;
    const bool fast = fast_scale(scale);
    const float r = 1.0f / scale;
    for (int64_t v = t; v < nvec; v += kSmallThreads)
      *reinterpret_cast<uint2*>(q + (v << 3)) = enc8<DT>(load16(x + (v << 3)), scale, r, fast);
    for (int64_t j = (nvec << 3) + t; j < n; j += kSmallThreads) q[j] = enc1<DT>(x[j], scale, r, fast);
  }
}

__global__ __launch_bounds__(kThreads) void debug_cast_kernel(const float* __restrict__ v, int64_t n,
                                                              uint8_t* __restrict__ q) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = tid; i < n; i += stride) q[i] = static_cast<uint8_t>(e4m3_encode(v[i]));
}

// Measurement reference with the quantizers' byte mix: q[i] = the high byte of the 16-bit
// element x[i] (2 bytes read, 1 written per element, no arithmetic).  Each lane moves 8
// elements per step (one 16-byte load, one 8-byte store), two steps in flight per wave,
// like the 1x128 group kernel; a scalar loop takes the last n % 512 elements.
__global__ __launch_bounds__(kThreads) void byte_mix_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                            uint8_t* __restrict__ q) {
  constexpr int kPer = 64 * 8;                               // elements per wave step
  const int64_t steps = n / kPer;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 6;
  const int64_t waves = (static_cast<int64_t>(gridDim.x) * kThreads) >> 6;
  const int lane = threadIdx.x & 63;
  auto high = [](uint32_t a, uint32_t b) {
    return (a >> 8 & 0xffu) | (a >> 16 & 0xff00u) | (b >> 8 & 0xffu) << 16 | (b >> 24) << 24;
  };
  for (int64_t i0 = wave; i0 < steps; i0 += 2 * waves) {
    U4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (i0 + u * waves < steps) v[u] = load16(x + (i0 + u * waves) * kPer + lane * 8);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (i0 + u * waves < steps)
        *reinterpret_cast<uint2*>(q + (i0 + u * waves) * kPer + lane * 8) =
            make_uint2(high(v[u].x, v[u].y), high(v[u].z, v[u].w));
  }
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (int64_t i = steps * kPer + tid; i < n; i += static_cast<int64_t>(gridDim.x) * kThreads)
    q[i] = static_cast<uint8_t>(x[i] >> 8);
}

inline unsigned grid_for(int64_t work_items, int64_t per_block, int64_t cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return static_cast<unsigned>(g);
}

constexpr int64_t kStreamCap = 256 * 16;     // 16 workgroups per CU on 256 CUs
constexpr int64_t kReduceCap = 256 * 4;      // whole-tensor reduction workgroups
constexpr int64_t kGroupCap = 256 * 256;     // group/block kernels loop beyond this grid

// 1x128 vector path: about sets_per_cu 16-lane sets per CU, each taking cg consecutive
// groups of one row.  Measured with cold inputs on A[4096, 7168] and A[4096, 4096]: 128
// sets per CU with two groups in flight per set led 64, 256 and 512 sets and 4 or 8 groups
// in flight, at 86-90% of a copy with the same byte mix and no arithmetic.
constexpr int kGroupUnroll = 2;
constexpr int64_t kGroupSetsPerCu = 128;

template <int DT, bool WRITE_Q, int UNROLL, bool E8M0 = false>
void launch_group_vec(const uint16_t* xp, int64_t rows, int64_t cols, int64_t sets_per_cu, uint8_t* q,
                      void* out, int64_t sstride, hipStream_t s) {
  const int64_t gcols = (cols + 127) / 128;
  const int64_t ngroups = rows * gcols;
  const int64_t target_sets = 256 * sets_per_cu;
  int64_t cg = (ngroups + target_sets - 1) / target_sets;
  cg = ((cg + UNROLL - 1) / UNROLL) * UNROLL;
  const int64_t nch = (gcols + cg - 1) / cg;
  const unsigned grid = grid_for(rows * nch, 16, kGroupCap);
  group_1x128_vec_kernel<DT, WRITE_Q, UNROLL, E8M0><<<grid, kThreads, 0, s>>>(xp, rows, cols, nch, cg, q, out, sstride);
}

template <int DT, bool E8M0>
void launch_groups_t(const void* x, int64_t rows, int64_t cols, int32_t group_rows, uint8_t* q,
                     void* out, bool write_q, int64_t sstride, hipStream_t s) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const bool vec = (cols % 8) == 0;
  if (group_rows == 1) {
    const int64_t gcols = (cols + 127) / 128;
    const int64_t ngroups = rows * gcols;
    if (cols % 128 == 0) {
      // 4096 elements per workgroup step, at most 32 workgroups per CU
      const unsigned grid = grid_for(ngroups * 128, kThreads * 16, 256 * 32);
      if (write_q) group_1x128_flat_kernel<DT, true, E8M0><<<grid, kThreads, 0, s>>>(xp, ngroups, gcols, q, out, sstride);
      else group_1x128_flat_kernel<DT, false><<<grid, kThreads, 0, s>>>(xp, ngroups, gcols, q, out, sstride);
    } else if (vec) {
      if (write_q) launch_group_vec<DT, true, kGroupUnroll, E8M0>(xp, rows, cols, kGroupSetsPerCu, q, out, sstride, s);
      else launch_group_vec<DT, false, kGroupUnroll>(xp, rows, cols, kGroupSetsPerCu, q, out, sstride, s);
    } else {
      const unsigned grid = grid_for(ngroups, 16, kGroupCap);
      if (write_q) group_1x128_scalar_kernel<DT, true, E8M0><<<grid, kThreads, 0, s>>>(xp, rows, cols, q, out, sstride);
      else group_1x128_scalar_kernel<DT, false><<<grid, kThreads, 0, s>>>(xp, rows, cols, q, out, sstride);
    }
  } else {
    const unsigned grid = grid_for(((rows + 127) / 128) * ((cols + 127) / 128), 1, kGroupCap);
    if (vec) {
      if (write_q) block_128x128_kernel<DT, true, true, E8M0><<<grid, kThreads, 0, s>>>(xp, rows, cols, q, out, sstride);
      else block_128x128_kernel<DT, false, true><<<grid, kThreads, 0, s>>>(xp, rows, cols, q, out, sstride);
    } else {
      if (write_q) block_128x128_kernel<DT, true, false, E8M0><<<grid, kThreads, 0, s>>>(xp, rows, cols, q, out, sstride);
      else block_128x128_kernel<DT, false, false><<<grid, kThreads, 0, s>>>(xp, rows, cols, q, out, sstride);
    }
  }
}

template <int DT>
void launch_tensor_amax_t(const void* x, int64_t n, float* amax, hipStream_t s) {
  uint32_t* w = reinterpret_cast<uint32_t*>(amax);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (n <= kSmallTensor) {                     // one workgroup, one launch
    tensor_small_kernel<DT, false, false><<<1, kSmallThreads, 0, s>>>(xp, n, w, nullptr);
    return;
  }
  init_word_kernel<<<1, 1, 0, s>>>(w);
  tensor_amax_kernel<<<grid_for(n, kThreads * 8 * 4, kReduceCap), kThreads, 0, s>>>(xp, n, w);
  finalize_word_kernel<DT><<<1, 1, 0, s>>>(w);
}

}  // namespace

namespace {

template <int DT>
void launch_rows_t(const void* xv, int64_t rows, int64_t cols, uint8_t* q, float* scales, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(xv);
  constexpr int64_t kRowsCap = 256 * 64;       // workgroups; the kernels loop over further rows
  if (cols % 8 != 0 || cols == 0) {           // (empty rows: scale 1, x and q never touched)
    rows_two_pass_kernel<DT, false><<<grid_for(rows, 1, kRowsCap), kThreads, 0, s>>>(x, rows, cols, q, scales);
    return;
  }
  const unsigned g_wave = grid_for(rows, kThreads / 64, kRowsCap);   // a row per wave
  const unsigned g_wg = grid_for(rows, 1, kRowsCap);                  // a row per workgroup
  // few rows (decode tokens): a workgroup per row, so that each row has four times the loads
  // in flight and no CU holds several of them
  if (rows <= 256 && cols > 512 && cols <= 16384) {
    if (cols <= 2048) rows_vec_kernel<DT, 4, 1><<<g_wg, kThreads, 0, s>>>(x, rows, cols, q, scales);
    else if (cols <= 4096) rows_vec_kernel<DT, 4, 2><<<g_wg, kThreads, 0, s>>>(x, rows, cols, q, scales);
    else if (cols <= 8192) rows_vec_kernel<DT, 4, 4><<<g_wg, kThreads, 0, s>>>(x, rows, cols, q, scales);
    else rows_vec_kernel<DT, 4, 8><<<g_wg, kThreads, 0, s>>>(x, rows, cols, q, scales);
    return;
  }
  if (cols <= 512) rows_vec_kernel<DT, 1, 1><<<g_wave, kThreads, 0, s>>>(x, rows, cols, q, scales);
  else if (cols <= 1024) rows_vec_kernel<DT, 1, 2><<<g_wave, kThreads, 0, s>>>(x, rows, cols, q, scales);
  else if (cols <= 2048) rows_vec_kernel<DT, 1, 4><<<g_wave, kThreads, 0, s>>>(x, rows, cols, q, scales);
  else if (cols <= 4096) rows_vec_kernel<DT, 1, 8><<<g_wave, kThreads, 0, s>>>(x, rows, cols, q, scales);
  else if (cols <= 8192) rows_vec_kernel<DT, 4, 4><<<g_wg, kThreads, 0, s>>>(x, rows, cols, q, scales);
  else if (cols <= 16384) rows_vec_kernel<DT, 4, 8><<<g_wg, kThreads, 0, s>>>(x, rows, cols, q, scales);
  else rows_two_pass_kernel<DT, true><<<g_wg, kThreads, 0, s>>>(x, rows, cols, q, scales);
}

}  // namespace

void launch_rows(int dt, const void* x, int64_t rows, int64_t cols, uint8_t* q, float* scales,
                 hipStream_t s) {
  if (dt == DT_BF16) launch_rows_t<DT_BF16>(x, rows, cols, q, scales, s);
  else launch_rows_t<DT_F16>(x, rows, cols, q, scales, s);
}

void launch_groups(int dt, const void* x, int64_t rows, int64_t cols, int32_t group_rows,
                   uint8_t* q, float* out, bool write_q, hipStream_t s) {
  const int64_t gc = (cols + 127) / 128;
  if (dt == DT_BF16) launch_groups_t<DT_BF16, false>(x, rows, cols, group_rows, q, out, write_q, gc, s);
  else launch_groups_t<DT_F16, false>(x, rows, cols, group_rows, q, out, write_q, gc, s);
}

void launch_groups_e8m0(int dt, const void* x, int64_t rows, int64_t cols, int32_t group_rows,
                        uint8_t* q, uint8_t* codes, hipStream_t s) {
  const int64_t row_bytes = e8m0_row_bytes((cols + 127) / 128);
  if (dt == DT_BF16) launch_groups_t<DT_BF16, true>(x, rows, cols, group_rows, q, codes, true, row_bytes, s);
  else launch_groups_t<DT_F16, true>(x, rows, cols, group_rows, q, codes, true, row_bytes, s);
}

void launch_tensor_amax(int dt, const void* x, int64_t n, float* amax, hipStream_t s) {
  if (dt == DT_BF16) launch_tensor_amax_t<DT_BF16>(x, n, amax, s);
  else launch_tensor_amax_t<DT_F16>(x, n, amax, s);
}

void launch_tensor_quantize(int dt, const void* x, int64_t n, float* scale, uint8_t* q,
                            hipStream_t s) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (n > kSmallTensor) {
    // every cast workgroup's first chunk lies wholly inside q
    const int chunks = static_cast<int>(std::min<int64_t>(kMaxCastBlocks, n / kCastChunk));
    const int partials = static_cast<int>(grid_for(n, int64_t{kPartialThreads} * 8, kMaxPartials));
    tensor_partial_kernel<<<partials, kPartialThreads, 0, s>>>(xp, n, chunks, q);
    if (dt == DT_BF16) tensor_cast_slots_kernel<DT_BF16><<<chunks, kCastThreads, 0, s>>>(xp, n, partials, q, scale);
    else tensor_cast_slots_kernel<DT_F16><<<chunks, kCastThreads, 0, s>>>(xp, n, partials, q, scale);
    return;
  }
  uint32_t* w = reinterpret_cast<uint32_t*>(scale);
  if (dt == DT_BF16) tensor_small_kernel<DT_BF16, true, true><<<1, kSmallThreads, 0, s>>>(xp, n, w, q);
  else tensor_small_kernel<DT_F16, true, true><<<1, kSmallThreads, 0, s>>>(xp, n, w, q);
}

void launch_tensor_static(int dt, const void* x, int64_t n, const float* scale, uint8_t* q,
                          uint32_t* amax_acc, hipStream_t s) {
  // 8192 elements per workgroup: a quarter of the atomics on the amax word (they serialize
  // on its one address) for the same loads in flight as the cast kernel
  const unsigned grid = grid_for(n, kThreads * 8 * 4, kStreamCap);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (dt == DT_BF16) {
    if (amax_acc) tensor_static_kernel<DT_BF16, true><<<grid, kThreads, 0, s>>>(xp, n, scale, q, amax_acc);
    else tensor_static_kernel<DT_BF16, false><<<grid, kThreads, 0, s>>>(xp, n, scale, q, nullptr);
  } else {
    if (amax_acc) tensor_static_kernel<DT_F16, true><<<grid, kThreads, 0, s>>>(xp, n, scale, q, amax_acc);
    else tensor_static_kernel<DT_F16, false><<<grid, kThreads, 0, s>>>(xp, n, scale, q, nullptr);
  }
}

void launch_delayed_update(float* history, int len, uint32_t* amax_acc, int* step, int interval,
                           int margin, float* scale, hipStream_t s) {
  delayed_update_kernel<<<1, 64, 0, s>>>(history, len, amax_acc, step, interval, margin, scale, nullptr);
}

void launch_delayed_quantize(int dt, const void* x, int64_t n, float* history, int len,
                             uint32_t* amax_acc, int* step, int interval, int margin, float* scale,
                             float* scale_used, uint8_t* q, hipStream_t s) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (n <= kSmallTensor) {
    if (dt == DT_BF16)
      delayed_small_kernel<DT_BF16><<<1, kSmallThreads, 0, s>>>(xp, n, history, len, amax_acc, step,
                                                               interval, margin, scale, scale_used, q);
    else
      delayed_small_kernel<DT_F16><<<1, kSmallThreads, 0, s>>>(xp, n, history, len, amax_acc, step,
                                                              interval, margin, scale, scale_used, q);
    return;
  }
  launch_tensor_static(dt, x, n, scale, q, amax_acc, s);
  delayed_update_kernel<<<1, 64, 0, s>>>(history, len, amax_acc, step, interval, margin, scale, scale_used);
}

void launch_byte_mix(const void* x, int64_t n, uint8_t* q, hipStream_t s) {
  const unsigned grid = grid_for(n, kThreads * 8, 256 * 32);      // up to 32 workgroups per CU
  byte_mix_kernel<<<grid, kThreads, 0, s>>>(static_cast<const uint16_t*>(x), n, q);
}

void launch_debug_cast(const float* v, int64_t n, uint8_t* q, hipStream_t s) {
  const unsigned grid = grid_for(n, kThreads, kStreamCap);
  debug_cast_kernel<<<grid, kThreads, 0, s>>>(v, n, q);
}

}  // namespace fp8amax
