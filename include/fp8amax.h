/*
 * fp8amax.h - C ABI of the MI355X (gfx950) FP8 E4M3 amax / quantize / scaled-GEMM library.
 *
 * The operation, as the pages describe it:
 *   - "Что такое FP8 инференс на H100 (Transformer Engine)?", section 3 (steps 2-6 and
 *     the pseudocode): before each GEMM take the largest magnitude (amax) of each
 *     operand, scale = amax / 448 (448 is the largest E4M3 value), divide the operand
 *     by its scale and round to FP8, multiply the FP8 operands with a float32
 *     accumulator, and multiply the result by scale_A * scale_B before the 16-bit
 *     output.
 *   - "FP8 chi tiết" (Transformers fine-grained FP8 page), opening bullets: weights are
 *     quantized per 128x128 block and activations per token in groups of 128 input
 *     channels, so blockwise scales change every 128 input channels.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers owned by the caller (PyTorch tensors in
 *     practice).  The library allocates nothing and keeps no state between calls.
 *   - Tensors are dense and row-major: the last index is contiguous and the leading
 *     dimension equals the column count.  A is [M, K], B (weights) is [N, K] and the
 *     product is C = A @ B^T, [M, N].
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All work
 *     is enqueued on it and the call returns without waiting; device faults surface
 *     at the caller's next synchronisation.
 *   - Arguments are validated on the host before any HIP call.  A non-zero status
 *     means nothing was launched (except FP8_ERR_LAUNCH, which reports a failed
 *     launch); outputs are then unspecified.
 *   - Empty inputs (a zero dimension) are valid; see each entry point.
 *   - Data pointers (x, q, qa, qb, c) must be 16-byte aligned and float32 pointers
 *     (scales, amax) 4-byte aligned (FP8_ERR_MISALIGNED otherwise).
 *   - FP8 bytes are OCP "e4m3fn" codes: 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 *     largest finite 448, S.1111.111 = NaN, no infinities.
 *
 * Rules the pages leave open (the same in every entry point):
 *   - scale = amax / 448 is one IEEE float32 division (round to nearest even, subnormal
 *     results kept); an amax of 0 gives scale 1.0; NaN or inf propagate.
 *   - q = e4m3(x / scale): one IEEE float32 division per element, then round to
 *     nearest even with saturation at +-448 (inf included); NaN gives 0x7F; the sign
 *     of zero and of values that round to zero is kept.
 *   - amax propagates NaN (a NaN anywhere in a block makes that block's amax NaN);
 *     a NaN amax or scale is always the canonical quiet NaN 0x7FC00000.
 */
#ifndef FP8AMAX_H
#define FP8AMAX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are 32-bit integers on both sides of the ABI.  A C++ translation unit
 * gives them int32_t as fixed underlying type, so that any value a C caller passes (an
 * unknown dtype, say, which the checks then reject) is a valid value of the type there
 * too; C sees plain enums of the same size. */
#ifdef __cplusplus
#define FP8_ENUM_BASE : int32_t
#else
#define FP8_ENUM_BASE
#endif

typedef enum FP8_ENUM_BASE {
  FP8_OK = 0,
  FP8_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  FP8_ERR_BAD_SHAPE = 2,    /* negative size, unsupported group/block shape, K rule broken */
  FP8_ERR_BAD_DTYPE = 3,    /* unknown fp8_dtype_t value */
  FP8_ERR_MISALIGNED = 4,   /* a base pointer is not 16-byte aligned */
  FP8_ERR_LAUNCH = 5,       /* the HIP runtime reported an error for a launch */
  FP8_ERR_TOO_LARGE = 6     /* a size exceeds what the kernels index (elements >= 2^40) */
} fp8_status_t;

/* 16-bit floating point types used for inputs (activations, weights) and outputs. */
typedef enum FP8_ENUM_BASE { FP8_BF16 = 0, FP8_F16 = 1 } fp8_dtype_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* fp8_status_string(fp8_status_t s);

/*
 * fp8_amax - largest magnitude per tensor or per block (Transformer Engine page,
 * section 3 step 2; block shapes from "FP8 chi tiết", opening bullets).
 *   x      : [rows, cols] of `dt` (bf16 or fp16).
 *   block_rows, block_cols : (0, 0) for one value over the whole tensor;
 *            (1, 128) for per-token groups of 128 columns; (128, 128) for weight blocks.
 *   amax   : float32 output, [ceil(rows/block_rows), ceil(cols/block_cols)] row-major,
 *            or [1] for the whole tensor.  Blocks on a ragged edge cover only the
 *            elements that exist.  An empty tensor gives 0 (whole-tensor mode) or an
 *            empty grid (nothing written).
 * Errors: NULL x or amax (when there is anything to write), negative sizes, other
 * block shapes, misaligned pointers, unknown dtype.
 */
fp8_status_t fp8_amax(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                      int32_t block_rows, int32_t block_cols, float* amax, void* stream);

/*
 * fp8_quantize_per_tensor - one scale for the whole tensor (Transformer Engine page,
 * section 3 steps 2-4 and the pseudocode).
 *   x     : [rows, cols] of `dt`.
 *   q     : uint8 output [rows, cols], e4m3fn codes of x / scale.
 *   scale : float32 output [1], amax / 448 (1.0 for an all-zero or empty tensor).
 * Up to 32768 elements: one launch.  Above: two launches, the first of which leaves
 * partial maxima in q that the second reads and then overwrites with the codes; so x and
 * scale must not overlap q, and q holds no codes until the call has completed on `stream`.
 * Errors: as fp8_amax.
 */
fp8_status_t fp8_quantize_per_tensor(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                     uint8_t* q, float* scale, void* stream);

/*
 * fp8_quantize_per_token_group - blockwise scales with amax, scale and cast fused in
 * one pass over x ("FP8 chi tiết", opening bullets).
 *   group_rows, group_cols : (1, 128) per-token activation groups, or (128, 128)
 *            weight blocks.  Other shapes give FP8_ERR_BAD_SHAPE.
 *   x      : [rows, cols] of `dt`.
 *   q      : uint8 output [rows, cols].
 *   scales : float32 output [ceil(rows/group_rows), ceil(cols/group_cols)] row-major.
 * Errors: as fp8_amax.
 */
fp8_status_t fp8_quantize_per_token_group(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                          int32_t group_rows, int32_t group_cols,
                                          uint8_t* q, float* scales, void* stream);

/*
 * fp8_gemm_scaled_tensorwise - C = out( (sum_k qa[m,k] * qb[n,k]) * sa * sb )
 * (Transformer Engine page, section 3 steps 5-6 and the pseudocode).
 *   qa : uint8 e4m3fn [M, K];  sa : float32 [1] (device)
 *   qb : uint8 e4m3fn [N, K];  sb : float32 [1] (device)
 *   c  : [M, N] of out_dt (bf16 or fp16), rounded to nearest even.
 * Products are accumulated in float32 on the gfx950 FP8 matrix cores.
 * Requires K % 16 == 0 (the task page pads hidden sizes to a multiple of 16) and K > 0.
 * M == 0 or N == 0 returns FP8_OK with nothing launched.
 * Every GEMM entry point returns FP8_ERR_TOO_LARGE, before any HIP call, when M, N or K
 * exceeds 2^31 - 1 or one of M K, N K, M N exceeds 2^40.
 */
fp8_status_t fp8_gemm_scaled_tensorwise(const uint8_t* qa, const float* sa,
                                        const uint8_t* qb, const float* sb,
                                        int64_t M, int64_t N, int64_t K,
                                        void* c, fp8_dtype_t out_dt, void* stream);

/*
 * fp8_gemm_scaled_blockwise - per 128-wide K slab g:
 *   C = out( sum_g sa[m, g] * sb[n / 128, g] * (sum_{k in slab g} qa[m,k] * qb[n,k]) )
 * ("FP8 chi tiết", opening bullets: 1x128 activation groups, 128x128 weight blocks).
 *   qa : uint8 e4m3fn [M, K];  sa : float32 [M, K/128]
 *   qb : uint8 e4m3fn [N, K];  sb : float32 [ceil(N/128), K/128]
 *   c  : [M, N] of out_dt.
 * Each slab's partial sum is float32 and is scaled in registers before it is added.
 * Requires K % 128 == 0 and K > 0.  M == 0 or N == 0 returns FP8_OK.
 */
fp8_status_t fp8_gemm_scaled_blockwise(const uint8_t* qa, const float* sa,
                                       const uint8_t* qb, const float* sb,
                                       int64_t M, int64_t N, int64_t K,
                                       void* c, fp8_dtype_t out_dt, void* stream);

/*
 * fp8_quantize_per_token_group_ue8m0 - fp8_quantize_per_token_group with UE8M0 scales
 * ("FP8 chi tiết", the UE8M0 scale format section: scales kept as packed float8_e8m0fnu
 * bytes instead of float32).  A group's scale is the smallest power of two not below
 * amax/448, clamped to 2^-127 .. 2^127 (amax 0 -> 2^0; NaN or infinite amax -> NaN), stored
 * as one e8m0fnu byte b (value 2^(b - 127), b = 255 is NaN); q = e4m3(x / scale).
 *   scales : uint8 output [ceil(rows/group_rows), G4] row-major, where G4 is
 *            ceil(cols/group_cols) rounded up to a multiple of 4 (four scales per 32-bit
 *            word); the padding bytes at the end of each row are set to 127.
 * Other arguments and errors: as fp8_quantize_per_token_group (scales need 4-byte
 * alignment).
 */
fp8_status_t fp8_quantize_per_token_group_ue8m0(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                                int32_t group_rows, int32_t group_cols,
                                                uint8_t* q, uint8_t* scales, void* stream);

/*
 * fp8_gemm_scaled_blockwise_ue8m0 - fp8_gemm_scaled_blockwise with UE8M0 scales (same
 * section): per 128-wide K slab g,
 *   C = out( sum_g 2^(sa[m,g] - 127) * 2^(sb[n/128,g] - 127) * (sum_{k in slab g} qa[m,k] * qb[n,k]) )
 *   sa : uint8 e8m0fnu [M, G4];  sb : uint8 e8m0fnu [ceil(N/128), G4], with G4 = K/128
 *        rounded up to a multiple of 4, the layout fp8_quantize_per_token_group_ue8m0
 *        writes (the padding bytes are read with their word and ignored).
 * The scales are applied inside the gfx950 scaled FP8 MFMA, so each slab's product is
 * added to the float32 accumulator directly.  A scale byte of 255 makes the affected
 * outputs NaN.  Requires K % 128 == 0 and K > 0; M == 0 or N == 0 returns FP8_OK.
 * qa, qb and c need 16-byte alignment, sa and sb 4-byte alignment.
 */
fp8_status_t fp8_gemm_scaled_blockwise_ue8m0(const uint8_t* qa, const uint8_t* sa,
                                             const uint8_t* qb, const uint8_t* sb,
                                             int64_t M, int64_t N, int64_t K,
                                             void* c, fp8_dtype_t out_dt, void* stream);

/*
 * fp8_quantize_rowwise - per-channel scaling (Transformer Engine page, section 5: a scale
 * per channel for the weights, beside per-tensor scaling; each scale as in section 3
 * steps 2-4): one float32 scale per row,
 *   scales[r] = amax(|x[r, :]|) / 448 (amax 0 -> 1.0, NaN -> NaN),
 *   q[r, c]   = e4m3(x[r, c] / scales[r]), saturating round-to-nearest-even.
 * For a weight W[N, K] a row is an output channel; for activations A[M, K] a row is a
 * token (the per-token scales of fp8_gemm_scaled_rowwise).
 *   x      : bf16/fp16 [rows, cols] row-major (device), 16-byte aligned.
 *   q      : uint8 output [rows, cols] (device), 16-byte aligned; may be NULL when cols == 0.
 *   scales : float32 output [rows] (device), 4-byte aligned.
 * Errors: FP8_ERR_BAD_SHAPE (negative sizes), FP8_ERR_TOO_LARGE, FP8_ERR_BAD_DTYPE,
 * FP8_ERR_NULL_POINTER, FP8_ERR_MISALIGNED, FP8_ERR_LAUNCH.  rows == 0 returns FP8_OK.
 */
fp8_status_t fp8_quantize_rowwise(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols, uint8_t* q,
                                  float* scales, void* stream);

/*
 * fp8_gemm_scaled_rowwise - C = A @ B^T with one scale per token and per output channel
 * (the per-channel scaling of the Transformer Engine page, section 5; product and scales as
 * in its section 3 steps 5-6):
 *   C[m, n] = out( sa[m] * sb[n] * sum_k qa[m, k] * qb[n, k] ), float32 accumulation.
 *   sa : float32 [M] (device), e.g. from fp8_quantize_rowwise on A; a single per-tensor
 *        activation scale is the case of M equal entries.
 *   sb : float32 [N] (device), e.g. from fp8_quantize_rowwise on W.
 * Other arguments, layout and errors: as fp8_gemm_scaled_tensorwise (K % 16 == 0).
 */
fp8_status_t fp8_gemm_scaled_rowwise(const uint8_t* qa, const float* sa, const uint8_t* qb,
                                     const float* sb, int64_t M, int64_t N, int64_t K, void* c,
                                     fp8_dtype_t out_dt, void* stream);

/*
 * fp8_gemm_grouped_blockwise - the mixture-of-experts product of the fine-grained FP8 page
 * (its section on MoE experts: grouped_mm / batched_mm with float32 scales; the block
 * scaling of its opening bullets): E experts, each with its own weight, and the routed
 * tokens already permuted into one contiguous segment per expert.  For every expert e and
 * every row t in [offsets[e], offsets[e + 1]):
 *   C[t, n] = out( sum_g sa[t, g] * sb[e, n / 128, g] * sum_{k in slab g} qa[t, k] * qb[e, n, k] )
 *   qa      : uint8 e4m3 [T, K] (device), the permuted activations (a token sent to k experts
 *             appears k times), e.g. from fp8_quantize_per_token_group (1 x 128).
 *   sa      : float32 [T, K/128] (device).
 *   qb      : uint8 e4m3 [E, N, K] (device), the experts' weights, each row-major [N, K].
 *   sb      : float32 [E, ceil(N/128), K/128] (device), each expert's 128 x 128 block scales.
 *   offsets : int32 [E + 1] (device), non-decreasing, offsets[0] = 0, offsets[E] = T.  They
 *             stay on the device (no host synchronisation; the call can be captured in a HIP
 *             graph).  Values outside [0, T] are clamped and an expert whose end precedes its
 *             start is empty, so any offsets give in-bounds accesses; rows of C that no
 *             segment covers are not written, rows covered twice get either result.
 *   c       : bf16/fp16 output [T, N] (device), 16-byte aligned.
 * Requires E >= 1 (at most 65536), K % 128 == 0 and K > 0; T == 0 or N == 0 returns FP8_OK.
 * qa, qb and c need 16-byte alignment, sa, sb and offsets 4-byte alignment.  Errors:
 * FP8_ERR_BAD_SHAPE, FP8_ERR_TOO_LARGE, FP8_ERR_BAD_DTYPE, FP8_ERR_NULL_POINTER,
 * FP8_ERR_MISALIGNED, FP8_ERR_LAUNCH.
 */
fp8_status_t fp8_gemm_grouped_blockwise(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                                       const int32_t* offsets, int64_t E, int64_t T, int64_t N, int64_t K,
                                       void* c, fp8_dtype_t out_dt, void* stream);

/*
 * fp8_gemm_grouped_blockwise_ue8m0 - fp8_gemm_grouped_blockwise with UE8M0 scales (the same
 * page: the newest DeepGEMM expert kernels take only e8m0fnu scale bytes):
 *   sa : uint8 e8m0fnu [T, G4];  sb : uint8 e8m0fnu [E, ceil(N/128), G4], G4 = K/128 rounded
 *        up to a multiple of 4 (the layout fp8_quantize_per_token_group_ue8m0 writes).
 * Everything else as fp8_gemm_grouped_blockwise.
 */
fp8_status_t fp8_gemm_grouped_blockwise_ue8m0(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb,
                                             const uint8_t* sb, const int32_t* offsets, int64_t E, int64_t T,
                                             int64_t N, int64_t K, void* c, fp8_dtype_t out_dt, void* stream);

/*
 * fp8_quantize_static - static scaling (the task page's FP8 recipe and calibration step: a
 * scale fixed before the pass instead of this tensor's amax): q = e4m3(x / *scale) in one
 * pass, saturating to +-448 where |x| > 448 * scale.
 *   scale    : float32 [1] (device), e.g. from calibration or from
 *              fp8_delayed_scaling_update; finite and > 0 (not checked on the device).
 *   amax_acc : NULL, or a uint32 (device) that receives max(current, float bits of this
 *              tensor's amax) by atomic max (float bits of non-negative values, inf and
 *              the canonical NaN 0x7FC00000 order as integers), for delayed scaling.
 *   x, q     : as fp8_quantize_per_tensor.
 * Errors: as fp8_quantize_per_tensor; rows * cols == 0 returns FP8_OK with nothing launched.
 */
fp8_status_t fp8_quantize_static(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                 const float* scale, uint8_t* q, uint32_t* amax_acc, void* stream);

/*
 * fp8_delayed_scaling_update - one step of delayed scaling (the task page's DelayedScaling
 * recipe: margin, interval), on device-resident state so that it can be captured in a
 * HIP graph:
 *   the amax recorded in *amax_acc since the last update is stored in the ring
 *   history[*step % len] and *amax_acc is cleared; *step is incremented; when the new *step
 *   is a multiple of `interval`, *scale = max(history) * 2^margin / 448 in float32 (an
 *   all-zero window gives 1, a NaN in the window gives NaN); otherwise *scale is unchanged.
 *   history  : float32 [len] (device), the last len amaxes; the most recent is at
 *              (*step - 1) % len.  Zero-fill it, *amax_acc and *step before the first step.
 *   amax_acc : uint32 (device), as written by fp8_quantize_static.
 *   step     : int32 (device), steps so far.
 *   scale    : float32 [1] (device), the scale fp8_quantize_static uses.
 * Requires len >= 1, interval >= 1, -126 <= margin <= 126 (else FP8_ERR_BAD_SHAPE); all
 * pointers non-NULL and 4-byte aligned.  Calls on one state must be ordered (one stream).
 */
fp8_status_t fp8_delayed_scaling_update(float* history, int32_t len, uint32_t* amax_acc, int32_t* step,
                                        int32_t interval, int32_t margin, float* scale, void* stream);

/*
 * fp8_quantize_delayed - one delayed-scaling step of one tensor in one call (the task
 * page's DelayedScaling recipe): exactly fp8_quantize_static(x, scale, q, amax_acc)
 * followed by fp8_delayed_scaling_update(history, len, amax_acc, step, interval, margin,
 * scale), and in addition
 *   scale_used : float32 [1] (device) output, the scale q was made with (the value *scale
 *                had on entry): the one the GEMM that consumes q must apply, since *scale
 *                may already hold the next step's scale when the call returns.
 * One launch for up to 32768 elements, two (the cast, then the update) above.
 * history, amax_acc, step, scale, interval, margin: as fp8_delayed_scaling_update (amax_acc
 * may hold amaxes recorded by fp8_quantize_static since the last update; they are folded
 * in).  x, q: as fp8_quantize_per_tensor; rows * cols == 0 is allowed (x and q may then be
 * NULL) and still performs the update with this tensor's amax taken as 0.
 * Errors: those of the two calls it replaces.  Calls on one state must be ordered.
 */
fp8_status_t fp8_quantize_delayed(const void* x, fp8_dtype_t dt, int64_t rows, int64_t cols,
                                  float* history, int32_t len, uint32_t* amax_acc, int32_t* step,
                                  int32_t interval, int32_t margin, float* scale, float* scale_used,
                                  uint8_t* q, void* stream);

/*
 * fp8_debug_cast_f32 - test hook: q[i] = e4m3(v[i]) with the same device encoder the
 * quantizers use (saturating round to nearest even; NaN -> 0x7F).  v is float32 [n],
 * q is uint8 [n].  n == 0 returns FP8_OK.
 */
fp8_status_t fp8_debug_cast_f32(const float* v, uint8_t* q, int64_t n, void* stream);

/*
 * fp8_debug_byte_mix - measurement reference, no part of the method: q[i] = the high byte
 * of the 16-bit element x[i], for n elements.  It moves the same bytes as a quantizer
 * (2 read, 1 written per element) with the same access pattern and no arithmetic, so its
 * rate is the ceiling a quantize pass can approach on the device.  x is [n] 16-bit, q is
 * uint8 [n], both 16-byte aligned, device memory owned by the caller; asynchronous on
 * `stream`.  Errors: FP8_ERR_BAD_SHAPE for n < 0, FP8_ERR_TOO_LARGE, FP8_ERR_NULL_POINTER,
 * FP8_ERR_MISALIGNED, all before any HIP call; n == 0 returns FP8_OK.
 */
fp8_status_t fp8_debug_byte_mix(const void* x, uint8_t* q, int64_t n, void* stream);

/*
 * fp8_debug_gemm_plan - test hook: the kernel launches a scaled GEMM of this shape makes,
 * computed by the same host code that the GEMM entry points run, without touching a GPU.
 *   mode  : which GEMM (fp8_scale_mode_t below); M, N, K as in that entry point.
 *   plan  : host pointer, filled on FP8_OK; plan->launches is 0 when M or N is 0.
 * Each launch names its kernel, the output tile of one workgroup, the grid, the columns
 * of C it writes, and two figures of its 32-bit buffer addressing: max_range, the largest
 * byte range any of its buffer descriptors covers, and max_offset, the largest exclusive
 * end of any byte offset it forms for a load of an element of one of its tiles (rows and
 * columns past the operand's end included).  The kernels compute both in 32-bit signed
 * arithmetic, so the dispatcher keeps them below 2^31.
 * Errors: the shape errors of the GEMM entry point (FP8_ERR_BAD_SHAPE,
 * FP8_ERR_TOO_LARGE) for that mode, FP8_ERR_BAD_SHAPE for an unknown mode, and
 * FP8_ERR_NULL_POINTER for plan == NULL.
 */
typedef enum FP8_ENUM_BASE {
  FP8_SCALE_TENSOR = 0,      /* fp8_gemm_scaled_tensorwise */
  FP8_SCALE_BLOCK = 1,       /* fp8_gemm_scaled_blockwise */
  FP8_SCALE_BLOCK_UE8M0 = 2, /* fp8_gemm_scaled_blockwise_ue8m0 */
  FP8_SCALE_ROW = 3          /* fp8_gemm_scaled_rowwise */
} fp8_scale_mode_t;

typedef enum FP8_ENUM_BASE {
  FP8_KERNEL_GEMV_STREAM = 1, /* one token, float32 block scales: persistent waves, one
                                 weight row per wave at a time */
  FP8_KERNEL_GEMV_VALU = 2,   /* one token: one weight row per wave on the vector ALUs */
  FP8_KERNEL_GEMV_MFMA = 3,   /* 2-16 tokens on the matrix cores */
  FP8_KERNEL_SKINNY = 4,      /* 17-128 tokens: weights streamed to registers, tokens in LDS */
  FP8_KERNEL_TILE = 5,        /* tiled LDS-DMA kernel */
  FP8_KERNEL_STAGED = 6       /* register-staged tiles with a zero-filled K tail */
} fp8_gemm_kernel_t;

typedef struct {
  int32_t kernel;      /* fp8_gemm_kernel_t */
  int32_t tile_m;      /* rows of C one workgroup covers (GEMV and SKINNY: all M rows) */
  int32_t tile_n;      /* columns of C one workgroup covers per pass */
  int32_t variant;     /* GEMV_STREAM: 1 KB chunks per row; GEMV_VALU: 1 KB loads in flight
                          per wave; GEMV_MFMA: 16-row weight blocks per wave; SKINNY: 16-token
                          blocks; TILE and STAGED: pipeline stages */
  int32_t waves;       /* waves per workgroup (SKINNY: the compute waves, plus one loader) */
  int32_t paired;      /* TILE: 1 if one wave of each SIMD pair issues the DMA for both */
  int64_t grid;        /* workgroups launched */
  int64_t threads;     /* threads per workgroup */
  int64_t n_begin;     /* first column of C the launch writes */
  int64_t n_end;       /* one past its last column */
  int64_t max_range;   /* bytes */
  int64_t max_offset;  /* bytes */
} fp8_gemm_launch_t;

typedef struct {
  int32_t launches;    /* 0, 1 or 2, in the order they are enqueued */
  int32_t reserved;
  fp8_gemm_launch_t launch[2];
} fp8_gemm_plan_t;

fp8_status_t fp8_debug_gemm_plan(int32_t mode, int64_t M, int64_t N, int64_t K, fp8_gemm_plan_t* plan);

/*
 * fp8_gemv_dynamic - the whole step for one token, the batch-1 decode case: the interface
 * of the Transformer Engine page's section 3 pseudocode (fp8_gemm takes the 16-bit operand,
 * takes its amax, scales, casts, multiplies and rescales inside), with the weights already
 * quantized, and with the dynamic activation scheme of the fine-grained FP8 page
 * (activation_scheme "dynamic": the activation scales are taken from each call's input).
 * The activation row x is quantized with the scheme that pairs with `mode`:
 *   FP8_SCALE_TENSOR      : one scale, sa float32 [1] (fp8_quantize_per_tensor of x as [1, K]);
 *   FP8_SCALE_ROW         : the row's scale, sa float32 [1] (fp8_quantize_rowwise of x as [1, K]);
 *   FP8_SCALE_BLOCK       : 1 x 128 groups, sa float32 [K/128] (fp8_quantize_per_token_group);
 *   FP8_SCALE_BLOCK_UE8M0 : 1 x 128 groups, sa uint8 e8m0fnu [G4], G4 = K/128 rounded up to a
 *                           multiple of 4, padding bytes 127 (fp8_quantize_per_token_group_ue8m0);
 * and its codes qa [K] and scales sa are written bit for bit as that quantizer writes them.
 * Then c [N] = the GEMM of `mode` with M = 1: fp8_gemm_scaled_tensorwise, _rowwise,
 * _blockwise or _blockwise_ue8m0 of (qa, sa) with (qb, sb), bit for bit (where an output is
 * NaN, both are NaN; sign and payload of an output NaN are not specified).
 *   mode : fp8_scale_mode_t.
 *   x    : bf16/fp16 [K] (device), 16-byte aligned, of `in_dt`.
 *   qb   : uint8 e4m3 [N, K] (device), 16-byte aligned; sb as the GEMM of `mode` takes it
 *          (float32 [1], [N] or [ceil(N/128), K/128]; UE8M0 bytes [ceil(N/128), G4]).
 *   qa   : uint8 output [K] (device), 16-byte aligned; sa: output as above, 4-byte aligned.
 *   c    : bf16/fp16 output [N] of `out_dt` (device), 16-byte aligned.
 * Requires K > 0 and K % 16 == 0 (K % 128 == 0 for the block modes).  With N >= 1, K <= 8192
 * and N * K < 2^31 all of it is one launch; otherwise the quantizer's launches and then the
 * GEMM's, with the same results.  N == 0 quantizes x only (c may be NULL).  x must not share
 * memory with qa, sa or c.  Errors: FP8_ERR_BAD_SHAPE (an unknown mode, K rule, negative N),
 * FP8_ERR_TOO_LARGE, FP8_ERR_BAD_DTYPE, FP8_ERR_NULL_POINTER, FP8_ERR_MISALIGNED, FP8_ERR_LAUNCH.
 */
fp8_status_t fp8_gemv_dynamic(int32_t mode, const void* x, fp8_dtype_t in_dt, const uint8_t* qb, const void* sb,
                              int64_t N, int64_t K, uint8_t* qa, void* sa, void* c, fp8_dtype_t out_dt,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8AMAX_H */
