/*
 * q2.h - C ABI of libq2: the Q2_0 ternary dequantize-and-multiply linear, its
 * rank-r side branch and the 4-bit nibble variant, as hand-written HIP kernels
 * for AMD CDNA4 (gfx950, MI355X).
 *
 * Format (We're Teaching Your Browser to Paint, aitherium.com, section "The
 * lucky break that wasn't luck"): a weight row of K inputs is cut into blocks
 * of 128; each block has 128 two-bit codes q in {0,1,2} and one f16 scale d;
 * the weight is (q - 1) * d.  Codes run along the input axis, four per byte,
 * least significant pair first: code k of a row is bits 2(k%4) and 2(k%4)+1
 * of byte k/4.  This library stores the codes and the scales as two arrays
 * (structure of arrays): packed u8 [N, K/4] and scales f16 [N, K/128], both
 * row-major.  A row is an independent byte run, so a row slice of a weight is
 * a plain pointer offset (same page, section "The GPU driver...").
 *
 * Conventions shared by every entry point:
 *  - Sizes are int64.  M, N, K, r >= 0; K must be a multiple of 128, and at
 *    most 2^24 for the linear entry points (Q2_ERR_SHAPE otherwise).  A call
 *    with M == 0 or N == 0 does nothing and returns Q2_OK; K == 0 writes
 *    zeros (an empty sum), or leaves y as it is under Q2_ACCUMULATE.
 *    Pointers to buffers of zero bytes may be NULL.
 *  - All array pointers are device pointers; all arrays are dense row-major.
 *    The caller owns every buffer and the library allocates no device memory.
 *    It keeps no state between calls except a per-device architecture check,
 *    the load-time error flags (see q2_pack) and the test control of
 *    q2_set_dispatch, and is safe to call from several host threads.
 *  - x, the packed codes, the q2_pack codes and the low-rank factor A must be
 *    16-byte aligned; every other array must be aligned to its element size;
 *    the low-rank workspace to 256 bytes.
 *  - bf16 activations and f16 scales / factors are passed as their uint16
 *    bit patterns.  Outputs are float32.
 *  - Every compute entry point is asynchronous on `stream` (0 = the null
 *    stream) and returns only argument, device or launch errors.  Arguments
 *    are checked before any HIP call, so argument errors are reported even on
 *    a host without a GPU.  q2_pack is the exception: it synchronizes on
 *    `stream` to report bad codes or scales.
 *  - Errors are negative q2_status values; nothing is thrown across the ABI.
 *    q2_strerror() names a status, q2_last_error() gives the calling thread's
 *    detail message for its most recent failed call.
 *  - Packed bytes holding the 2-bit value 3 are outside the format: q2_pack
 *    refuses to produce them, q2_dequant decodes them as (3 - 1) * d, and the
 *    products of q2_linear / q2_linear_lowrank treat them the same way.
 */
#ifndef Q2_H
#define Q2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  Q2_OK = 0,
  Q2_ERR_ARG = -1,       /* NULL pointer for a non-empty buffer, negative size      */
  Q2_ERR_SHAPE = -2,     /* K not a multiple of 128                                 */
  Q2_ERR_ALIGN = -3,     /* pointer not aligned as stated above                     */
  Q2_ERR_CODE = -4,      /* q2_pack: a code above 2                                 */
  Q2_ERR_SCALE = -5,     /* q2_pack: scale not exactly representable in f16, or NaN/inf */
  Q2_ERR_DEVICE = -6,    /* current device is not gfx950                            */
  Q2_ERR_HIP = -7,       /* HIP runtime or launch error                             */
  Q2_ERR_WORKSPACE = -8, /* low-rank workspace too small                            */
  Q2_ERR_FORMAT = -9     /* q2_import_gemlite: a zero point that is not -scale       */
} q2_status;

/*
 * q2_pack - load-time conversion to the Q2_0 layout.
 * Source: We're Teaching Your Browser to Paint (aitherium.com), section "The
 * lucky break that wasn't luck": the conversion changes no value; the only
 * rounding is the f32 -> f16 scale cast, which must round-trip exactly or the
 * conversion stops.
 *   codes      u8  [N, K], each in {0, 1, 2}                    (in)
 *   scales     f32 [N, K/128]                                   (in)
 *   packed     u8  [N, K/4]; byte j = c[4j] | c[4j+1]<<2 | c[4j+2]<<4 | c[4j+3]<<6   (out)
 *   scales_f16 u16 [N, K/128]: f16 bits of scales, nearest-even  (out)
 *   bad_index  host int64*, may be NULL: on Q2_ERR_CODE / Q2_ERR_SCALE, the
 *              flat row-major index of the first bad code / scale; -1 on success.
 * Codes are checked before scales.  Synchronizes `stream`.  Allocates
 * nothing: the error flags live in a small file-scope device array (one per
 * device), so q2_pack and q2_import_gemlite calls of one process run one at
 * a time (a host lock).  The outputs are fully written even when an error is
 * returned, but must not be used then.
 */
int q2_pack(const uint8_t* codes, const float* scales, int64_t N, int64_t K,
            uint8_t* packed, uint16_t* scales_f16, int64_t* bad_index, hipStream_t stream);

/*
 * q2_import_gemlite - load-time import of a transposed, group-quantised
 * ternary weight (the gemlite-int2 kind) into Q2_0, with no numeric change.
 * Source: We're Teaching Your Browser to Paint, section "The lucky break that
 * wasn't luck": the source's codes are {0,1,2}, four per byte, least
 * significant pair first, along the input axis; each group has a scale and a
 * zero point, and every zero equals minus its scale, so each weight is
 * (q - 1) * scale -- the Q2_0 formula.  The conversion is a transpose and a
 * regroup; the f32 -> f16 scale cast must be exact or it stops.  The layout
 * beyond that is this library's reading:
 *   codes_t    u8  [K/4, N]: byte j of column n holds codes 4j..4j+3 of
 *              weight row n (input-major)                             (in)
 *   scales_t   f32 [K/G, N]; zeros_t f32 [K/G, N]: weight = q * scale + zero  (in)
 *   G          group length: divides 128 or is a multiple of it, and divides
 *              K (Q2_ERR_SHAPE otherwise)
 *   packed     u8  [N, K/4], 16-byte aligned; scales_f16 u16 [N, K/128]  (out)
 *   bad_index  host int64*, may be NULL: the first bad flat index (weight
 *              index n * K + k for a code, group index g * N + n otherwise),
 *              -1 on success.
 * Checked, and reported in this order: a code 3 (Q2_ERR_CODE); a zero that
 * is not exactly -scale (Q2_ERR_FORMAT); a scale that is not a finite exact
 * f16 value, then a group whose scale differs from its block's first group
 * when G < 128 (Q2_ERR_SCALE).  Synchronizes `stream`; allocates nothing
 * and shares q2_pack's device flags and host lock.  The outputs must not be
 * used after an error.
 */
int q2_import_gemlite(const uint8_t* codes_t, const float* scales_t, const float* zeros_t,
                      int64_t N, int64_t K, int64_t G, uint8_t* packed, uint16_t* scales_f16,
                      int64_t* bad_index, hipStream_t stream);

/*
 * q2_linear - y = x W^T with W[n, k] = (q[n, k] - 1) * d[n, k/128].
 * Source: We're Teaching Your Browser to Paint, section "The lucky break that
 * wasn't luck" (format and formula) and section "The GPU driver..." (the
 * 2-bit matmul is the projection kernel of the image transformer).
 *   x_bf16     u16 [M, K] bf16 activations                      (in)
 *   packed     u8  [N, K/4] codes as produced by q2_pack          (in)
 *   scales_f16 u16 [N, K/128]                                   (in)
 *   y          f32 [M, N], overwritten                          (out)
 * Products are exact and accumulate in fp32; every call is run-to-run
 * bitwise deterministic.  M <= 16 runs a streaming GEMV kernel, larger M a
 * matrix-core GEMM.  Asynchronous.
 */
int q2_linear(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16,
              float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * q2_lowrank_workspace_bytes - device bytes q2_linear_lowrank needs for M
 * rows and rank r: M * r8 * 4 rounded up to a multiple of 256, with r8 = r
 * rounded up to a multiple of 8 (the bf16 hi and lo limbs of x A^T, padded
 * rows); 0 when M or r is 0.  Negative arguments, and M or r beyond what the
 * linear accepts (M > 2^46, r > 65535), give 0; a size beyond SIZE_MAX gives
 * SIZE_MAX.
 */
size_t q2_lowrank_workspace_bytes(int64_t M, int64_t r);

/*
 * q2_linear_lowrank - y = x W^T + (x A^T) B^T: the Q2_0 linear plus a rank-r
 * side branch.  Source: mindview-t2i-turbo model card, section "One step"
 * (the branch y = W x + B (A x) on the transformer's large matrices; ranks
 * 4, 32 and 64 appear there and in "Two and four steps").
 *   A_f16      u16 [r, K] f16                                   (in)
 *   B_f16      u16 [N, r] f16                                   (in)
 *   r          rank, 0 <= r <= 65535; r == 0 is exactly q2_linear
 *   workspace  device scratch of >= q2_lowrank_workspace_bytes(M, r) bytes,
 *              256-byte aligned, owned by the caller; overwritten.
 * x A^T is computed once per call (into the workspace) and B (x A^T) is
 * added inside the Q2_0 linear kernel, into the same accumulators as the
 * quantised product.  Asynchronous; calls that share a workspace must be
 * ordered on one stream.
 */
int q2_linear_lowrank(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16,
                      const uint16_t* A_f16, const uint16_t* B_f16, int64_t r,
                      float* y, int64_t M, int64_t N, int64_t K,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * q2_linear_lowrank_noalloc - q2_linear_lowrank without a workspace argument
 * and without any allocation, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The x A^T scratch lives in a file-scope device array of
 * Q2_NOALLOC_SCRATCH_BYTES (8 MiB) per device, held until the process ends:
 * calls with q2_lowrank_workspace_bytes(M, r) above that size are refused
 * with Q2_ERR_WORKSPACE.  The array's device address is looked up once per
 * device, at the first call made with that device current.  Every call on a
 * device shares that device's array and overwrites it entirely (nothing in it
 * needs to start at zero), so calls that overlap on one device -- on
 * different streams, or from different host threads without ordering -- race
 * and must not be issued; calls ordered on one stream are safe.  Every other
 * argument, the result (bit for bit) and the errors are those of
 * q2_linear_lowrank.  Asynchronous.
 */
#define Q2_NOALLOC_SCRATCH_BYTES 8388608u
int q2_linear_lowrank_noalloc(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16,
                              const uint16_t* A_f16, const uint16_t* B_f16, int64_t r,
                              float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Flags of q2_linear_ex. */
#define Q2_ACCUMULATE 0x1u  /* y += result: y is read, the result added in fp32 once */

/*
 * q2_linear_ex - q2_linear (r == 0) or q2_linear_lowrank (r > 0) with flags.
 * Source: We're Teaching Your Browser to Paint, section "The GPU driver, and
 * the bug that looked like broken math": the fused output projection takes
 * the concatenation of two activations along its input axis, and is computed
 * as two multiplies over the matching input slices of the weight (q2_slice),
 * whose results are summed.  With Q2_ACCUMULATE the second call adds into the
 * first call's y: each output becomes y_old + v in fp32, where v is exactly
 * the value the call would write without the flag (so the sum is run-to-run
 * deterministic).  For a low-rank weight, A is sliced along its input axis
 * the same way and B is shared: the two branch terms add up to the branch of
 * the whole input.
 *   flags  0 or Q2_ACCUMULATE; other bits give Q2_ERR_ARG.
 * Every other argument, the rules on A, B and the workspace (when r > 0)
 * and the errors are those of q2_linear_lowrank.  With Q2_ACCUMULATE, y must
 * not overlap any input.  Asynchronous.
 */
int q2_linear_ex(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16,
                 const uint16_t* A_f16, const uint16_t* B_f16, int64_t r,
                 float* y, int64_t M, int64_t N, int64_t K,
                 void* workspace, size_t workspace_bytes, uint32_t flags, hipStream_t stream);

/*
 * q2_slice - load-time slicing of a packed weight: rows [n0, n1) and inputs
 * [k0, k1) of a Q2_0 matrix of N rows and K inputs, copied into a dense
 * packed matrix of n1 - n0 rows and k1 - k0 inputs.
 * Source: We're Teaching Your Browser to Paint, section "The GPU driver, and
 * the bug that looked like broken math": a fused projection (one matrix for
 * Q, K, V and the MLP input) is cut into its logical row ranges once at load
 * time, since each row is an independent byte run; the fused output
 * projection is cut along its input axis.  Codes and scales are copied
 * unchanged, so the slice's weights equal W[n0:n1, k0:k1] exactly.
 *   packed, scales_f16   the source, as produced by q2_pack         (in)
 *   n0, n1               0 <= n0 <= n1 <= N, else Q2_ERR_ARG
 *   k0, k1               0 <= k0 <= k1 <= K, else Q2_ERR_ARG; multiples of
 *                        128 (whole blocks), else Q2_ERR_SHAPE
 *   out_packed  u8  [n1 - n0, (k1 - k0)/4], 16-byte aligned          (out)
 *   out_scales  u16 [n1 - n0, (k1 - k0)/128]                         (out)
 * A row range alone needs no copy: rows [n0, n1) of packed start at byte
 * n0 * K/4 and their scales at element n0 * K/128.  The outputs must not
 * overlap the source.  An empty range does nothing.  Asynchronous.
 */
int q2_slice(const uint8_t* packed, const uint16_t* scales_f16, int64_t N, int64_t K,
             int64_t n0, int64_t n1, int64_t k0, int64_t k1,
             uint8_t* out_packed, uint16_t* out_scales, hipStream_t stream);

/*
 * q2_a8_workspace_bytes - device bytes q2_linear_a8 needs for M rows of K
 * inputs: M * K rounded up to 256 (the int8 codes), plus M * 4 rounded up to
 * 256 (the row scales); 0 when M or K is 0 or negative.
 */
size_t q2_a8_workspace_bytes(int64_t M, int64_t K);

/*
 * q2_linear_a8 - the Q2_0 linear with 8-bit activations:
 * y[m, n] = s[m] * sum_k c[m, k] * W[n, k], where per row m, s[m] = max_k
 * |x[m, k]| / 127 and c[m, k] = round-half-even(x[m, k] / s[m]) clamped to
 * [-127, 127] (float32, IEEE division; a row of zeros has s = 0, c = 0).
 * Source: We're Teaching Your Browser to Paint, section "The GPU driver, and
 * the bug that looked like broken math" (the GPU path quantizes activations
 * to 8 bits, at a few-percent error floor); the per-row symmetric scheme and
 * its rounding are this library's reading.
 *   x_bf16, packed, scales_f16, y, M, N, K   as q2_linear (x finite)
 *   workspace  device scratch of >= q2_a8_workspace_bytes(M, K) bytes,
 *              256-byte aligned, owned by the caller.  After the call it holds
 *              the codes as int8 [M, K] at offset 0, each group of 16
 *              consecutive codes of a row stored as a transposed 4 x 4 byte
 *              matrix (byte 16 p + 4 j + i holds code 16 p + 4 i + j), and the
 *              scales f32 [M] at offset M * K rounded up to 256.
 * Each block's sum of code products, sum c[m, k] (q[n, k] - 1), is an integer
 * computed exactly on the int8 matrix cores; it is multiplied by the block
 * scale and accumulated in fp32, and the row scale is applied once per
 * output.  Asynchronous; calls that share a workspace must be ordered on one
 * stream.
 */
int q2_linear_a8(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16,
                 float* y, int64_t M, int64_t N, int64_t K,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * q4_linear - 4-bit variant: y = x W^T with W[n, k] = (q[n, k] - z[n, k/128]) * s[n, k/128],
 * q[n, k] = (packed4[n, k/2] >> (4 * (k & 1))) & 15 (the low nibble holds the even k).
 * Source: You Can Now Just Ask for an Image (aitherium.com), section "The bug
 * that hid in one flipped bit" (nibble order), and We're Teaching Your
 * Browser to Paint, section "What's left" ((q - zero) * scale).  The group
 * length 128 and the f16 zero point in code units are this library's reading.
 *   packed4    u8  [N, K/2]  (in);  scale_f16, zero_f16  u16 [N, K/128]  (in)
 *   y          f32 [M, N]    (out).   Asynchronous.
 */
int q4_linear(const uint16_t* x_bf16, const uint8_t* packed4, const uint16_t* scale_f16,
              const uint16_t* zero_f16, float* y, int64_t M, int64_t N, int64_t K,
              hipStream_t stream);

/*
 * q2_dequant - test export: w[n, k] = (q - 1) * d as float32 [N, K], exact;
 * a zero weight is written as +0.  Same layout rules as q2_linear.  Asynchronous.
 */
int q2_dequant(const uint8_t* packed, const uint16_t* scales_f16, float* w,
               int64_t N, int64_t K, hipStream_t stream);

/*
 * q2_set_dispatch - test and profiling control of the launch choice, for the
 * whole process; not needed for correct use.  path: NULL, "" or "auto"
 * (M <= 16 runs the GEMV, larger M the GEMM), "gemv" (the GEMV whenever
 * M <= 16) or "gemm" (always the GEMM).  tile: NULL or "" for the automatic
 * GEMM configuration, else a configuration name (w48x192, w96x192,
 * w64x128, w32x128, w32x64, kg2x1x4, kg4x2x2, kg2x1x2, kg2x2x4, kg2x2x2,
 * kg2x1x4r3, kg6x3x2), or an int8
 * configuration of q2_linear_a8 (a8_6x3x2, a8_4x2x2, a8_2x2x2, a8_2x1x4,
 * a8_1x2x4, a8_1x1x4, a8_8x3x2, a8_6x3x1r3, a8_4x4x2, a8_6x3x2r3, a8_4x2x4,
 * a8_6x2x2, a8_4x3x2), which leaves the bf16 entry points automatic and vice
 * versa; a forced configuration that cannot take a call's shape makes that
 * call fail with Q2_ERR_HIP.  path applies to the bf16 entry points only,
 * ksplit to both.  ksplit: 0 automatic, 1 the whole K in one workgroup, 2 the
 * K blocks in two parts (K-group and int8 configurations of non-accumulating
 * calls only, else Q2_ERR_HIP at the call).  An unknown name or value gives
 * Q2_ERR_ARG and changes nothing.
 * The environment variables Q2_FORCE_PATH, Q2_GEMM_TILE and Q2_GEMM_KSPLIT
 * (same values) are read once, at the first linear call, as the initial
 * setting.  Results never depend on it beyond fp32 summation order.
 */
int q2_set_dispatch(const char* path, const char* tile, int ksplit);

/* q2_strerror - static name of a status code; never NULL. */
const char* q2_strerror(int status);

/* q2_last_error - the calling thread's detail message for its last failed call
 * ("" if none).  Valid until that thread's next call into the library. */
const char* q2_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* Q2_H */
