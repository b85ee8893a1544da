// q2_internal.h - host-side launchers shared between the C ABI and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q2dev {

// One linear call: x [M, K] bf16, weights in format fmt (0 = Q2_0, 1 = 4-bit),
// y [M, N] fp32.  lr_t / lr_b / r describe an optional low-rank term the
// kernels add into their accumulators (lr_t = bf16 limbs [M, 2r] of x A^T,
// lr_b = B f16 [N, r]).
struct LinearArgs {
  const uint16_t* x;
  const uint8_t* w;
  const uint16_t* s;     // f16 scale per (row, block)
  const uint16_t* z;     // f16 zero point per (row, block), 4-bit only
  float* y;
  int64_t M, N, K;
  const uint16_t* lr_t;
  const uint16_t* lr_b;
  int r;
  int acc;               // 1: y += result (y is read), 0: y = result
};

// The Q2_0 linear over 8-bit activations: int8 codes [M, K] (each group of 16
// stored as a transposed 4 x 4 byte matrix, byte 4 j + i = element 4 i + j),
// row scales [M]; y [M, N] fp32 = row scale * (codes W^T).
struct A8Args {
  const uint8_t* xq;
  const uint8_t* w;
  const uint16_t* s;
  const float* row_scale;
  float* y;
  int64_t M, N, K;
};

// Path selection for tests: force_path 0 = automatic, 1 = force GEMV, 2 = force
// GEMM; force_cfg 0 = automatic GEMM configuration, else the number that
// gemm_config_id gives for a configuration name (-1 for an unknown name);
// force_ksplit 0 = automatic, 1 = whole K, 2 = K in two parts (K-group
// configurations without accumulation only).
hipError_t launch_linear(const LinearArgs& a, int fmt, int force_path, int force_cfg, int force_ksplit,
                         hipStream_t stream);
int gemm_config_id(const char* name);
hipError_t launch_quantize_rows_i8(const uint16_t* x, uint8_t* xq, float* row_scale, int64_t M, int64_t K,
                                   hipStream_t stream);
// force_cfg 0 = automatic, else the number a8_config_id gives for a name;
// force_ksplit as for launch_linear.
hipError_t launch_linear_a8(const A8Args& a, int force_cfg, int force_ksplit, hipStream_t stream);
int a8_config_id(const char* name);
// y[0 .. count) = 0 (before a K-split GEMM adds its parts into y).
hipError_t launch_zero_y(float* y, int64_t count, hipStream_t stream);
hipError_t launch_lowrank_t(const uint16_t* x, const uint16_t* A, uint16_t* t_limbs,
                            int64_t M, int64_t K, int r, hipStream_t stream);
// The current device's four 64-bit error flags for the load-time checks (a
// file-scope device array; the address is looked up once per device).
hipError_t check_flags(unsigned long long** flags);
hipError_t launch_pack(const uint8_t* codes, const float* scales, int64_t N, int64_t K,
                       uint8_t* packed, uint16_t* scales_f16, unsigned long long* flags,
                       hipStream_t stream);
hipError_t launch_dequant(const uint8_t* packed, const uint16_t* scales, float* w,
                          int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_import(const uint8_t* codes_t, const float* scales_t, const float* zeros_t, int64_t N, int64_t K,
                         int64_t G, uint8_t* packed, uint16_t* scales_f16, unsigned long long* flags,
                         hipStream_t stream);
hipError_t launch_slice(const uint8_t* packed, const uint16_t* scales, int64_t K, int64_t n0, int64_t rows,
                        int64_t k0, int64_t ks, uint8_t* out, uint16_t* out_scales, hipStream_t stream);

}  // namespace q2dev
