// peaks.hip - measurement kernels for the benchmark (not part of the linear's
// ABI): the bf16 matrix-core rate of a back-to-back MFMA loop, the HBM read
// rate of a streaming read (of a large buffer, and of buffers the size of
// one small streaming call's weights), and the fixed cost of a launch, against
// which the kernels' achieved rates are also reported.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CHAINS = 8;   // independent accumulators per wave: one MFMA's latency hidden behind the others

// Every wave runs `iters` rounds of CHAINS independent 16x16x32 bf16 MFMAs
// (16384 flops each) on operands held in registers, then stores the sum of
// its accumulators so that nothing is optimised away.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int iters, uint32_t seed) {
  const int lane = threadIdx.x & 63;
  const uint32_t v = seed ^ (uint32_t)(lane * 0x9E3779B1u);
  // small bf16 values (exponent near 1) so the sums stay finite
  const uint32_t w = 0x3F803F80u | (v & 0x007F007Fu);
  const u32x4 ua = u32x4{w, w ^ 0x10001u, w ^ 0x20002u, w ^ 0x30003u};
  const u32x4 ub = u32x4{w ^ 0x40004u, w ^ 0x50005u, w ^ 0x60006u, w ^ 0x70007u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, ua);
  const bf16x8 b = __builtin_bit_cast(bf16x8, ub);
  f32x4 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  f32x4 s = acc[0];
#pragma unroll
  for (int c = 1; c < CHAINS; ++c) s += acc[c];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

// Grid-stride read of `n16` 16-byte pieces; each thread folds what it read
// into one word and stores it, so every load is needed.
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* src, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 x0 = u32x4{0u, 0u, 0u, 0u}, x1 = x0, x2 = x0, x3 = x0;
  int64_t i = t;
  for (; i + 3 * stride < n16; i += 4 * stride) {      // four loads in flight per thread
    x0 ^= src[i];
    x1 ^= src[i + stride];
    x2 ^= src[i + 2 * stride];
    x3 ^= src[i + 3 * stride];
  }
  for (; i < n16; i += stride) x0 ^= src[i];
  const u32x4 x = x0 ^ x1 ^ x2 ^ x3;
  out[t] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// Does nothing: back-to-back launches of it give the fixed cost of a launch.
__global__ __launch_bounds__(256) void empty_kernel() {}

}  // namespace

extern "C" {

// Launches `blocks` x 256 threads of a kernel that does nothing.
int q2peak_empty(int blocks, hipStream_t stream) {
  if (blocks <= 0) return -1;
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)blocks), dim3(256), 0, stream);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// Launches blocks x 256 threads of the MFMA loop; out must hold blocks * 256 floats.
// Flops of one launch: blocks * 4 waves * iters * CHAINS * 16384.
int q2peak_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters, 0x1234567u);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int q2peak_mfma_chains(void) { return CHAINS; }

// Reads `bytes` (a multiple of 16, 16-byte aligned) from src with blocks x 256
// threads; out must hold blocks * 256 words.
int q2peak_read(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return -1;
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
