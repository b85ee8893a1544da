// q2_pack.hip - load-time Q2_0 packing with validation, import of a
// transposed group-quantised ternary weight, slicing of packed weights, and
// the exact decode used by tests.
//
// Packing follows the Q2_0 layout of "We're Teaching Your Browser to Paint"
// (aitherium.com), section "The lucky break that wasn't luck": four 2-bit
// codes per byte along the input axis, the first code in the two least
// significant bits; one f16 scale per 128 weights.  The only rounding allowed
// is the f32 -> f16 scale cast and it must round-trip exactly.  Bad inputs are
// reported through two 64-bit device flags that hold the smallest offending
// flat index (atomicMin, so the reported index is independent of scheduling).
#include <mutex>

#include "q2_device.h"
#include "q2_internal.h"

namespace q2dev {

// The error flags of q2_pack (two) and q2_import_gemlite (four), one set per
// device in a file-scope array, so neither call allocates.  Both calls reset
// the flags, wait for their kernels and read the flags back under one host
// lock, so they never overlap on a device.
static __device__ __align__(16) unsigned long long g_check_flags[4];

hipError_t check_flags(unsigned long long** flags) {
  static std::mutex lock;
  static unsigned long long* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(lock);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_check_flags));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<unsigned long long*>(p);
  }
  *flags = addr[dev];
  return hipSuccess;
}

// One thread per 16 codes (16 bytes in, one packed dword out).
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* codes, uint32_t* packed, int64_t n16,
                                                         unsigned long long* flags) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const q2_u32x4 v = reinterpret_cast<const q2_u32x4*>(codes)[i];
    uint32_t out = 0;
    int first_bad = -1;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t code = (v[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      if (code > 2u && first_bad < 0) first_bad = k;
      out |= (code & 3u) << (2 * k);
    }
    packed[i] = out;
    if (first_bad >= 0) atomicMin(&flags[0], (unsigned long long)(16 * i + first_bad));
  }
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const float* s, uint16_t* sh, int64_t count,
                                                          unsigned long long* flags) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    const float f = s[i];
    const _Float16 h = (_Float16)f;                 // round to nearest even
    sh[i] = __builtin_bit_cast(uint16_t, h);
    const bool finite = __builtin_isfinite(f);
    if (!finite || (float)h != f) atomicMin(&flags[1], (unsigned long long)i);
  }
}

// One thread per 16 weights.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* packed, const uint16_t* s, float* w,
                                                     int64_t N, int64_t K) {
  const int64_t per_row = K / 16;
  const int64_t total = N * per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / per_row;
    const int64_t k0 = (i - row * per_row) * 16;
    const uint32_t word = *reinterpret_cast<const uint32_t*>(packed + row * (K / 4) + k0 / 4);
    const float d = f16_to_f32(s[row * (K / BLOCK_K) + k0 / BLOCK_K]);
    float* out = w + row * K + k0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int q = (int)((word >> (2 * k)) & 3u);
      out[k] = (q == 1) ? 0.0f : (float)(q - 1) * d;
    }
  }
}

// Rows [n0, n0 + rows) and input columns [k0, k0 + ks) of a packed matrix
// with K inputs per row (K, k0 and ks multiples of 128) into a dense packed
// matrix of ks inputs per row.  Rows are independent byte runs and a block's
// codes are 32 whole bytes, so this is a plain copy: one thread per 16 code
// bytes (the source and destination offsets are multiples of 16), then one
// per scale.
__global__ __launch_bounds__(256) void slice_kernel(const uint8_t* packed, const uint16_t* s, int64_t K,
                                                    int64_t n0, int64_t rows, int64_t k0, int64_t ks,
                                                    uint8_t* out, uint16_t* out_s) {
  const int64_t chunks = ks / 64;                 // 16-byte pieces per output row
  const int64_t nb = ks / BLOCK_K;                // scales per output row
  const int64_t code_work = rows * chunks;
  const int64_t total = code_work + rows * nb;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    if (i < code_work) {
      const int64_t row = i / chunks, c = i - row * chunks;
      const q2_u32x4 v = *reinterpret_cast<const q2_u32x4*>(packed + (n0 + row) * (K / 4) + k0 / 4 + 16 * c);
      *reinterpret_cast<q2_u32x4*>(out + row * (ks / 4) + 16 * c) = v;
    } else {
      const int64_t j = i - code_work, row = j / nb, b = j - row * nb;
      out_s[row * nb + b] = s[(n0 + row) * (K / BLOCK_K) + k0 / BLOCK_K + b];
    }
  }
}

// Import of a transposed group-quantised ternary weight (source bytes
// [K/4, N], input-major; f32 scales and zeros [K/G, N]).  Its code bytes
// already hold four codes each in the Q2_0 order, so the codes are a byte
// transpose; one thread per source byte (reads coalesced along N).  A code 3
// is flagged with the flat index n * K + k of the weight.
__global__ __launch_bounds__(256) void import_codes_kernel(const uint8_t* src, uint8_t* packed, int64_t N,
                                                           int64_t K, unsigned long long* flags) {
  const int64_t total = N * (K / 4);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t j = i / N, n = i - j * N;
    const uint32_t b = src[i];
    packed[n * (K / 4) + j] = (uint8_t)b;
    const uint32_t three = b & (b >> 1) & 0x55u;          // bit 2p set where code p is 3
    if (three) atomicMin(&flags[0], (unsigned long long)(n * K + 4 * j + (__builtin_ctz(three) >> 1)));
  }
}

// One thread per (block b, row n), along N: the groups that cover block b are
// checked (zero == -scale, flag 1; finite exact f16 scale, flag 2; the same
// scale as the block's first group, flag 3, indices g * N + n) and the block's
// scale is written as f16.
__global__ __launch_bounds__(256) void import_scales_kernel(const float* st, const float* zt, uint16_t* sh,
                                                            int64_t N, int64_t K, int64_t G,
                                                            unsigned long long* flags) {
  const int64_t KB = K / BLOCK_K;
  const int64_t total = N * KB;
  const int64_t per = G < BLOCK_K ? BLOCK_K / G : 1;     // groups per block
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t b = i / N, n = i - b * N;
    const int64_t g0 = G < BLOCK_K ? b * per : b * BLOCK_K / G;
    const float s0 = st[g0 * N + n];
    for (int64_t q = 0; q < per; ++q) {
      const int64_t idx = (g0 + q) * N + n;
      const float sv = st[idx], zv = zt[idx];
      if (!(zv == -sv)) atomicMin(&flags[1], (unsigned long long)idx);
      const _Float16 h = (_Float16)sv;
      if (!__builtin_isfinite(sv) || (float)h != sv) atomicMin(&flags[2], (unsigned long long)idx);
      if (sv != s0) atomicMin(&flags[3], (unsigned long long)idx);
    }
    sh[n * KB + b] = __builtin_bit_cast(uint16_t, (_Float16)s0);
  }
}

static unsigned grid_for(int64_t work) {
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

hipError_t launch_pack(const uint8_t* codes, const float* scales, int64_t N, int64_t K, uint8_t* packed,
                       uint16_t* scales_f16, unsigned long long* flags, hipStream_t stream) {
  const int64_t n16 = N * K / 16;
  const int64_t ns = N * (K / BLOCK_K);
  hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for(n16)), dim3(256), 0, stream, codes,
                     reinterpret_cast<uint32_t*>(packed), n16, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(ns)), dim3(256), 0, stream, scales, scales_f16, ns, flags);
  return hipGetLastError();
}

hipError_t launch_import(const uint8_t* codes_t, const float* scales_t, const float* zeros_t, int64_t N, int64_t K,
                         int64_t G, uint8_t* packed, uint16_t* scales_f16, unsigned long long* flags,
                         hipStream_t stream) {
  hipLaunchKernelGGL(import_codes_kernel, dim3(grid_for(N * (K / 4))), dim3(256), 0, stream, codes_t, packed, N, K,
                     flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(import_scales_kernel, dim3(grid_for(N * (K / BLOCK_K))), dim3(256), 0, stream, scales_t,
                     zeros_t, scales_f16, N, K, G, flags);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* packed, const uint16_t* scales, float* w, int64_t N, int64_t K,
                          hipStream_t stream) {
  hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(N * K / 16)), dim3(256), 0, stream, packed, scales, w, N, K);
  return hipGetLastError();
}

hipError_t launch_slice(const uint8_t* packed, const uint16_t* scales, int64_t K, int64_t n0, int64_t rows,
                        int64_t k0, int64_t ks, uint8_t* out, uint16_t* out_scales, hipStream_t stream) {
  const int64_t work = rows * (ks / 64 + ks / BLOCK_K);
  hipLaunchKernelGGL(slice_kernel, dim3(grid_for(work)), dim3(256), 0, stream, packed, scales, K, n0, rows, k0, ks,
                     out, out_scales);
  return hipGetLastError();
}

}  // namespace q2dev
