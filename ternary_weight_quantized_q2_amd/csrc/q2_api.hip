// q2_api.hip - the C ABI of libq2: argument validation, device check, dispatch.
// Every argument check runs before the first HIP call, so a host without a GPU
// still gets argument, shape and alignment errors.
#include <atomic>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "q2.h"
#include "q2_internal.h"

namespace {

thread_local char g_detail[320];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_detail[0] = '\0';
  return Q2_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// pointer must be non-NULL when the buffer is non-empty, and aligned
int check_ptr(const void* p, bool nonempty, size_t align, const char* name) {
  if (nonempty && p == nullptr) return fail(Q2_ERR_ARG, "%s is NULL for a non-empty buffer", name);
  if (p != nullptr && !aligned(p, align)) return fail(Q2_ERR_ALIGN, "%s is not %zu-byte aligned", name, align);
  return Q2_OK;
}

int check_sizes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return fail(Q2_ERR_ARG, "negative size (M=%lld N=%lld K=%lld)", (long long)M,
                                           (long long)N, (long long)K);
  if (K % 128 != 0) return fail(Q2_ERR_SHAPE, "K=%lld is not a multiple of 128", (long long)K);
  // keep every element index inside int64 with room to spare
  const int64_t lim = (int64_t)1 << 46;
  if (M > lim || N > lim || K > lim || (M > 0 && K > lim / M) || (N > 0 && K > lim / N) ||
      (M > 0 && N > lim / M))
    return fail(Q2_ERR_ARG, "sizes too large");
  return Q2_OK;
}

// The linear kernels address one tile's activation rows and weight columns
// with 32-bit offsets; K up to 2^24 keeps them in range for every tile shape.
int check_linear_k(int64_t K) {
  if (K > ((int64_t)1 << 24)) return fail(Q2_ERR_SHAPE, "K=%lld exceeds 16777216", (long long)K);
  return Q2_OK;
}

std::atomic<int> g_arch_ok[64];
std::mutex g_check_lock;              // q2_pack and q2_import_gemlite share the device's error flags

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(Q2_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  const int slot = (dev >= 0 && dev < 64) ? dev : -1;
  if (slot >= 0) {
    const int st = g_arch_ok[slot].load(std::memory_order_relaxed);
    if (st == 1) return Q2_OK;
    if (st == -1) return fail(Q2_ERR_DEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(Q2_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (slot >= 0) g_arch_ok[slot].store(good ? 1 : -1, std::memory_order_relaxed);
  if (!good) return fail(Q2_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return Q2_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(Q2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Test and profiling control of the launch choice: the path (0 automatic,
// 1 GEMV, 2 GEMM), a GEMM configuration (0 automatic, else its number, -1 an
// unknown name) and the K split (0 automatic, 1 or 2, -1 anything else).  The
// environment (Q2_FORCE_PATH=gemv|gemm, Q2_GEMM_TILE=<name>,
// Q2_GEMM_KSPLIT=1|2) is read once per process, at the first linear call;
// q2_set_dispatch replaces it.  The hot path only loads three integers.
struct Dispatch {
  std::atomic<int> path{0}, cfg{0}, ksplit{0};
};
Dispatch g_dispatch;
std::once_flag g_dispatch_env;

int parse_path(const char* v) {
  if (v == nullptr || *v == 0 || std::strcmp(v, "auto") == 0) return 0;
  if (std::strcmp(v, "gemv") == 0) return 1;
  if (std::strcmp(v, "gemm") == 0) return 2;
  return -1;
}

// bf16 GEMM configurations keep their numbers; the int8 ones (q2_linear_a8)
// are numbered from kA8Base on.
constexpr int kA8Base = 1000;

int parse_cfg(const char* v) {
  if (v == nullptr || *v == 0) return 0;
  const int id = q2dev::gemm_config_id(v);
  if (id >= 0) return id;
  const int a8 = q2dev::a8_config_id(v);
  return a8 > 0 ? kA8Base + a8 : a8;
}

int parse_ksplit(const char* v) {
  if (v == nullptr || *v == 0) return 0;
  if (std::strcmp(v, "1") == 0) return 1;
  if (std::strcmp(v, "2") == 0) return 2;
  return -1;
}

void read_dispatch_env() {
  std::call_once(g_dispatch_env, [] {
    const int p = parse_path(std::getenv("Q2_FORCE_PATH"));
    g_dispatch.path.store(p < 0 ? 0 : p);
    g_dispatch.cfg.store(parse_cfg(std::getenv("Q2_GEMM_TILE")));
    g_dispatch.ksplit.store(parse_ksplit(std::getenv("Q2_GEMM_KSPLIT")));
  });
}

int linear_common(int fmt, const uint16_t* x, const uint8_t* w, const uint16_t* s, const uint16_t* z, float* y,
                  int64_t M, int64_t N, int64_t K, const uint16_t* lr_t, const uint16_t* lr_b, int64_t r,
                  bool accumulate, hipStream_t stream) {
  q2dev::LinearArgs a;
  a.x = x; a.w = w; a.s = s; a.z = z; a.y = y;
  a.M = M; a.N = N; a.K = K;
  a.lr_t = lr_t; a.lr_b = lr_b; a.r = (int)r;
  a.acc = accumulate ? 1 : 0;
  read_dispatch_env();
  int path = g_dispatch.path.load(std::memory_order_relaxed);
  if (path == 1 && M > 16) path = 0;
  int cfg = g_dispatch.cfg.load(std::memory_order_relaxed);
  if (cfg < 0) return fail(Q2_ERR_ARG, "unknown Q2_GEMM_TILE configuration");
  if (cfg >= kA8Base) cfg = 0;                        // an int8 configuration: automatic here
  const int ks = g_dispatch.ksplit.load(std::memory_order_relaxed);
  if (ks < 0) return fail(Q2_ERR_ARG, "Q2_GEMM_KSPLIT must be 1 or 2");
  return hip_status(q2dev::launch_linear(a, fmt, path, cfg, ks, stream),
                    fmt == 0 ? "q2 linear launch" : "q4 linear launch");
}

// The Q2_0 linear entry points: y = x W^T (+ (x A^T) B^T when r > 0), written
// or, with Q2_ACCUMULATE, added to y.
int linear_entry(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16, const uint16_t* A_f16,
                 const uint16_t* B_f16, int64_t r, float* y, int64_t M, int64_t N, int64_t K, void* workspace,
                 size_t workspace_bytes, uint32_t flags, hipStream_t stream, bool validate_only = false) {
  int st = check_sizes(M, N, K);
  if (st || (st = check_linear_k(K))) return st;
  if (flags & ~(uint32_t)Q2_ACCUMULATE) return fail(Q2_ERR_ARG, "unknown flag bits 0x%x", flags & ~Q2_ACCUMULATE);
  if (r < 0) return fail(Q2_ERR_ARG, "negative rank r=%lld", (long long)r);
  if (r > 65535) return fail(Q2_ERR_ARG, "rank r=%lld too large (at most 65535)", (long long)r);
  if ((st = check_ptr(x_bf16, M > 0 && K > 0, 16, "x")) ||
      (st = check_ptr(packed, N > 0 && K > 0, 16, "packed")) ||
      (st = check_ptr(scales_f16, N > 0 && K > 0, 2, "scales_f16")))
    return st;
  if (r > 0 && ((st = check_ptr(A_f16, K > 0, 16, "A")) || (st = check_ptr(B_f16, N > 0, 2, "B")))) return st;
  if ((st = check_ptr(y, M > 0 && N > 0, 4, "y"))) return st;
  if (M == 0 || N == 0) return ok();
  const bool accumulate = (flags & Q2_ACCUMULATE) != 0;
  if (accumulate && K == 0) return ok();           // an empty sum added: y stays as it is
  if (validate_only) return ok();
  uint16_t* tl = nullptr;
  if (r > 0) {
    const size_t need = q2_lowrank_workspace_bytes(M, r);
    if (workspace_bytes < need)
      return fail(Q2_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (workspace == nullptr) return fail(Q2_ERR_ARG, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(Q2_ERR_ALIGN, "workspace is not 256-byte aligned");
    tl = static_cast<uint16_t*>(workspace);
  }
  if ((st = check_device())) return st;
  if (r > 0 &&
      (st = hip_status(q2dev::launch_lowrank_t(x_bf16, A_f16, tl, M, K, (int)r, stream), "low-rank x A^T launch")))
    return st;
  return linear_common(0, x_bf16, packed, scales_f16, nullptr, y, M, N, K, tl, B_f16, r, accumulate, stream);
}

// Scratch of q2_linear_lowrank_noalloc: the x A^T limbs live in this
// file-scope device array instead of a caller workspace.  Each device holds its
// own copy; its address is looked up once per device (with that device
// current) and kept, and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)Q2_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

int noalloc_scratch(void** out) {
  static std::mutex lock;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(Q2_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(Q2_ERR_DEVICE, "device %d out of range", dev);
  std::lock_guard<std::mutex> g(lock);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(Q2_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return Q2_OK;
}

}  // namespace

extern "C" {

const char* q2_strerror(int status) {
  switch (status) {
    case Q2_OK: return "Q2_OK";
    case Q2_ERR_ARG: return "Q2_ERR_ARG: invalid argument";
    case Q2_ERR_SHAPE: return "Q2_ERR_SHAPE: K must be a multiple of 128";
    case Q2_ERR_ALIGN: return "Q2_ERR_ALIGN: misaligned pointer";
    case Q2_ERR_CODE: return "Q2_ERR_CODE: code outside {0,1,2}";
    case Q2_ERR_SCALE: return "Q2_ERR_SCALE: scale not exactly representable in f16";
    case Q2_ERR_DEVICE: return "Q2_ERR_DEVICE: current device is not gfx950";
    case Q2_ERR_HIP: return "Q2_ERR_HIP: HIP runtime error";
    case Q2_ERR_WORKSPACE: return "Q2_ERR_WORKSPACE: workspace too small or misaligned";
    case Q2_ERR_FORMAT: return "Q2_ERR_FORMAT: zero point is not minus the scale";
    default: return "unknown q2 status";
  }
}

const char* q2_last_error(void) { return g_detail; }

int q2_set_dispatch(const char* path, const char* tile, int ksplit) {
  read_dispatch_env();
  const int p = parse_path(path), c = parse_cfg(tile);
  if (p < 0) return fail(Q2_ERR_ARG, "path must be NULL, \"auto\", \"gemv\" or \"gemm\"");
  if (c < 0) return fail(Q2_ERR_ARG, "unknown GEMM configuration \"%s\"", tile);
  if (ksplit < 0 || ksplit > 2) return fail(Q2_ERR_ARG, "ksplit must be 0 (automatic), 1 or 2");
  g_dispatch.path.store(p);
  g_dispatch.cfg.store(c);
  g_dispatch.ksplit.store(ksplit);
  return ok();
}

size_t q2_a8_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || M > ((int64_t)1 << 40) / K) return 0;
  const size_t codes = ((size_t)M * (size_t)K + 255u) & ~(size_t)255u;
  return codes + (((size_t)M * 4u + 255u) & ~(size_t)255u);
}

int q2_linear_a8(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16, float* y, int64_t M,
                 int64_t N, int64_t K, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_sizes(M, N, K);
  if (st || (st = check_linear_k(K))) return st;
  if ((st = check_ptr(x_bf16, M > 0 && K > 0, 16, "x")) ||
      (st = check_ptr(packed, N > 0 && K > 0, 16, "packed")) ||
      (st = check_ptr(scales_f16, N > 0 && K > 0, 2, "scales_f16")) ||
      (st = check_ptr(y, M > 0 && N > 0, 4, "y")))
    return st;
  if (M == 0 || N == 0) return ok();
  const size_t need = q2_a8_workspace_bytes(M, K);
  if (workspace_bytes < need)
    return fail(Q2_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (need > 0 && workspace == nullptr) return fail(Q2_ERR_ARG, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(Q2_ERR_ALIGN, "workspace is not 256-byte aligned");
  if ((st = check_device())) return st;
  if (K == 0) return linear_common(0, x_bf16, packed, scales_f16, nullptr, y, M, N, K, nullptr, nullptr, 0, false,
                                   stream);
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  float* rs = reinterpret_cast<float*>(xq + (((size_t)M * (size_t)K + 255u) & ~(size_t)255u));
  if ((st = hip_status(q2dev::launch_quantize_rows_i8(x_bf16, xq, rs, M, K, stream), "8-bit quantisation launch")))
    return st;
  read_dispatch_env();
  const int cfg = g_dispatch.cfg.load(std::memory_order_relaxed);
  if (cfg < 0) return fail(Q2_ERR_ARG, "unknown Q2_GEMM_TILE configuration");
  const int ks = g_dispatch.ksplit.load(std::memory_order_relaxed);
  if (ks < 0) return fail(Q2_ERR_ARG, "Q2_GEMM_KSPLIT must be 1 or 2");
  q2dev::A8Args a;
  a.xq = xq; a.w = packed; a.s = scales_f16; a.row_scale = rs; a.y = y;
  a.M = M; a.N = N; a.K = K;
  return hip_status(q2dev::launch_linear_a8(a, cfg >= kA8Base ? cfg - kA8Base : 0, ks, stream), "a8 linear launch");
}

size_t q2_lowrank_workspace_bytes(int64_t M, int64_t r) {
  if (M <= 0 || r <= 0 || M > ((int64_t)1 << 46) || r > 65535) return 0;   // outside what the linear accepts
  // bf16 hi and lo limbs of x A^T per row, each r rounded up to a multiple of 8
  const size_t row = (size_t)((r + 7) & ~(int64_t)7) * 4u;
  if ((size_t)M > (SIZE_MAX - 255u) / row) return SIZE_MAX;                 // no buffer can be that large
  const size_t b = (size_t)M * row;
  return (b + 255u) & ~(size_t)255u;
}

int q2_pack(const uint8_t* codes, const float* scales, int64_t N, int64_t K, uint8_t* packed,
            uint16_t* scales_f16, int64_t* bad_index, hipStream_t stream) {
  if (bad_index) *bad_index = -1;
  int st = check_sizes(0, N, K);
  if (st) return st;
  const bool ne = N > 0 && K > 0;
  if ((st = check_ptr(codes, ne, 16, "codes")) || (st = check_ptr(scales, ne, 4, "scales")) ||
      (st = check_ptr(packed, ne, 16, "packed")) || (st = check_ptr(scales_f16, ne, 2, "scales_f16")))
    return st;
  if (!ne) return ok();
  if ((st = check_device())) return st;

  // One pack or import at a time per process: they share the device's flags.
  std::lock_guard<std::mutex> serial(g_check_lock);
  unsigned long long* flags = nullptr;
  hipError_t e = q2dev::check_flags(&flags);
  if (e != hipSuccess) return hip_status(e, "q2_pack flags");
  unsigned long long host[2] = {~0ull, ~0ull};
  e = hipMemsetAsync(flags, 0xFF, sizeof host, stream);
  if (e == hipSuccess) e = q2dev::launch_pack(codes, scales, N, K, packed, scales_f16, flags, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(host, flags, sizeof host, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "q2_pack");
  if (host[0] != ~0ull) {
    if (bad_index) *bad_index = (int64_t)host[0];
    return fail(Q2_ERR_CODE, "code above 2 at flat index %llu", host[0]);
  }
  if (host[1] != ~0ull) {
    if (bad_index) *bad_index = (int64_t)host[1];
    return fail(Q2_ERR_SCALE, "scale at flat index %llu is not an exact f16 value", host[1]);
  }
  return ok();
}

int q2_linear(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16, float* y, int64_t M,
              int64_t N, int64_t K, hipStream_t stream) {
  return linear_entry(x_bf16, packed, scales_f16, nullptr, nullptr, 0, y, M, N, K, nullptr, 0, 0u, stream);
}

int q2_linear_lowrank(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16,
                      const uint16_t* A_f16, const uint16_t* B_f16, int64_t r, float* y, int64_t M, int64_t N,
                      int64_t K, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return linear_entry(x_bf16, packed, scales_f16, A_f16, B_f16, r, y, M, N, K, workspace, workspace_bytes, 0u,
                      stream);
}

int q2_linear_lowrank_noalloc(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16,
                              const uint16_t* A_f16, const uint16_t* B_f16, int64_t r, float* y, int64_t M, int64_t N,
                              int64_t K, hipStream_t stream) {
  int st = check_sizes(M, N, K);
  if (st) return st;
  if (r < 0 || r > 65535) return linear_entry(x_bf16, packed, scales_f16, A_f16, B_f16, r, y, M, N, K, nullptr, 0, 0u,
                                              stream);                  // the same argument error
  const size_t need = (r > 0 && M > 0) ? q2_lowrank_workspace_bytes(M, r) : 0;
  if (need > kNoAllocScratchBytes)
    return fail(Q2_ERR_WORKSPACE, "M=%lld r=%lld needs %zu bytes of scratch; this entry point holds %zu",
                (long long)M, (long long)r, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    // Arguments first (as for q2_linear_lowrank), so argument errors never touch the device.
    if ((st = linear_entry(x_bf16, packed, scales_f16, A_f16, B_f16, r, y, M, N, K, nullptr, 0, 0u, nullptr,
                           /*validate_only=*/true)))
      return st;
    if (M > 0 && N > 0 && ((st = check_device()) || (st = noalloc_scratch(&ws)))) return st;
  }
  return linear_entry(x_bf16, packed, scales_f16, A_f16, B_f16, r, y, M, N, K, ws, ws ? kNoAllocScratchBytes : 0, 0u,
                      stream);
}

int q2_linear_ex(const uint16_t* x_bf16, const uint8_t* packed, const uint16_t* scales_f16, const uint16_t* A_f16,
                 const uint16_t* B_f16, int64_t r, float* y, int64_t M, int64_t N, int64_t K, void* workspace,
                 size_t workspace_bytes, uint32_t flags, hipStream_t stream) {
  return linear_entry(x_bf16, packed, scales_f16, A_f16, B_f16, r, y, M, N, K, workspace, workspace_bytes, flags,
                      stream);
}

int q4_linear(const uint16_t* x_bf16, const uint8_t* packed4, const uint16_t* scale_f16, const uint16_t* zero_f16,
              float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  int st = check_sizes(M, N, K);
  if (st || (st = check_linear_k(K))) return st;
  if ((st = check_ptr(x_bf16, M > 0 && K > 0, 16, "x")) ||
      (st = check_ptr(packed4, N > 0 && K > 0, 16, "packed4")) ||
      (st = check_ptr(scale_f16, N > 0 && K > 0, 2, "scale_f16")) ||
      (st = check_ptr(zero_f16, N > 0 && K > 0, 2, "zero_f16")) || (st = check_ptr(y, M > 0 && N > 0, 4, "y")))
    return st;
  if (M == 0 || N == 0) return ok();
  if ((st = check_device())) return st;
  return linear_common(1, x_bf16, packed4, scale_f16, zero_f16, y, M, N, K, nullptr, nullptr, 0, false, stream);
}

int q2_import_gemlite(const uint8_t* codes_t, const float* scales_t, const float* zeros_t, int64_t N, int64_t K,
                      int64_t G, uint8_t* packed, uint16_t* scales_f16, int64_t* bad_index, hipStream_t stream) {
  if (bad_index) *bad_index = -1;
  int st = check_sizes(0, N, K);
  if (st) return st;
  if (G <= 0 || G % 4 != 0 || (128 % G != 0 && G % 128 != 0) || K % G != 0)
    return fail(Q2_ERR_SHAPE, "group length G=%lld must divide 128 or be a multiple of it, and divide K=%lld",
                (long long)G, (long long)K);
  const bool ne = N > 0 && K > 0;
  if ((st = check_ptr(codes_t, ne, 1, "codes_t")) || (st = check_ptr(scales_t, ne, 4, "scales_t")) ||
      (st = check_ptr(zeros_t, ne, 4, "zeros_t")) || (st = check_ptr(packed, ne, 16, "packed")) ||
      (st = check_ptr(scales_f16, ne, 2, "scales_f16")))
    return st;
  if (!ne) return ok();
  if ((st = check_device())) return st;

  std::lock_guard<std::mutex> serial(g_check_lock);
  unsigned long long* flags = nullptr;
  hipError_t e = q2dev::check_flags(&flags);
  if (e != hipSuccess) return hip_status(e, "q2_import_gemlite flags");
  unsigned long long host[4] = {~0ull, ~0ull, ~0ull, ~0ull};
  e = hipMemsetAsync(flags, 0xFF, sizeof host, stream);
  if (e == hipSuccess) e = q2dev::launch_import(codes_t, scales_t, zeros_t, N, K, G, packed, scales_f16, flags, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(host, flags, sizeof host, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "q2_import_gemlite");
  // Reported in the order codes, zero points, scale values, block agreement.
  if (host[0] != ~0ull) {
    if (bad_index) *bad_index = (int64_t)host[0];
    return fail(Q2_ERR_CODE, "code 3 at weight index %llu", host[0]);
  }
  if (host[1] != ~0ull) {
    if (bad_index) *bad_index = (int64_t)host[1];
    return fail(Q2_ERR_FORMAT, "zero point at group index %llu is not minus its scale", host[1]);
  }
  if (host[2] != ~0ull) {
    if (bad_index) *bad_index = (int64_t)host[2];
    return fail(Q2_ERR_SCALE, "scale at group index %llu is not an exact f16 value", host[2]);
  }
  if (host[3] != ~0ull) {
    if (bad_index) *bad_index = (int64_t)host[3];
    return fail(Q2_ERR_SCALE, "scale at group index %llu differs from its 128-weight block's first group",
                host[3]);
  }
  return ok();
}

int q2_slice(const uint8_t* packed, const uint16_t* scales_f16, int64_t N, int64_t K, int64_t n0, int64_t n1,
             int64_t k0, int64_t k1, uint8_t* out_packed, uint16_t* out_scales, hipStream_t stream) {
  int st = check_sizes(0, N, K);
  if (st) return st;
  if (n0 < 0 || n1 < n0 || n1 > N || k0 < 0 || k1 < k0 || k1 > K)
    return fail(Q2_ERR_ARG, "slice rows [%lld, %lld) / inputs [%lld, %lld) outside N=%lld K=%lld", (long long)n0,
                (long long)n1, (long long)k0, (long long)k1, (long long)N, (long long)K);
  if (k0 % 128 != 0 || k1 % 128 != 0)
    return fail(Q2_ERR_SHAPE, "slice inputs [%lld, %lld) not on 128-weight block boundaries", (long long)k0,
                (long long)k1);
  const bool ne = n1 > n0 && k1 > k0;
  if ((st = check_ptr(packed, ne, 16, "packed")) || (st = check_ptr(scales_f16, ne, 2, "scales_f16")) ||
      (st = check_ptr(out_packed, ne, 16, "out_packed")) || (st = check_ptr(out_scales, ne, 2, "out_scales")))
    return st;
  if (!ne) return ok();
  if ((st = check_device())) return st;
  return hip_status(q2dev::launch_slice(packed, scales_f16, K, n0, n1 - n0, k0, k1 - k0, out_packed, out_scales,
                                        stream),
                    "slice launch");
}

int q2_dequant(const uint8_t* packed, const uint16_t* scales_f16, float* w, int64_t N, int64_t K,
               hipStream_t stream) {
  int st = check_sizes(0, N, K);
  if (st) return st;
  const bool ne = N > 0 && K > 0;
  if ((st = check_ptr(packed, ne, 16, "packed")) || (st = check_ptr(scales_f16, ne, 2, "scales_f16")) ||
      (st = check_ptr(w, ne, 4, "w")))
    return st;
  if (!ne) return ok();
  if ((st = check_device())) return st;
  return hip_status(q2dev::launch_dequant(packed, scales_f16, w, N, K, stream), "dequant launch");
}

}  // extern "C"
