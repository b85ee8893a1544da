// Host-side driver for the C ABI's argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code.  Every
// call here must be rejected (or be an empty no-op) before the library makes
// any HIP call, so the driver runs without a GPU.  Exit status 0 when every
// status matches; the sanitizers abort on any memory or UB error.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "q2.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: got %d (%s), want %d\n", what, got, q2_strerror(got), want);
    ++failures;
  }
}

int main() {
  // 16-byte aligned addresses that are never dereferenced: every call below
  // fails validation or is empty before touching them.
  alignas(256) static unsigned char arena[1024];
  void* F = arena;
  unsigned char* F1 = arena + 1;
  const int64_t big = INT64_MAX, small = INT64_MIN;

  for (int st = 1; st >= -12; --st) {
    const char* s = q2_strerror(st);
    if (s == nullptr || std::strlen(s) == 0) ++failures;
  }
  if (q2_last_error() == nullptr) ++failures;

  // workspace sizes at and beyond the limits
  if (q2_lowrank_workspace_bytes(big, 32) != 0 || q2_lowrank_workspace_bytes(1536, big) != 0 ||
      q2_lowrank_workspace_bytes(small, 4) != 0 || q2_lowrank_workspace_bytes(3, 5) != 256 ||
      q2_lowrank_workspace_bytes((int64_t)1 << 46, 65528) != ((size_t)1 << 48) * 65528u ||
      q2_lowrank_workspace_bytes((int64_t)1 << 46, 65535) != SIZE_MAX)
    ++failures;
  if (q2_a8_workspace_bytes(big, big) != 0 || q2_a8_workspace_bytes(small, 128) != 0 ||
      q2_a8_workspace_bytes(3, 128) != 768 || q2_a8_workspace_bytes(1, big) != 0)
    ++failures;

  auto u16 = [](void* p) { return static_cast<const uint16_t*>(p); };
  auto u8 = [](void* p) { return static_cast<const uint8_t*>(p); };
  auto f32 = [](void* p) { return static_cast<float*>(p); };

  // q2_linear: sizes, K, alignment, NULL, overflow
  expect(q2_linear(u16(F), u8(F), u16(F), f32(F), -1, 8, 128, nullptr), Q2_ERR_ARG, "linear M<0");
  expect(q2_linear(u16(F), u8(F), u16(F), f32(F), 4, 8, 100, nullptr), Q2_ERR_SHAPE, "linear K%128");
  expect(q2_linear(u16(F), u8(F), u16(F), f32(F), big, 8, 128, nullptr), Q2_ERR_ARG, "linear M huge");
  expect(q2_linear(u16(F), u8(F), u16(F), f32(F), 4, big, 128, nullptr), Q2_ERR_ARG, "linear N huge");
  expect(q2_linear(u16(F), u8(F), u16(F), f32(F), 4, 8, (int64_t)1 << 40, nullptr), Q2_ERR_SHAPE, "linear K huge");
  expect(q2_linear(u16(F), u8(F), u16(F), f32(F), (int64_t)1 << 30, (int64_t)1 << 30, 128, nullptr), Q2_ERR_ARG,
         "linear M*N huge");
  expect(q2_linear(u16(F1), u8(F), u16(F), f32(F), 4, 8, 128, nullptr), Q2_ERR_ALIGN, "linear x align");
  expect(q2_linear(nullptr, u8(F), u16(F), f32(F), 4, 8, 128, nullptr), Q2_ERR_ARG, "linear x null");
  expect(q2_linear(nullptr, nullptr, nullptr, nullptr, 0, 0, 0, nullptr), Q2_OK, "linear empty");

  // q2_linear_lowrank / q2_linear_ex
  const size_t need = q2_lowrank_workspace_bytes(16, 8);
  expect(q2_linear_lowrank(u16(F), u8(F), u16(F), u16(F), u16(F), small, f32(F), 16, 8, 128, F, need, nullptr),
         Q2_ERR_ARG, "lowrank r min");
  expect(q2_linear_lowrank(u16(F), u8(F), u16(F), u16(F), u16(F), big, f32(F), 16, 8, 128, F, need, nullptr),
         Q2_ERR_ARG, "lowrank r max");
  expect(q2_linear_lowrank(u16(F), u8(F), u16(F), u16(F), u16(F), 8, f32(F), 16, 8, 128, F, need - 1, nullptr),
         Q2_ERR_WORKSPACE, "lowrank workspace");
  expect(q2_linear_ex(u16(F), u8(F), u16(F), nullptr, nullptr, 0, f32(F), 16, 8, 128, nullptr, 0, 0xFFFFFFFFu,
                      nullptr),
         Q2_ERR_ARG, "ex flags");
  expect(q2_linear_ex(u16(F), u8(F), u16(F), nullptr, nullptr, 0, f32(F), 16, 8, 0, nullptr, 0, Q2_ACCUMULATE,
                      nullptr),
         Q2_OK, "ex empty sum");

  // q2_linear_a8
  expect(q2_linear_a8(u16(F), u8(F), u16(F), f32(F), 16, 8, 256, F, 10, nullptr), Q2_ERR_WORKSPACE, "a8 ws");
  expect(q2_linear_a8(u16(F), u8(F), u16(F), f32(F), big, 8, 256, F, 0, nullptr), Q2_ERR_ARG, "a8 M huge");

  // q4_linear, q2_dequant
  expect(q4_linear(u16(F), u8(F), u16(F), u16(F), f32(F), 3, 5, 64, nullptr), Q2_ERR_SHAPE, "q4 K");
  expect(q4_linear(u16(F), u8(F), u16(F), nullptr, f32(F), 3, 5, 128, nullptr), Q2_ERR_ARG, "q4 zero null");
  expect(q2_dequant(u8(F), u16(F), f32(F), 4, 130, nullptr), Q2_ERR_SHAPE, "dequant K");

  // q2_pack
  int64_t bad = 7;
  expect(q2_pack(u8(F), static_cast<const float*>(F), 4, 100, static_cast<uint8_t*>(F), static_cast<uint16_t*>(F),
                 &bad, nullptr),
         Q2_ERR_SHAPE, "pack K");
  if (bad != -1) ++failures;
  expect(q2_pack(u8(F), static_cast<const float*>(F), big, 128, static_cast<uint8_t*>(F),
                 static_cast<uint16_t*>(F), nullptr, nullptr),
         Q2_ERR_ARG, "pack N huge");

  // q2_slice: ranges at the int64 limits
  expect(q2_slice(u8(F), u16(F), 8, 512, 0, big, 0, 128, static_cast<uint8_t*>(F), static_cast<uint16_t*>(F),
                  nullptr),
         Q2_ERR_ARG, "slice n1 huge");
  expect(q2_slice(u8(F), u16(F), 8, 512, small, 4, 0, 128, static_cast<uint8_t*>(F), static_cast<uint16_t*>(F),
                  nullptr),
         Q2_ERR_ARG, "slice n0 min");
  expect(q2_slice(u8(F), u16(F), 8, 512, 0, 4, 0, big, static_cast<uint8_t*>(F), static_cast<uint16_t*>(F),
                  nullptr),
         Q2_ERR_ARG, "slice k1 huge");
  expect(q2_slice(u8(F), u16(F), 8, 512, 0, 4, 64, 256, static_cast<uint8_t*>(F), static_cast<uint16_t*>(F),
                  nullptr),
         Q2_ERR_SHAPE, "slice block");

  // q2_import_gemlite: group lengths at the limits
  expect(q2_import_gemlite(u8(F), static_cast<const float*>(F), static_cast<const float*>(F), 8, 512, big,
                           static_cast<uint8_t*>(F), static_cast<uint16_t*>(F), &bad, nullptr),
         Q2_ERR_SHAPE, "import G huge");
  expect(q2_import_gemlite(u8(F), static_cast<const float*>(F), static_cast<const float*>(F), 8, 512, small,
                           static_cast<uint8_t*>(F), static_cast<uint16_t*>(F), &bad, nullptr),
         Q2_ERR_SHAPE, "import G min");
  expect(q2_import_gemlite(u8(F), static_cast<const float*>(F), static_cast<const float*>(F), 8, 512, 48,
                           static_cast<uint8_t*>(F), static_cast<uint16_t*>(F), &bad, nullptr),
         Q2_ERR_SHAPE, "import G 48");

  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("abi driver ok\n");
  return 0;
}
