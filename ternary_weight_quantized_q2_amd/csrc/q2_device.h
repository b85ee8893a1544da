// q2_device.h - device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core layout used everywhere (v_mfma_f32_16x16x32_bf16, wave64):
//   lane l, column c = l % 16, lane group g = l / 16.
//   A operand: 8 bf16 of row c;  B operand: 8 bf16 of column c;  both hold the
//   K-slots 8g .. 8g+7 of the instruction's 32-wide K window, so a dot product
//   is correct whenever A and B put the same real k in the same (g, element).
//   C/D: 4 fp32 of column c, rows 4g + 0..3.
//
// Weight decoding by a floating-point "magic number": a 2-bit or 4-bit code q
// is OR-ed into the fraction bits of bf16 1.0, which gives the exact bf16
// value 1 + q/4 (2-bit code in fraction bits 5-6) or 1 + q/16 (4-bit code in
// fraction bits 3-6).  One shift and one and-or build two bf16 weights (the
// two 16-bit halves of a dword), so the decode costs about one VALU op per
// weight.  The constant 1 is removed through the accumulator: per 128-block
// the MFMA accumulator starts at -1.25 * sum(x) (2-bit) so that it ends at
// sum x (q - 1) / 4 exactly in real arithmetic; the 4-bit path starts it at
// -(1 + z/16) * sum(x) and ends at sum x (q - z) / 16.
//
// The offset start is exact in real arithmetic but not in fp32: the two sums
// round in different orders, so a block whose weights are all zero would leave
// rounding noise of the size of ulp(1.25 |S|).  Every kernel therefore tests
// each (weight row, block) for an all-zero block -- every 2-bit code equal to
// 1, or every 4-bit code equal to an integer zero point -- and applies a scale
// of 0 to it, so such a block adds exactly nothing (column_all below).
//
// Two pair orders are used.  Strided pairs (GEMV): because a dword's two
// halves are 16 bits apart, one shift and one and-or make a 2-bit pair of codes
// (j, j+8) of the dword's 16 codes, or a 4-bit pair of codes (j, j+4) of its 8;
// the activations are then stored in shared memory in the same pair order by
// the staging threads.  Consecutive pairs (GEMM): the activation fragments are
// read from shared memory as copied, so the weight pairs hold codes (2p, 2p+1);
// building them costs a byte permute and a packed shift more per dword.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 q2_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 q2_bf16x2 __attribute__((ext_vector_type(2)));
typedef float q2_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t q2_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t q2_u32x2 __attribute__((ext_vector_type(2)));

namespace q2dev {

constexpr int WAVE = 64;
constexpr int BLOCK_K = 128;          // weights per Q2_0 block / 4-bit group

// Output tiles of the GEMM kernels are stored non-temporally, so the fp32
// output does not displace the operands that later tiles read from L2.  Under
// accumulation (y += result) a thread first loads every y value it will write,
// all at once, before the tile's final reduction: a load issued after a store
// would wait for that store (loads and stores share one counter), so loading
// piece by piece between the stores would pay one memory round trip each.
__device__ __forceinline__ float y_old(const float* p, bool valid) {
  return valid ? __builtin_nontemporal_load(p) : 0.0f;
}
__device__ __forceinline__ q2_f32x4 y_old4(const q2_f32x4* p, bool valid) {
  return valid ? __builtin_nontemporal_load(p) : q2_f32x4{0.f, 0.f, 0.f, 0.f};
}

// Piece t of the row-major stores of a BM x BN output tile by THREADS
// threads: 16 bytes at tile row `row`, columns 4q .. 4q+3.  False when the
// piece is past the tile or past its nrows valid rows or ncols valid columns
// (tile-relative 32-bit counts, so no 64-bit row index lives across the
// kernel's main loop).
template <int BM, int BN, int THREADS>
__device__ __forceinline__ bool row_piece(int t, int tid, int nrows, int ncols, int& row, int& q) {
  const int idx = tid + t * THREADS;
  row = idx / (BN / 4);
  q = idx - row * (BN / 4);
  return idx < BM * (BN / 4) && row < nrows && 4 * q < ncols;
}

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over `bytes` bytes from `base` for untyped 32-bit loads
// (stride 0; the third word selects the 32-bit data format).  A copy through
// it takes a 32-bit per-lane offset and a wave-uniform scalar offset, so the
// address arithmetic of the global-to-LDS copies stays in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// and all its LDS operations are done, then meet the other waves.  Unlike
// __syncthreads this does not drain every outstanding load, so the
// global-to-LDS copies of later blocks stay in flight across the barrier.
// Vector-memory loads complete in issue order, so "at most N outstanding"
// means everything issued before the last N has landed.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));   // vmcnt(N) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Consecutive workgroup ids are dispatched to the eight XCDs in turn.  This
// hands each XCD a contiguous range of tile numbers instead, and the numbers
// run over groups of group_m row tiles, row-fastest inside a group: with
// group_m = all row tiles each XCD reads 1/8 of the weights and all of x (few
// rows), with group_m = 1/8 of them each XCD reads 1/8 of x and all of the
// weights (many rows), and in between the tile grid is cut into 8 blocks.
__device__ __forceinline__ int xcd_tile(int b, int tiles) {
  const int per = tiles >> 3, rem = tiles & 7;
  const int xcd = b & 7, local = b >> 3;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
}

__device__ __forceinline__ q2_f32x4 mfma(q2_u32x4 a, q2_u32x4 b, q2_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(q2_bf16x8, a),
                                                  __builtin_bit_cast(q2_bf16x8, b), c, 0, 0, 0);
}

// (a & m) | o in one v_and_or_b32.  gfx950 VOP3 encodings take no literal
// operands, so the two constants are passed in VGPRs (kept live by the caller);
// written plainly, the compiler splits the expression into an AND and an OR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// Decoder constants: mask of the code field in each 16-bit half, and the bf16
// pattern of 1.0 in both halves.
struct DecodeConsts {
  uint32_t mask, one;
};
__device__ __forceinline__ DecodeConsts q2_consts() {
  DecodeConsts k;
  // opaque to the optimiser so both stay in VGPRs
  asm("v_mov_b32 %0, 0x00600060" : "=v"(k.mask));
  asm("v_mov_b32 %0, 0x3f803f80" : "=v"(k.one));
  return k;
}
__device__ __forceinline__ DecodeConsts q4_consts() {
  DecodeConsts k;
  asm("v_mov_b32 %0, 0x00780078" : "=v"(k.mask));
  asm("v_mov_b32 %0, 0x3f803f80" : "=v"(k.one));
  return k;
}

// ---- 2-bit codes -----------------------------------------------------------
// Pair J (0..7) of dword w: halves = bf16(1 + c_J/4), bf16(1 + c_{J+8}/4).
template <int J>
__device__ __forceinline__ uint32_t q2_pair(uint32_t w, DecodeConsts k) {
  uint32_t s;
  if constexpr (J <= 2) s = w << (5 - 2 * J);
  else s = w >> (2 * J - 5);
  return and_or(s, k.mask, k.one);
}
// B operand for half H (0/1) of a codes dword: pairs 4H .. 4H+3.
template <int H>
__device__ __forceinline__ q2_u32x4 q2_bfrag(uint32_t w, DecodeConsts k) {
  return q2_u32x4{q2_pair<4 * H>(w, k), q2_pair<4 * H + 1>(w, k), q2_pair<4 * H + 2>(w, k),
                  q2_pair<4 * H + 3>(w, k)};
}

// ---- 4-bit codes -----------------------------------------------------------
// Pair J (0..3) of dword w (8 nibbles): halves = bf16(1 + q_J/16), bf16(1 + q_{J+4}/16).
template <int J>
__device__ __forceinline__ uint32_t q4_pair(uint32_t w, DecodeConsts k) {
  uint32_t s;
  if constexpr (J == 0) s = w << 3;
  else s = w >> (4 * J - 3);
  return and_or(s, k.mask, k.one);
}
__device__ __forceinline__ q2_u32x4 q4_bfrag(uint32_t w, DecodeConsts k) {
  return q2_u32x4{q4_pair<0>(w, k), q4_pair<1>(w, k), q4_pair<2>(w, k), q4_pair<3>(w, k)};
}

// ---- consecutive pairs -------------------------------------------------------
// The GEMM reads its activation fragments as 8 consecutive x straight from
// shared memory, so there a weight dword must hold two consecutive codes.
// For 2-bit codes one byte permute copies the byte of four codes into bits
// 8-15 of both 16-bit halves, and a packed 16-bit shift (different amount per
// half) brings code 2p to the low half's bits 5-6 and code 2p+1 to the high
// half's: 2.5 VALU ops per pair.  For 4-bit codes the even and odd nibbles are
// separated once per dword, a byte permute pairs nibble 2p (low half) with
// nibble 2p+1 (high half) and one shift-or lands both in bits 3-6.
struct NatConsts {
  uint32_t mask, one, sh01, sh23;
};
__device__ __forceinline__ NatConsts q2_nat_consts() {
  NatConsts k;
  asm("v_mov_b32 %0, 0x00600060" : "=v"(k.mask));
  asm("v_mov_b32 %0, 0x3f803f80" : "=v"(k.one));
  asm("v_mov_b32 %0, 0x00050003" : "=v"(k.sh01));   // low half >> 3, high half >> 5
  asm("v_mov_b32 %0, 0x00090007" : "=v"(k.sh23));   // low half >> 7, high half >> 9
  return k;
}
__device__ __forceinline__ NatConsts q4_nat_consts() {
  NatConsts k;
  asm("v_mov_b32 %0, 0x0f0f0f0f" : "=v"(k.mask));
  asm("v_mov_b32 %0, 0x3f803f80" : "=v"(k.one));
  k.sh01 = k.sh23 = 0;
  return k;
}

// Independent shifts of the two 16-bit halves of v (amounts in the halves of sh).
__device__ __forceinline__ uint32_t pk_shr16(uint32_t v, uint32_t sh) {
  uint32_t r;
  asm("v_pk_lshrrev_b16 %0, %1, %2" : "=v"(r) : "v"(sh), "v"(v));
  return r;
}

// Byte B of w in bits 8-15 of both halves, zeros elsewhere (selector 0x0C = 0).
template <int B>
__device__ __forceinline__ uint32_t byte_to_halves(uint32_t w) {
  return __builtin_amdgcn_perm(w, w, 0x000C000Cu | (B << 8) | (B << 24));
}

// B operand from 16-bit half H of a 2-bit codes dword (codes 8H .. 8H+7): dword
// p holds bf16(1 + c/4) of codes 8H + 2p (low half) and 8H + 2p + 1 (high half).
template <int H>
__device__ __forceinline__ q2_u32x4 q2_bfrag_nat(uint32_t w, const NatConsts& k) {
  const uint32_t u0 = byte_to_halves<2 * H>(w), u1 = byte_to_halves<2 * H + 1>(w);
  return q2_u32x4{and_or(pk_shr16(u0, k.sh01), k.mask, k.one), and_or(pk_shr16(u0, k.sh23), k.mask, k.one),
                  and_or(pk_shr16(u1, k.sh01), k.mask, k.one), and_or(pk_shr16(u1, k.sh23), k.mask, k.one)};
}

// B operand from a 4-bit codes dword (8 nibbles): dword p holds bf16(1 + q/16)
// of nibbles 2p (low half) and 2p + 1 (high half).
__device__ __forceinline__ q2_u32x4 q4_bfrag_nat(uint32_t w, const NatConsts& k) {
  const uint32_t e = w & k.mask, o = (w >> 4) & k.mask;
  q2_u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t t = __builtin_amdgcn_perm(o, e, 0x0C000C00u | (uint32_t)p | ((uint32_t)(p + 4) << 16));
    r[p] = (t << 3) | k.one;
  }
  return r;
}

// ---- activation pair order -------------------------------------------------
// nx[h] = (x[2h], x[2h+1]) for 16 consecutive x.  2-bit order: out[j] =
// (x[j], x[j+8]) for j = 0..7.
__device__ __forceinline__ void q2_xpairs(const uint32_t nx[8], uint32_t out[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t a = nx[j >> 1], b = nx[4 + (j >> 1)];
    out[j] = (j & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
  }
}
// 4-bit order, two groups of 8 x: out[4i + j] = (x[8i + j], x[8i + j + 4]).
__device__ __forceinline__ void q4_xpairs(const uint32_t nx[8], uint32_t out[8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = nx[4 * i + (j >> 1)], b = nx[4 * i + 2 + (j >> 1)];
      out[4 * i + j] = (j & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
  }
}

// Sum of 16 bf16 (8 dwords) in fp32, fixed order.
__device__ __forceinline__ float bf16_sum16(const uint32_t nx[8]) {
  const q2_bf16x2 one = __builtin_bit_cast(q2_bf16x2, 0x3F803F80u);
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int h = 0; h < 8; h += 2) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(q2_bf16x2, nx[h]), one, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(q2_bf16x2, nx[h + 1]), one, s1, false);
  }
  return s0 + s1;
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// ---- all-zero blocks ---------------------------------------------------------
// In the matrix-core layout the four lanes c, c + 16, c + 32, c + 48 hold the
// codes of one weight row (column c) of a 128-weight block between them.  The
// lane verdicts below are wave masks (one bit per lane, straight from the
// vector compares); column_all turns one into the mask whose bit l is set when
// all four lanes of column l % 16 said yes.  The folding runs on the scalar
// unit; the caller applies the mask with one v_cndmask per value.
__device__ __forceinline__ uint64_t column_all(uint64_t b) {
  uint64_t f = b & (b >> 16);
  f &= f >> 32;                        // bit c: lanes c, c+16, c+32, c+48 all set
  f &= 0xFFFFull;
  f |= f << 16;
  f |= f << 32;                        // replicated to every lane group
  return f;
}

// Lanes whose part of the block is all zero weights.  2-bit: every code is 1
// (bytes 0x55).  4-bit: every nibble equals the zero point z, which then has to
// be an integer in 0..15 (a zero point that is not an integer leaves no
// weight of the block at zero).
template <int DW>
__device__ __forceinline__ uint64_t q2_part_zero(const uint32_t (&w)[DW]) {
  // codes dwords compared in pairs as 64-bit values: one compare per 32 codes
  static_assert(DW % 2 == 0, "pairs of code dwords");
  uint64_t m = ~0ull;
#pragma unroll
  for (int i = 0; i < DW; i += 2)
    m &= __builtin_amdgcn_ballot_w64((((uint64_t)w[i + 1] << 32) | w[i]) == 0x5555555555555555ull);
  return m;
}
template <int DW>
__device__ __forceinline__ uint64_t q4_part_zero(const uint32_t (&w)[DW], float z) {
  // v = z when z is an integer in 0..15 (NaN clamps to 0 and then fails the compare).
  const uint32_t v = (uint32_t)__builtin_fminf(__builtin_fmaxf(z, 0.f), 15.f);
  const uint32_t pat = __builtin_amdgcn_perm(0u, v | (v << 4), 0x00000000u);   // the nibble in all eight places
  uint64_t m = __builtin_amdgcn_ballot_w64((float)v == z);
#pragma unroll
  for (int i = 0; i < DW; ++i) m &= __builtin_amdgcn_ballot_w64(w[i] == pat);
  return m;
}

// v with the lanes of `mask` set to 0 (bits of a float or of an f16 word).
__device__ __forceinline__ uint32_t zero_where(uint32_t v, uint64_t mask) {
  uint32_t r;
  asm("v_cndmask_b32_e64 %0, %1, 0, %2" : "=v"(r) : "v"(v), "s"(mask));
  return r;
}

// Exact split of an f16 value into bf16 hi + lo (8 + at most 3 significant bits).
__device__ __forceinline__ void f16_split_bf16(uint16_t h, uint16_t& hi, uint16_t& lo) {
  const float f = f16_to_f32(h);
  const uint32_t fb = __builtin_bit_cast(uint32_t, f);
  const float fh = __builtin_bit_cast(float, fb & 0xFFFF0000u);
  hi = (uint16_t)(fb >> 16);
  lo = (uint16_t)(__builtin_bit_cast(uint32_t, f - fh) >> 16);
}

// Exact bf16 limbs of two f16 values packed in a dword: the high limb is the
// upper half of each value's fp32 bits, the low limb the rest (at most three
// significant bits, exact in bf16).  Returned as packed bf16 pairs.
__device__ __forceinline__ uint32_t f16x2_bf16_hi(uint32_t h2) {
  const uint32_t f0 = __builtin_bit_cast(uint32_t, f16_to_f32((uint16_t)(h2 & 0xFFFFu)));
  const uint32_t f1 = __builtin_bit_cast(uint32_t, f16_to_f32((uint16_t)(h2 >> 16)));
  return __builtin_amdgcn_perm(f1, f0, 0x07060302u);
}
__device__ __forceinline__ uint32_t f16x2_bf16_lo(uint32_t h2) {
  const float f0 = f16_to_f32((uint16_t)(h2 & 0xFFFFu)), f1 = f16_to_f32((uint16_t)(h2 >> 16));
  const float l0 = f0 - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f0) & 0xFFFF0000u);
  const float l1 = f1 - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f1) & 0xFFFF0000u);
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, l1), __builtin_bit_cast(uint32_t, l0), 0x07060302u);
}

// Round fp32 to bf16 (nearest even; finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rn(float f) {
  const uint32_t b = __builtin_bit_cast(uint32_t, f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

}  // namespace q2dev
