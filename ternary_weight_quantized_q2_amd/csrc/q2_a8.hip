// q2_a8.hip - the Q2_0 linear with 8-bit activations, on the int8 matrix cores.
//
// The GPU path of the pages runs its activations through 8-bit quantisation
// ("We're Teaching Your Browser to Paint", section "The GPU driver, and the bug
// that looked like broken math").  Here each row of x is quantised
// symmetrically: s_m = max_k |x[m,k]| / 127 and q[m,k] = x[m,k] / s_m rounded
// half to even and clamped to [-127, 127].  With the Q2_0 weight (c - 1) d of
// a code c and block scale d (same page, section "The lucky break that wasn't
// luck"),
//
//   y[m,n] = s_m * sum_b d[n,b] * T[m,n,b],   T = sum over the block's 128 k of q[m,k] (c[n,k] - 1),
//
// and T is an integer of magnitude at most 127 * 128 (at most 2 * 127 * 128
// for a code 3, which the pack step never writes).  The int8 matrix-core
// instruction v_mfma_i32_16x16x64_i8 computes T exactly from the int8
// activation codes and the weights c - 1 in {-1, 0, 1}; the block scale is
// applied in fp32 per block and the row scale once in the epilogue.  An
// all-zero weight block gives T = 0 exactly, so it adds nothing.
#include "q2_device.h"
#include "q2_internal.h"
#include <algorithm>
#include <cmath>
#include <cstring>

namespace q2dev {

typedef int q2_i32x4 __attribute__((ext_vector_type(4)));

// ============================================================================
// Quantiser: bf16 [M, K] -> int8 codes [M, K] + row scales [M]
// ============================================================================
// One workgroup per row.  s = max |x| / 127 and code = round-half-even(x / s),
// clamped to [-127, 127], both with IEEE float32 division; a row of zeros has
// s = 0 and codes 0.  Each group of 16 consecutive codes is stored transposed
// as a 4 x 4 byte matrix, byte 4 j + i holding the code of element 4 i + j, so
// that byte j of a packed 2-bit code byte and byte j of a code dword line up
// (see wts_i8 below).  Thread t takes the 16-element groups t, t + 256, ...;
// the first QZ8_REG of them stay in registers between the maximum and the
// quantisation (rows up to 16384), so such a row is read from HBM once.
constexpr int QZ8_THREADS = 256;
constexpr int QZ8_REG = 4;

__device__ __forceinline__ float qz8_amax16(const q2_u32x4& v0, const q2_u32x4& v1, float amax) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    amax = fmaxf(amax, fabsf(__builtin_bit_cast(float, v0[d] << 16)));
    amax = fmaxf(amax, fabsf(__builtin_bit_cast(float, v0[d] & 0xFFFF0000u)));
    amax = fmaxf(amax, fabsf(__builtin_bit_cast(float, v1[d] << 16)));
    amax = fmaxf(amax, fabsf(__builtin_bit_cast(float, v1[d] & 0xFFFF0000u)));
  }
  return amax;
}

// Codes of 16 consecutive bf16 values, in the transposed byte order.
__device__ __forceinline__ q2_u32x4 qz8_codes16(const q2_u32x4& v0, const q2_u32x4& v1, float sc) {
  uint32_t q[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t h = (e < 8) ? v0[e >> 1] : v1[(e - 8) >> 1];
    const float xv = __builtin_bit_cast(float, (e & 1) ? (h & 0xFFFF0000u) : (h << 16));
    float cv = 0.f;
    if (sc > 0.f) cv = fminf(fmaxf(__builtin_rintf(xv / sc), -127.f), 127.f);
    q[e] = (uint32_t)(int)cv & 0xFFu;
  }
  q2_u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = q[j] | (q[4 + j] << 8) | (q[8 + j] << 16) | (q[12 + j] << 24);
  return o;
}

__global__ __launch_bounds__(QZ8_THREADS) void quantize_rows_i8_kernel(const uint16_t* x, uint8_t* xq,
                                                                       float* row_scale, int64_t K) {
  __shared__ float wmax[QZ8_THREADS / 64];
  const int64_t m = blockIdx.x;
  const uint16_t* xr = x + m * K;
  uint8_t* qr = xq + m * K;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int64_t STEP = 16 * QZ8_THREADS;
  q2_u32x4 v[QZ8_REG][2];
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < QZ8_REG; ++r) {                 // K is a multiple of 128
    const int64_t k = 16 * (int64_t)tid + r * STEP;
    if (k < K) {
      v[r][0] = *reinterpret_cast<const q2_u32x4*>(xr + k);
      v[r][1] = *reinterpret_cast<const q2_u32x4*>(xr + k + 8);
    } else {
      v[r][0] = v[r][1] = q2_u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int r = 0; r < QZ8_REG; ++r) amax = qz8_amax16(v[r][0], v[r][1], amax);
  for (int64_t k = 16 * (int64_t)tid + QZ8_REG * STEP; k < K; k += STEP)
    amax = qz8_amax16(*reinterpret_cast<const q2_u32x4*>(xr + k), *reinterpret_cast<const q2_u32x4*>(xr + k + 8),
                      amax);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) wmax[wv] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < QZ8_THREADS / 64; ++w) amax = fmaxf(amax, wmax[w]);
  const float sc = amax / 127.0f;
  if (tid == 0) row_scale[m] = sc;
#pragma unroll
  for (int r = 0; r < QZ8_REG; ++r) {
    const int64_t k = 16 * (int64_t)tid + r * STEP;
    if (k < K) *reinterpret_cast<q2_u32x4*>(qr + k) = qz8_codes16(v[r][0], v[r][1], sc);
  }
  for (int64_t k = 16 * (int64_t)tid + QZ8_REG * STEP; k < K; k += STEP)
    *reinterpret_cast<q2_u32x4*>(qr + k) = qz8_codes16(*reinterpret_cast<const q2_u32x4*>(xr + k),
                                                       *reinterpret_cast<const q2_u32x4*>(xr + k + 8), sc);
}

hipError_t launch_quantize_rows_i8(const uint16_t* x, uint8_t* xq, float* row_scale, int64_t M, int64_t K,
                                   hipStream_t stream) {
  if (M > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_rows_i8_kernel, dim3((unsigned)M), dim3(QZ8_THREADS), 0, stream, x, xq, row_scale, K);
  return hipGetLastError();
}

// ============================================================================
// int8 matrix-core GEMM
// ============================================================================
// Operand layout of v_mfma_i32_16x16x64_i8: lane l holds 16 int8 values of
// row l % 16 of A and of column l % 16 of B, for K slots chosen by l / 16;
// which 16 of the 64 K indices a lane's bytes stand for is free, as long as A
// and B agree.  Lane group g takes, in step t (0, 1) of a 128-block, the 16
// weights 32 g + 16 t .. 32 g + 16 t + 15: one dword of the packed codes (the
// lane reads its column's bytes 8 g .. 8 g + 7 of the block once) and one
// 16-byte group of the activation codes (group 2 g + t of the row's block).
//
// Weights c - 1 from a code dword: (w >> 2 j) & 0x03030303 puts code 4 i + j
// in byte i, and a byte permute through the table {-1, 0, 1, 2} maps c to
// c - 1 (a code 3 to 2, the weight 2 d the bf16 kernels give it too).  Dword j
// of the B fragment is then codes 4 i + j, matching the activation group's
// transposed byte order.
__device__ __forceinline__ q2_u32x4 wts_i8(uint32_t w) {
  const uint32_t tab = 0x020100FFu;                       // bytes -1, 0, 1, 2
  q2_u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_perm(tab, tab, (w >> (2 * j)) & 0x03030303u);
  return r;
}

__device__ __forceinline__ q2_i32x4 mfma_i8(q2_u32x4 a, q2_u32x4 b, q2_i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(q2_i32x4, a), __builtin_bit_cast(q2_i32x4, b), c,
                                               0, 0, 0);
}

// Activation stage: BM rows of 128 bytes (a row's block), chunk q of row r at
// position q ^ a8_swz(r).  A fragment read has lane (c, g) read chunk 2 g + t
// of row c.  Measured on gfx950, a 16-byte LDS read serves 16 lanes per pass
// from 64 four-byte banks, a pass taking lanes c in quads {0, 3} of one lane
// group and quads {1, 2} of the next (lane groups 0 / 1 and 2 / 3 pair up):
// with the swizzle below the 16 lanes of every pass hit 16 distinct 16-byte
// bank slots (address bits 4..7), and so do the 16 lanes of each lane group.
// (The plain q ^ (r >> 1) measured 1.45 times the conflict-free read time.)
__device__ __forceinline__ int a8_swz(int r) {
  return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 2);
}

constexpr int cmax3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

// Structure as in the bf16 K-group kernel: a workgroup of KG groups of four
// waves owns a BM x BN tile (BM = 16 MT, BN = 64 NT); wave w computes the
// columns w & 3 of the tile from blocks KG s + (w >> 2) of each set s of KG
// consecutive blocks, and the KG partial sums are added in group order through
// LDS at the end.  Every operand moves HBM -> LDS with direct global-to-LDS
// copies into a ring of NSET sets; the copies of set s + NSET - 1 are issued
// during set s, spread over its row tiles.  No row sums are needed: the
// weights c - 1 are decoded signed.
template <int MT, int NT, int KG, int NSET>
__global__ __launch_bounds__(256 * KG) void gemm_a8_kernel(A8Args a, int tiles_m, int group_m, int kpart) {
  constexpr int W = 4 * KG;                                   // waves
  constexpr int BM = 16 * MT, BN = 64 * NT;
  constexpr int XSTAGE = BM * 128;                            // one activation block
  constexpr int CPB = 2 * BN;                                 // 16-byte code chunks per block
  constexpr int CODE_SLOT = CPB * 16;
  constexpr int SWORDS = 4 * BN;                              // bytes of scale words per block
  constexpr int WSTAGE = CODE_SLOT + SWORDS;
  constexpr int NST = NSET * KG;                              // block stages of the ring
  constexpr int OFF_W = NST * XSTAGE;
  constexpr int RING = OFF_W + NST * WSTAGE;
  constexpr int OS = BN + 4;                                  // output tile row stride (floats)
  constexpr int SMEM = cmax3(RING, (KG - 1) * BM * BN * 4, BM * OS * 4);
  constexpr int NTASK = KG * MT;                              // 16-row activation tiles per set
  constexpr int XT = (NTASK + W - 1) / W;                     // tasks per wave (at most)
  constexpr int XUM = 2 * XT;                                 // activation copy units per wave
  constexpr int CINS = KG * CPB / 64;                         // 64-chunk code copies per set
  constexpr int CU = (CINS + W - 1) / W;                      // code copies per wave
  constexpr int NWU = CU + 1;                                 // weight copies per wave (codes, scale words)
  constexpr int NU = XUM + NWU;
  constexpr int UPT = (NU + MT - 1) / MT;                     // copy units issued per row tile
  static_assert(NSET == 2 || NSET == 3, "ring depth");
  static_assert(XT <= 2, "activation tasks per wave");
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wv & 3, kg = wv >> 2;
  const int c = lane & 15, g = lane >> 4;
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  // With kpart > 0 the K blocks are split in two parts of kpart blocks: the
  // two workgroups of a tile take one part each (adjacent numbers, so one XCD)
  // and add their results into y, which the launcher has zeroed.
  const int nparts = kpart > 0 ? 2 : 1;
  int tile = xcd_tile((int)blockIdx.x, tiles_m * tiles_n * nparts);
  const int part = tile & (nparts - 1);
  tile = tile >> (nparts - 1);
  const int grp = tile / (group_m * tiles_n), gi = tile - grp * group_m * tiles_n;
  const int gm = min(group_m, tiles_m - grp * group_m);          // row tiles in this group
  const int tm = grp * group_m + gi % gm, tn = gi / gm;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t nw = n0 + wn * (BN / 4);
  const int64_t M = a.M, N = a.N, K = a.K, KB = K / BLOCK_K;
  const int kb0 = part * kpart;                                  // this workgroup takes blocks kb0 .. kb - 1
  const int kb = kpart > 0 ? min((int)KB, kb0 + kpart) : (int)KB;
  const int NS = kb > kb0 ? (kb - kb0 + KG - 1) / KG : 0;       // sets
  const int64_t row_bytes = K / 4;

  // ---- copy sources.  Task t of a set is row tile t % MT of block t / MT;
  // wave wv owns tasks wv, wv + W, ...  Copy kk (0, 1) of a task fills tile
  // rows 8 kk .. 8 kk + 7; lane l covers row 8 kk + (l >> 3), position l & 7,
  // which holds chunk (l & 7) ^ a8_swz(row).  Rows past M are clamped to M - 1.
  int xtasks = 0;
#pragma unroll
  for (int k2 = 0; k2 < XT; ++k2) xtasks += (wv + W * k2 < NTASK) ? 1 : 0;
  const int set_units = 2 * xtasks + NWU;                     // copies this wave issues per set
  uint32_t xoff[XT][2];
#pragma unroll
  for (int k2 = 0; k2 < XT; ++k2) {
    const int it = (wv + W * k2) % MT;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int rin = 8 * kk + (lane >> 3);
      int64_t gr = m0 + 16 * it + rin;
      gr = gr < M ? gr : M - 1;
      xoff[k2][kk] = (uint32_t)((gr - m0) * K) + (uint32_t)(((lane & 7) ^ a8_swz(rin)) << 4);
    }
  }
  // Code copy v of wave wv: copy index ci = v * W + wv of the set (clamped to
  // the last one, which is then copied twice with identical bytes), block
  // ci * 64 / CPB, chunks from (ci * 64) % CPB of that block.  LDS bytes
  // col * 32 + 16 h hold the column's 16-byte half h ^ ((col >> 2) & 1).
  uint32_t woff[CU];
#pragma unroll
  for (int v = 0; v < CU; ++v) {
    int ci = v * W + wv;
    ci = ci < CINS ? ci : CINS - 1;
    const int pos = (ci * 64) % CPB + lane;
    const int col = pos >> 1;
    const int unit = ((pos & 1) ^ ((col >> 2) & 1)) << 4;
    const int64_t gc = (n0 + col < N) ? col : N - 1 - n0;
    woff[v] = (uint32_t)(gc * row_bytes + unit);
  }
  // Scale words: the waves of group kg cover block kg of the set, wave wn the
  // columns sq * 64 + lane with sq = min(wn, NT - 1).  Each scale is copied as
  // the aligned word that holds it, through a resource based 4 bytes below the
  // tile's first scale: with h the half-word position of the column's block-0
  // scale, the word of block blk sits at so_e (blk even) or so_o (blk odd)
  // plus 2 blk.
  const int sq = wn < NT ? wn : NT - 1;
  const int64_t ncols = (N - n0) < BN ? (N - n0) : BN;
  int64_t sgc = sq * 64 + lane;
  sgc = sgc < ncols ? sgc : ncols - 1;
  const uint32_t svl = (uint32_t)(2 * sgc * KB);
  const uint32_t sbytes = (uint32_t)(2 * ncols * KB + 8);
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(reinterpret_cast<const uint8_t*>(a.s + n0 * KB) - 4, sbytes);
  const uint32_t sh = (uint32_t)(((uintptr_t)(a.s + n0 * KB) + svl) >> 1) & 1u;
  const uint32_t so_e = svl + 4 - 2 * sh, so_o = svl + 2 + 2 * sh;
  const int64_t nrows = (M - m0) < BM ? (M - m0) : BM;
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(a.xq + m0 * K, (uint32_t)(nrows * K));
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(a.w + n0 * row_bytes, (uint32_t)(ncols * row_bytes));

  // ---- read side
  int aoff[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) aoff[t] = c * 128 + (((2 * g + t) ^ a8_swz(c)) << 4);
  const int coff = c * 32 + ((((g >> 1) ^ ((c >> 2) & 1)) << 4) | ((g & 1) << 3));
  uint32_t shalf = 0;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int64_t r = nw + 16 * j + c;
    r = r < N ? r : N - 1;
    shalf |= (uint32_t)((((uintptr_t)(a.s + r * KB)) >> 1) & 1) << j;
  }

  // Copies of set `set` into ring slot `slot`, one unit at a time: units
  // 0 .. XUM-1 the activation copies of this wave's tasks, then the codes and
  // the scale words.  Blocks past the end re-copy the last one.
  auto issue_unit = [&](int unit, int set, int slot) {
    const int b0 = kb0 + KG * set;
    if (unit < XUM) {
      const int k2 = unit >> 1, kk = unit & 1;
      if (k2 < xtasks) {
        const int task = wv + W * k2;
        const int q = task / MT, it = task - q * MT;
        int blk = b0 + q;
        blk = blk < kb ? blk : kb - 1;
        const uint32_t xo = xoff[k2][kk];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (lds_void*)(smem + (slot * KG + q) * XSTAGE + (16 * it + 8 * kk) * 128), 16, xo,
            (uint32_t)blk * 128u, 0, 0);
      }
    } else if (unit < XUM + CU) {
      const int v = unit - XUM;
      int ci = v * W + wv;                                     // uniform
      ci = ci < CINS ? ci : CINS - 1;
      const int q = ci * 64 / CPB;
      int blk = b0 + q;
      blk = blk < kb ? blk : kb - 1;
      const uint32_t wo = woff[v];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (lds_void*)(smem + OFF_W + (slot * KG + q) * WSTAGE + ((ci * 64) % CPB) * 16), 16, wo,
          (uint32_t)blk * 32u, 0, 0);
    } else {
      int blk = b0 + kg;
      blk = blk < kb ? blk : kb - 1;
      const int dst = OFF_W + (slot * KG + kg) * WSTAGE + CODE_SLOT + sq * 256;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(smem + dst), 4, (blk & 1) ? so_o : so_e,
                                               2u * (uint32_t)blk, 0, 0);
    }
  };
  auto issue_set = [&](int set, int slot) {
    for (int un = 0; un < NU; ++un) issue_unit(un, set, slot);
  };
  // Wait until at most n of this wave's copies are in flight (n is uniform and
  // one of the per-set counts).
  auto wait_copies = [&](int n) {
    asm volatile("" ::: "memory");
    if (n == 0) {
      __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));
    } else if (n == NWU) {
      __builtin_amdgcn_s_waitcnt((NWU & 15) | (7 << 4) | (15 << 8) | ((NWU >> 4) << 14));
    } else if (n == NWU + 2) {
      __builtin_amdgcn_s_waitcnt(((NWU + 2) & 15) | (7 << 4) | (15 << 8) | (((NWU + 2) >> 4) << 14));
    } else {
      __builtin_amdgcn_s_waitcnt(((NWU + 4) & 15) | (7 << 4) | (15 << 8) | (((NWU + 4) >> 4) << 14));
    }
    asm volatile("" ::: "memory");
  };

  q2_f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = q2_f32x4{0.f, 0.f, 0.f, 0.f};

  // Weights of one block for this wave's columns (from its weight stage).
  auto decode = [&](const uint8_t* wst, int blk, q2_u32x4 (&bf)[NT][2], float (&dc)[NT]) {
    const uint32_t pmask = (uint32_t)(blk & 1) ? 0xFFu : 0u;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int col0 = wn * (BN / 4) + 16 * j;
      const q2_u32x2 v = *reinterpret_cast<const q2_u32x2*>(wst + col0 * 32 + coff);
      bf[j][0] = wts_i8(v[0]);
      bf[j][1] = wts_i8(v[1]);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(wst + CODE_SLOT + (col0 + c) * 4);
      dc[j] = f16_to_f32((uint16_t)(sw >> ((((shalf ^ pmask) >> j) & 1) * 16)));
    }
  };
  // Matrix-core steps of one block over the staged activations `st`; the
  // copies of set `cset` (if >= 0) are issued UPT units per row tile.
  auto mainblk = [&](const uint8_t* st, const q2_u32x4 (&bf)[NT][2], const float (&dc)[NT], int cset, int cslot) {
    q2_u32x4 a0[2], a1[2];
    auto rd = [&](int i, q2_u32x4 (&av)[2]) {
#pragma unroll
      for (int t = 0; t < 2; ++t) av[t] = *reinterpret_cast<const q2_u32x4*>(st + i * 2048 + aoff[t]);
    };
    auto tile = [&](int i, const q2_u32x4 (&av)[2]) {
      q2_i32x4 tmp[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) tmp[j] = mfma_i8(av[0], bf[j][0], q2_i32x4{0, 0, 0, 0});
#pragma unroll
      for (int j = 0; j < NT; ++j) tmp[j] = mfma_i8(av[1], bf[j][1], tmp[j]);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(dc[j], (float)tmp[j][e], acc[i][j][e]);
    };
    rd(0, a0);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (cset >= 0) {
#pragma unroll
        for (int un = UPT * i; un < UPT * i + UPT; ++un)
          if (un < NU) issue_unit(un, cset, cslot);
      }
      if (i & 1) {
        if (i + 1 < MT) rd(i + 1, a0);
        tile(i, a1);
      } else {
        if (i + 1 < MT) rd(i + 1, a1);
        tile(i, a0);
      }
    }
  };

  // Set s sits in ring slot s % NSET.  At the top of set s every wave has
  // waited for its own copies of set s (with NSET = 3 the copies of set s + 1
  // may still be in flight); the barrier publishes them and marks set s - 1
  // done, so its slot receives the copies of set s + NSET - 1 during set s.
  if (NS > 0) {
    issue_set(0, 0);
    if constexpr (NSET == 3) {
      if (NS > 1) issue_set(1, 1);
    }
    int slot = 0;
    for (int s = 0; s < NS; ++s) {
      if constexpr (NSET == 3) {
        wait_copies(s + 1 < NS ? set_units : 0);
        stage_barrier<63>();
      } else {
        stage_barrier<0>();
      }
      const int cset = (s + NSET - 1 < NS) ? s + NSET - 1 : -1;       // the set copied during this one
      const int cslot = (slot + NSET - 1 >= NSET) ? slot - 1 : slot + NSET - 1;   // (s + NSET - 1) % NSET
      const int bp = kb0 + KG * s + kg;
      if (bp < kb) {
        q2_u32x4 bf[NT][2];
        float dc[NT];
        decode(smem + OFF_W + (slot * KG + kg) * WSTAGE, bp, bf, dc);
        mainblk(smem + (slot * KG + kg) * XSTAGE, bf, dc, cset, cslot);
      } else if (cset >= 0) {
        issue_set(cset, cslot);
      }
      slot = (slot + 1 == NSET) ? 0 : slot + 1;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);          // every copy of this wave has landed
  __syncthreads();                        // and every wave is done reading the stages

  // Partial sums of groups 1 .. KG-1 -> LDS -> added in group order by group 0.
  const bool split = kpart > 0;
  const bool rows16 = !split && (N & 3) == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
  float* const red = reinterpret_cast<float*>(smem);
  constexpr int PART = MT * NT * 4 * 64;  // floats per wave
  if (kg > 0) {
    float* const mine = red + ((kg - 1) * 4 + wn) * PART;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) mine[((i * NT + j) * 4 + e) * 64 + lane] = acc[i][j][e];
  }
  __syncthreads();
  if (kg == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = acc[i][j][e];
#pragma unroll
          for (int q = 1; q < KG; ++q) v += red[(((q - 1) * 4 + wn) * PART) + ((i * NT + j) * 4 + e) * 64 + lane];
          acc[i][j][e] = v;
        }
  }
  if (rows16) {
    // The finished tile goes through LDS (rows padded to OS floats) and is
    // stored as 16-byte pieces of contiguous rows, times the row scale.
    constexpr int RP = (BM * (BN / 4) + 64 * W - 1) / (64 * W);
    __syncthreads();                      // the partial sums are read; their space takes the tile
    float* const out = reinterpret_cast<float*>(smem);
    if (kg == 0) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) out[(16 * i + 4 * g + e) * OS + wn * (BN / 4) + 16 * j + c] = acc[i][j][e];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < RP; ++t) {
      int row, q;
      if (row_piece<BM, BN, 64 * W>(t, tid, (int)nrows, (int)ncols, row, q)) {
        q2_f32x4 v = *reinterpret_cast<const q2_f32x4*>(&out[row * OS + 4 * q]);
        v *= a.row_scale[m0 + row];
        __builtin_nontemporal_store(v, reinterpret_cast<q2_f32x4*>(&a.y[(m0 + row) * N + n0 + 4 * q]));
      }
    }
  } else if (kg == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + 16 * i + 4 * g + e;
        const float rsc = m < M ? a.row_scale[m] : 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int64_t n = nw + 16 * j + c;
          const float v = acc[i][j][e] * rsc;
          if (m < M && n < N) {
            if (split) unsafeAtomicAdd(&a.y[m * N + n], v);
            else __builtin_nontemporal_store(v, &a.y[m * N + n]);
          }
        }
      }
    }
  }
}

// ============================================================================
// Launch
// ============================================================================
// Row tiles per group of the XCD tile order: as for the bf16 K-group kernels,
// the power of two p (at most the row-tile count) that minimises the modelled
// HBM reads, 8 XCDs x their x rows (again every round once those rows exceed
// ~2.5 MB of the 4 MB L2) plus p times the weights.
static int a8_group_rows(const A8Args& a, int bm, int tiles_m, int tiles_n, int nparts) {
  const double xrow = (double)std::min<int64_t>(bm, a.M) * (double)a.K;     // one row tile of codes
  const double wb = (double)a.N * (double)a.K * 0.265625;
  const double rounds = std::max(1.0, std::ceil((double)tiles_m * tiles_n * nparts / 8.0 / 32.0));
  auto cost = [&](int p) {
    const int group = (tiles_m + p - 1) / p;
    const double xpart = group * xrow;
    return 8.0 * xpart * (xpart <= 2.5e6 ? 1.0 : rounds) + p * wb;
  };
  int best = 1;
  for (int p = 2; p <= 8 && p <= tiles_m; p *= 2)
    if (cost(p) < cost(best)) best = p;
  return (tiles_m + best - 1) / best;
}

template <int MT, int NT, int KG, int NSET>
static hipError_t run_a8(const A8Args& a, int ksplit, hipStream_t stream) {
  constexpr int BM = 16 * MT, BN = 64 * NT;
  const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int64_t KB = a.K / BLOCK_K;
  if (ksplit != 1 && ksplit != 2) return hipErrorInvalidValue;
  const int kpart = (ksplit == 2) ? (int)((KB + 1) / 2) : 0;
  const int64_t grid = tiles_m * tiles_n * (kpart > 0 ? 2 : 1);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (kpart > 0) {
    const hipError_t e = launch_zero_y(a.y, a.M * a.N, stream);
    if (e != hipSuccess) return e;
  }
  const int group_m = a8_group_rows(a, BM, (int)tiles_m, (int)tiles_n, kpart > 0 ? 2 : 1);
  hipLaunchKernelGGL((gemm_a8_kernel<MT, NT, KG, NSET>), dim3((unsigned)grid), dim3(256 * KG), 0, stream, a,
                     (int)tiles_m, group_m, kpart);
  return hipGetLastError();
}

// int8 GEMM configurations: MT x NT x KG (tile 16 MT x 64 NT, KG groups of
// four waves), ring depth 2 unless named r3.  Tests and profiling can force
// any of them by name.
static const char* const kA8CfgNames[] = {"auto",     "a8_6x3x2", "a8_4x2x2",   "a8_2x2x2",   "a8_2x1x4",
                                          "a8_1x2x4", "a8_1x1x4", "a8_8x3x2",   "a8_6x3x1r3", "a8_4x4x2",
                                          "a8_6x3x2r3", "a8_4x2x4", "a8_6x2x2", "a8_4x3x2"};
enum A8Cfg { A8_AUTO, A8_6x3x2, A8_4x2x2, A8_2x2x2, A8_2x1x4, A8_1x2x4, A8_1x1x4, A8_8x3x2, A8_6x3x1R3,
             A8_4x4x2, A8_6x3x2R3, A8_4x2x4, A8_6x2x2, A8_4x3x2, A8_COUNT };
static_assert(sizeof kA8CfgNames / sizeof kA8CfgNames[0] == A8_COUNT, "configuration names");

int a8_config_id(const char* name) {
  for (int i = 0; i < A8_COUNT; ++i)
    if (std::strcmp(name, kA8CfgNames[i]) == 0) return i;
  return -1;
}

static hipError_t run_a8_cfg(const A8Args& a, int cfg, int ksplit, hipStream_t stream) {
  switch (cfg) {
    case A8_6x3x2: return run_a8<6, 3, 2, 2>(a, ksplit, stream);
    case A8_4x2x2: return run_a8<4, 2, 2, 2>(a, ksplit, stream);
    case A8_2x2x2: return run_a8<2, 2, 2, 2>(a, ksplit, stream);
    case A8_2x1x4: return run_a8<2, 1, 4, 2>(a, ksplit, stream);
    case A8_1x2x4: return run_a8<1, 2, 4, 2>(a, ksplit, stream);
    case A8_1x1x4: return run_a8<1, 1, 4, 2>(a, ksplit, stream);
    case A8_8x3x2: return run_a8<8, 3, 2, 2>(a, ksplit, stream);
    case A8_6x3x1R3: return run_a8<6, 3, 1, 3>(a, ksplit, stream);
    case A8_4x4x2: return run_a8<4, 4, 2, 2>(a, ksplit, stream);
    case A8_6x3x2R3: return run_a8<6, 3, 2, 3>(a, ksplit, stream);
    case A8_4x2x4: return run_a8<4, 2, 4, 2>(a, ksplit, stream);
    case A8_6x2x2: return run_a8<6, 2, 2, 2>(a, ksplit, stream);
    case A8_4x3x2: return run_a8<4, 3, 2, 2>(a, ksplit, stream);
    default: return hipErrorInvalidValue;
  }
}

// Automatic choice: the widest tile whose workgroup count still covers a good
// part of the chip; long K over few tiles splits the K blocks in two.
static int a8_auto_cfg(const A8Args& a, int& ksplit) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  const int64_t KB = a.K / BLOCK_K;
  ksplit = 1;
  int cfg;
  if (a.M <= 16) cfg = tiles(16, 128) >= 128 ? A8_1x2x4 : A8_1x1x4;
  else if (a.M <= 64) cfg = tiles(32, 128) >= 128 ? A8_2x2x2 : A8_2x1x4;
  else if (a.M <= 256) cfg = tiles(64, 128) >= 128 ? A8_4x2x2 : A8_2x2x2;
  else cfg = tiles(96, 192) >= 160 ? A8_6x3x2 : A8_4x2x2;
  if (KB >= 64) {
    const int bm = cfg == A8_6x3x2 ? 96 : cfg == A8_4x2x2 ? 64 : cfg == A8_1x2x4 || cfg == A8_1x1x4 ? 16 : 32;
    const int bn = cfg == A8_6x3x2 ? 192 : (cfg == A8_2x1x4 || cfg == A8_1x1x4) ? 64 : 128;
    if (tiles(bm, bn) < 256) ksplit = 2;
  }
  return cfg;
}

hipError_t launch_linear_a8(const A8Args& a, int force_cfg, int force_ksplit, hipStream_t stream) {
  int ksplit = 1;
  int cfg = a8_auto_cfg(a, ksplit);
  if (force_cfg > 0) {
    cfg = force_cfg;
    ksplit = 1;
  }
  if (force_ksplit > 0) ksplit = force_ksplit;
  return run_a8_cfg(a, cfg, ksplit, stream);
}

}  // namespace q2dev
