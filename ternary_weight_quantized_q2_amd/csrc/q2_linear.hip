// q2_linear.hip - the Q2_0 ternary linear (and the 4-bit variant) on CDNA4.
//
// y = x W^T for packed weights; every operand of the GEMMs reaches LDS through
// direct copies, the weights are decoded into bf16 matrix-core operands by a
// magic-number OR, and 16x16x32 bf16 MFMAs accumulate each 128-wide block
// from a start value of -1.25 (or -(1 + z/16)) times the block's row sums,
// after which one FMA per output applies the block's f16 scale.
//  * gemm_kgroup_kernel (M > 16, any raggedness, the rank-r branch up to
//    r = 64 in its prologue): KG groups of four waves on a 16 MT x 64 NT tile,
//    the groups taking alternate K blocks of the same output columns and
//    summed once at the end, in XCD-contiguous tile order, optionally with
//    the K blocks split over two workgroups.
//  * gemm_kernel (the rank-r branch above r = 64 or with the 4-bit format,
//    narrow mid-size outputs): four waves splitting N, one block per barrier.
//  * gemv_kernel (M <= 16): a workgroup owns 16 weight rows; its waves split
//    K, stream the codes with coalesced loads, transpose them through LDS into
//    the matrix-core layout and finish with a fixed-order reduction.
//  * lowrank_t_kernel: x A^T once per call, as bf16 hi/lo limbs, for the
//    branch y += (x A^T) B^T that the GEMMs and the GEMV add into their
//    accumulators (the K-group kernel in its prologue, the four-wave kernel
//    after its last block, the GEMV in one wave while the others stream).
//
// Every summation order is fixed, so results are bitwise reproducible.  The
// GEMMs write y with non-temporal stores: the fp32 outputs (tens of MB) would
// otherwise push the activations and weights that later tiles re-read out of
// the caches.
#include "q2_device.h"
#include "q2_internal.h"
#include <algorithm>
#include <cmath>
#include <cstring>

namespace q2dev {

template <int FMT> struct WFmt;
template <> struct WFmt<0> {           // Q2_0: 32 bytes of codes per row and block
  static constexpr int BLOCK_BYTES = 32;
  static constexpr int LANE_DW = 2;    // lane group g holds dwords 2g, 2g+1
};
template <> struct WFmt<1> {           // 4-bit: 64 bytes per row and group
  static constexpr int BLOCK_BYTES = 64;
  static constexpr int LANE_DW = 4;    // lane group g holds dwords 4g .. 4g+3
};

template <int FMT>
__device__ __forceinline__ void decode_block(const uint32_t (&w)[WFmt<FMT>::LANE_DW], q2_u32x4 (&bf)[4],
                                             DecodeConsts k) {
  if constexpr (FMT == 0) {
    bf[0] = q2_bfrag<0>(w[0], k);
    bf[1] = q2_bfrag<1>(w[0], k);
    bf[2] = q2_bfrag<0>(w[1], k);
    bf[3] = q2_bfrag<1>(w[1], k);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) bf[t] = q4_bfrag(w[t], k);
  }
}

// Accumulator start value of a block from the staged, pre-scaled block sum
// s4 (-1.25 S for 2-bit, -S for 4-bit): 2-bit -1.25 S, 4-bit -(1 + z/16) S.
template <int FMT>
__device__ __forceinline__ q2_f32x4 block_cinit(q2_f32x4 s4, float zp) {
  if constexpr (FMT == 0) {
    return s4;
  } else {
    const float k = 1.f + zp * 0.0625f;
    return q2_f32x4{k * s4[0], k * s4[1], k * s4[2], k * s4[3]};
  }
}

// Scale d (and zero point z) of one (weight row, block) of the matrix-core
// layout from the bits that hold them (in the low half), with d = 0 when every
// weight of the block is zero: such a block then adds exactly nothing, where
// its offset-started sum would leave rounding noise.  w is this lane's part of
// the block's codes; all lanes of the wave must call this together.
template <int FMT>
__device__ __forceinline__ void block_scale(const uint32_t (&w)[WFmt<FMT>::LANE_DW], uint32_t sbits,
                                            uint32_t zbits, float& dc, float& zc) {
  zc = (FMT == 1) ? f16_to_f32((uint16_t)zbits) : 0.f;
  uint64_t pz;
  if constexpr (FMT == 0) pz = q2_part_zero(w);
  else pz = q4_part_zero(w, zc);
  dc = f16_to_f32((uint16_t)zero_where(sbits, column_all(pz)));
}

template <int FMT>
__device__ __forceinline__ void stage_pairs(const uint32_t (&nx)[8], uint32_t (&pr)[8]) {
  if constexpr (FMT == 0) q2_xpairs(nx, pr);
  else q4_xpairs(nx, pr);
}

// 16 activations (32 bytes) of one row; `row` must be a valid row.
__device__ __forceinline__ void load_x16(const uint16_t* x, int64_t row, int64_t K, int64_t k0, uint32_t (&nx)[8]) {
  const q2_u32x4* p = reinterpret_cast<const q2_u32x4*>(x + row * K + k0);
  const q2_u32x4 v0 = p[0], v1 = p[1];
  nx[0] = v0[0]; nx[1] = v0[1]; nx[2] = v0[2]; nx[3] = v0[3];
  nx[4] = v1[0]; nx[5] = v1[1]; nx[6] = v1[2]; nx[7] = v1[3];
}

// Sum over 8 consecutive lanes with DPP moves (no LDS traffic); the total is
// exact in the lane with (lane & 7) == 0, in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum8_lanes(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x104>(v);   // row_shl:4 (lane i reads lane i + 4)
  return v;
}

// ---- low-rank operands -----------------------------------------------------
// The limbs of x A^T are stored [M, 2 r8] (hi | lo), r8 = r rounded up to a
// multiple of 8, the padding columns zero, so every row and both halves start
// on a 16-byte boundary.
__host__ __device__ __forceinline__ int lr_pad(int r) { return (r + 7) & ~7; }

// A'' = [T_hi, T_hi, T_lo] (row m of the limbs), B'' = [B_hi, B_lo, B_hi] (row n of B),
// so sum_q A''[m,q] B''[n,q] = T_hi B_hi + T_hi B_lo + T_lo B_hi.  With r % 8 == 0 the
// eight elements of a lane group lie in one part and one aligned 16-byte run.
__device__ __forceinline__ q2_u32x4 lr_afrag(const uint16_t* tl, int64_t m, int r, int q0, bool vec) {
  if (q0 >= 3 * r) return q2_u32x4{0u, 0u, 0u, 0u};
  const int rs = lr_pad(r);
  if (vec) {
    const int part = q0 / r, jj = q0 - part * r;
    return *reinterpret_cast<const q2_u32x4*>(tl + m * 2 * rs + (part == 2 ? rs : 0) + jj);
  }
  uint32_t e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = q0 + k;
    uint32_t v = 0;
    if (q < 3 * r) {
      const int part = q / r, jj = q - part * r;
      v = tl[m * 2 * rs + (part == 2 ? rs : 0) + jj];
    }
    e[k] = v;
  }
  return q2_u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
}

__device__ __forceinline__ q2_u32x4 lr_bfrag(const uint16_t* B, int64_t n, int r, int q0, bool vec) {
  if (q0 >= 3 * r) return q2_u32x4{0u, 0u, 0u, 0u};
  uint16_t h[8];
  const int part0 = q0 / r;
  if (vec) {
    const int jj = q0 - part0 * r;
    const q2_u32x4 v = *reinterpret_cast<const q2_u32x4*>(B + n * r + jj);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      h[2 * d] = (uint16_t)(v[d] & 0xFFFFu);
      h[2 * d + 1] = (uint16_t)(v[d] >> 16);
    }
  }
  uint32_t e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = q0 + k;
    uint32_t v = 0;
    if (q < 3 * r) {
      const int part = vec ? part0 : q / r;
      const uint16_t hv = vec ? h[k] : B[n * r + (q - part * r)];
      uint16_t hi, lo;
      f16_split_bf16(hv, hi, lo);
      v = (part == 1) ? lo : hi;
    }
    e[k] = v;
  }
  return q2_u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
}

// ============================================================================
// GEMM, M > 16
// ============================================================================
// With LR, the four-wave kernel copies the workgroup's rows of the low-rank
// limbs x A^T and its columns of B into LDS in the prologue, so the extra MFMA
// steps after its last block never wait on global memory (r <= LR_RMAX,
// r % 8 == 0).  The K-group kernel takes the branch up to the same rank.
constexpr int LR_RMAX = 64;

// Chunk swizzle of an activation row: chunk q of row r sits at position
// q ^ row_swz(r), row_swz a bit rotation of r mod 16.  Plain q ^ (r & 15) is
// conflict-free for 16 lanes in isolation but measured at two thirds of the
// LDS read rate of the rotated form for the 64-lane fragment reads.
__device__ __forceinline__ int row_swz(int r) { return ((r >> 2) & 3) | ((r & 3) << 2); }

template <int FMT>
__device__ __forceinline__ void decode_block_nat(const uint32_t (&w)[WFmt<FMT>::LANE_DW], q2_u32x4 (&bf)[4],
                                                 const NatConsts& k) {
  if constexpr (FMT == 0) {
    bf[0] = q2_bfrag_nat<0>(w[0], k);
    bf[1] = q2_bfrag_nat<1>(w[0], k);
    bf[2] = q2_bfrag_nat<0>(w[1], k);
    bf[3] = q2_bfrag_nat<1>(w[1], k);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) bf[t] = q4_bfrag_nat(w[t], k);
  }
}

// A workgroup owns a BM x BN output tile; its four waves split it along N
// (BM x BN/4 each), so every wave decodes only its own weight columns and the
// activation tile in LDS is shared by all four.
//
// K-slot assignment of the 16x16x32 MFMA: in K step t of a 128-block, lane
// group g covers k = 32g + 8t .. 32g + 8t + 7.  The activation fragment is then
// one 16-byte chunk of a row (chunk 4g + t), and the lane's weight codes for
// the whole block are 8 contiguous bytes (2-bit) or 16 (4-bit).
//
// Every operand moves HBM -> LDS with direct global-to-LDS copies (no
// registers, no VALU): activations into a ring of XS block buffers, weight
// codes, scales and zero points into a ring of 3.  Since the main loop issues
// no other vector-memory loads, the only waits are the explicit ones in
// stage_barrier.  Activation chunks are XOR-swizzled per row (row_swz) so
// fragment reads run at the full LDS rate; weight units are swizzled too.
// A scale or zero point is copied as the 4-byte word that holds it (aligned
// down; the word never leaves the 16-byte granule of the value), so the copies
// need no alignment beyond the element's.
//
// Per block the accumulator of each 16x16 tile starts at -1.25 * S (2-bit) or
// -(1 + z/16) * S (4-bit), S the block's row sums of x.  S of block b+1 is
// computed during block b with matrix-core steps against a constant B operand
// (-1.25 resp. -1 in every element), split over the waves by 16-row tile, and
// handed over in LDS.
template <int FMT, int BM, int BN, bool LR>
__global__ __launch_bounds__(256) void gemm_kernel(LinearArgs a, int tiles_m, int lr_vec) {
  constexpr int MT = BM / 16;            // 16-row tiles per wave
  constexpr int NT = BN / 64;            // 16-column tiles per wave (4 waves along N)
  constexpr int DW = WFmt<FMT>::LANE_DW;
  constexpr int BBYTES = WFmt<FMT>::BLOCK_BYTES;
  constexpr int XS = LR ? 3 : 4;         // activation ring: b, b+1 (row sums), in-flight
  constexpr int WS = 3;                  // weight ring: b, b+1, b+2
  constexpr int XSTAGE = BM * 256;       // bytes per activation block
  constexpr int CU = (FMT == 0) ? (BN * 2 + 255) / 256 : BN / 64;   // 16-byte code copies per thread per block
  constexpr int CODE_BYTES = CU * 4096;  // code chunk slots of a weight stage (2-bit: padded past BN * 32)
  constexpr int WSTAGE = CODE_BYTES + ((FMT == 0) ? 1024 : 2048);   // codes + 256 scale [+ 256 zero] words
  constexpr int XU = BM / 16;            // activation copies (16 B) per thread per block
  constexpr int WU = CU + ((FMT == 0) ? 1 : 2);        // all weight copies per thread per block
  static_assert(BM % 16 == 0 && BN % 64 == 0 && BN <= 256, "tile shape");

  // One shared array carved by hand.  (With several LDS objects the compiler
  // tracks the copies per object and drains them before every read of that
  // object; the ordering here is explicit in stage_barrier instead.)
  constexpr int LRM = LR ? BM : 0, LRN = LR ? BN : 0;
  constexpr int OFF_W = XS * XSTAGE;
  constexpr int OFF_S = OFF_W + WS * WSTAGE;
  constexpr int OFF_LT = OFF_S + 2 * BM * 4;
  constexpr int OFF_LB = OFF_LT + LRM * 2 * LR_RMAX * 2;
  constexpr int SMEM = OFF_LB + LRN * LR_RMAX * 2;
  __shared__ __align__(16) uint8_t smem[SMEM];
  uint8_t* const xs = smem;
  uint8_t* const wsm = smem + OFF_W;
  float (*const ss)[BM] = reinterpret_cast<float (*)[BM]>(smem + OFF_S);
  uint16_t* const lt = reinterpret_cast<uint16_t*>(smem + OFF_LT);   // limbs of the tile's rows, row stride 2r
  uint16_t* const lb = reinterpret_cast<uint16_t*>(smem + OFF_LB);   // B (f16) of the tile's columns, row stride r

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t nw = n0 + wv * (BN / 4);   // first row of W for this wave
  const int64_t M = a.M, N = a.N, K = a.K, KB = K / BLOCK_K;
  const int64_t row_bytes = (FMT == 0) ? K / 4 : K / 2;
  const NatConsts kc = (FMT == 0) ? q2_nat_consts() : q4_nat_consts();

  // ---- copy sources (byte offsets from the tile's block base; K <= 2^24 keeps
  // them in 32 bits).  They are widened to 64 bits at the copy: with a 32-bit
  // offset operand the host compilation pass drops the kernel's launch stub.
  uint32_t xoff[XU];
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int pos = (u * 4 + wv) * 64 + lane;      // 16-byte chunk position in the stage
    const int row = pos >> 4;
    const int q = (pos & 15) ^ row_swz(row);
    const int64_t gr = (m0 + row < M) ? row : M - 1 - m0;
    xoff[u] = (uint32_t)(gr * K * 2 + q * 16);
  }
  uint32_t woff[CU];
#pragma unroll
  for (int v = 0; v < CU; ++v) {
    const int pos = (v * 4 + wv) * 64 + lane;
    int col, unit;
    if constexpr (FMT == 0) {                      // 2 chunks per column (slots past 2 BN: padding)
      col = pos >> 1;
      col = col < BN ? col : BN - 1;
      unit = ((pos & 1) ^ ((col >> 2) & 1)) << 4;
    } else {                                       // 4 chunks per column
      col = pos >> 2;
      unit = ((pos & 3) ^ ((col >> 1) & 3)) << 4;
    }
    const int64_t gc = (n0 + col < N) ? col : N - 1 - n0;
    woff[v] = (uint32_t)(gc * row_bytes + unit);
  }
  // Scale / zero-point word of column wv*64 + lane of the tile (clamped).
  int64_t sgc = wv * 64 + lane;
  sgc = sgc < BN ? sgc : BN - 1;
  sgc = (n0 + sgc < N) ? n0 + sgc : N - 1;
  const int64_t s_idx = sgc * KB;                  // element index of the column's block-0 scale

  // ---- read side: lane offsets within a stage
  int aoff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) aoff[t] = c * 256 + (((4 * g + t) ^ row_swz(c)) << 4);
  const int coff = (FMT == 0) ? c * 32 + ((((g >> 1) ^ ((c >> 2) & 1)) << 4) | ((g & 1) << 3))
                              : c * 64 + ((g ^ ((c >> 1) & 3)) << 4);
  // Which half of its word holds the scale (zero point) of this lane's column j at block 0.
  uint32_t shalf = 0, zhalf = 0;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int64_t r = nw + 16 * j + c;
    r = r < N ? r : N - 1;
    shalf |= (uint32_t)((((uintptr_t)(a.s + r * KB)) >> 1) & 1) << j;
    if constexpr (FMT == 1) zhalf |= (uint32_t)((((uintptr_t)(a.z + r * KB)) >> 1) & 1) << j;
  }

  // Blocks past the end re-copy the last block into a buffer nobody reads, so
  // every wave issues the same number of copies per block and the vmcnt
  // arithmetic of stage_barrier stays exact.
  auto x_issue = [&](int64_t blk, int stage) {
    blk = blk < KB ? blk : KB - 1;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(a.x + m0 * K + blk * BLOCK_K);
#pragma unroll
    for (int u = 0; u < XU; ++u)
      __builtin_amdgcn_global_load_lds(base + (uint64_t)xoff[u], (lds_void*)(smem + stage * XSTAGE + (u * 4 + wv) * 1024),
                                       16, 0, 0);
  };
  auto w_issue = [&](int64_t blk, int stage) {
    blk = blk < KB ? blk : KB - 1;
    const uint8_t* base = a.w + n0 * row_bytes + blk * BBYTES;
    const int dst = OFF_W + stage * WSTAGE;   // LDS copies must name the shared array itself
#pragma unroll
    for (int v = 0; v < CU; ++v)
      __builtin_amdgcn_global_load_lds(base + (uint64_t)woff[v], (lds_void*)(smem + dst + (v * 4 + wv) * 1024), 16, 0,
                                       0);
    // Byte offset of the aligned word holding element s_idx + blk (may start 2 bytes before it).
    const int64_t si = 2 * (s_idx + blk);
    const uint8_t* sp = reinterpret_cast<const uint8_t*>(a.s);
    __builtin_amdgcn_global_load_lds(sp + (si - (int64_t)(((uintptr_t)sp + si) & 3)),
                                     (lds_void*)(smem + dst + CODE_BYTES + wv * 256), 4, 0, 0);
    if constexpr (FMT == 1) {
      const uint8_t* zp = reinterpret_cast<const uint8_t*>(a.z);
      __builtin_amdgcn_global_load_lds(zp + (si - (int64_t)(((uintptr_t)zp + si) & 3)),
                                       (lds_void*)(smem + dst + CODE_BYTES + 1024 + wv * 256), 4, 0, 0);
    }
  };
  auto afrag = [&](const uint8_t* st, int i, int t) -> q2_u32x4 {
    return *reinterpret_cast<const q2_u32x4*>(st + i * 4096 + aoff[t]);
  };

  // Row sums of the block in stage `st` for this wave's 16-row tiles (i = wv, wv + 4, ...).
  const uint32_t sone = (FMT == 0) ? 0xBFA0BFA0u : 0xBF80BF80u;   // bf16 -1.25 / -1 pairs
  const q2_u32x4 sones = q2_u32x4{sone, sone, sone, sone};
  auto s_compute = [&](const uint8_t* st, int buf) {
#pragma unroll
    for (int ii = 0; ii < (MT + 3) / 4; ++ii) {
      const int i = wv + 4 * ii;
      if (i < MT) {
        q2_f32x4 s4 = q2_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) s4 = mfma(afrag(st, i, t), sones, s4);
        if (c == 0) *reinterpret_cast<q2_f32x4*>(&ss[buf][16 * i + 4 * g]) = s4;
      }
    }
  };

  q2_f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = q2_f32x4{0.f, 0.f, 0.f, 0.f};

  // One block: decode this wave's weights from LDS, then run the MFMAs.
  auto compute = [&](const uint8_t* st, const uint8_t* wst, const float* sb, int64_t blk) {
    q2_u32x4 bf[NT][4];
    float dc[NT], zc[NT];
    const uint32_t par = (uint32_t)(blk & 1) ? 0xFFu : 0u;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int col0 = wv * (BN / 4) + 16 * j;
      uint32_t w[DW];
      if constexpr (FMT == 0) {
        const q2_u32x2 v = *reinterpret_cast<const q2_u32x2*>(wst + col0 * 32 + coff);
        w[0] = v[0]; w[1] = v[1];
      } else {
        const q2_u32x4 v = *reinterpret_cast<const q2_u32x4*>(wst + col0 * 64 + coff);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
      }
      decode_block_nat<FMT>(w, bf[j], kc);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(wst + CODE_BYTES + (col0 + c) * 4);
      uint32_t zb = 0;
      if constexpr (FMT == 1) {
        const uint32_t zw = *reinterpret_cast<const uint32_t*>(wst + CODE_BYTES + 1024 + (col0 + c) * 4);
        zb = zw >> ((((zhalf ^ par) >> j) & 1) * 16);
      }
      block_scale<FMT>(w, sw >> ((((shalf ^ par) >> j) & 1) * 16), zb, dc[j], zc[j]);
    }
    // A fragments of tile i+1 are read from LDS while tile i's MFMAs run;
    // tile i's MFMAs are issued before tile i-1's rescale so the FMAs run in
    // the matrix core's shadow; two temporaries keep everything in VGPRs.
    q2_f32x4 t0[NT], t1[NT];
    q2_u32x4 a0[4], a1[4];
    q2_f32x4 s0, s1;
    auto rd = [&](int i, q2_u32x4 (&av)[4], q2_f32x4& s4) {
      s4 = *reinterpret_cast<const q2_f32x4*>(&sb[16 * i + 4 * g]);
#pragma unroll
      for (int t = 0; t < 4; ++t) av[t] = afrag(st, i, t);
    };
    auto tile = [&](const q2_u32x4 (&av)[4], q2_f32x4 s4, q2_f32x4 (&tmp)[NT]) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < NT; ++j) tmp[j] = mfma(av[t], bf[j][t], t == 0 ? block_cinit<FMT>(s4, zc[j]) : tmp[j]);
    };
    auto rescale = [&](int i, const q2_f32x4 (&tmp)[NT]) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(dc[j], tmp[j][e], acc[i][j][e]);
    };
    rd(0, a0, s0);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i & 1) {
        if (i + 1 < MT) rd(i + 1, a0, s0);
        tile(a1, s1, t1);
        rescale(i - 1, t0);
      } else {
        if (i + 1 < MT) rd(i + 1, a1, s1);
        tile(a0, s0, t0);
        if (i > 0) rescale(i - 1, t1);
      }
    }
    if ((MT - 1) & 1) rescale(MT - 1, t1);
    else rescale(MT - 1, t0);
  };

  if constexpr (LR) {
    // Copy the limbs of this tile's rows and its columns of B into LDS.  These
    // are the oldest copies of the wave, so the first stage_barrier already
    // covers them.  Both copies are whole 64-lane instructions because
    // r % 8 == 0 makes BM*2r/8 and BN*r/8 multiples of 64 for these tiles.
    const int r = a.r;
    const int tch = 2 * r / 8, bch = r / 8;               // 16-byte chunks per row
    for (int base = wv * 64; base < BM * tch; base += 256) {
      const int idx = base + lane;
      const int row = idx / tch, ch = idx - row * tch;
      int64_t gr = m0 + row;
      gr = gr < M ? gr : M - 1;
      __builtin_amdgcn_global_load_lds(a.lr_t + gr * 2 * r + ch * 8, (lds_void*)(smem + OFF_LT + base * 16), 16, 0,
                                       0);
    }
    for (int base = wv * 64; base < BN * bch; base += 256) {
      const int idx = base + lane;
      const int col = idx / bch, ch = idx - col * bch;
      int64_t gn = n0 + col;
      gn = gn < N ? gn : N - 1;
      __builtin_amdgcn_global_load_lds(a.lr_b + gn * r + ch * 8, (lds_void*)(smem + OFF_LB + base * 16), 16, 0,
                                       0);
    }
  }

  if (KB > 0) {
    // At the top of block b: activations b and b+1 and the weights of b have
    // landed and the row sums of b are in ss[b & 1].  With XS = 4 the
    // activations of b+1 were issued two blocks ago (one block's copies came
    // after them), with XS = 3 one block ago (only that block's weight copies
    // came after them).
    x_issue(0, 0);
    w_issue(0, 0);
    x_issue(1, 1);
    w_issue(1, 1);
    if constexpr (XS == 4) {
      x_issue(2, 2);
      stage_barrier<2 * XU + 2 * WU>();
    } else {
      stage_barrier<XU + 2 * WU>();
    }
    s_compute(xs, 0);
    int sx = 0, sw = 0;                  // stages of block b
    for (int64_t b = 0; b < KB; ++b) {
      if constexpr (XS == 4) stage_barrier<XU + WU>();
      else stage_barrier<WU>();
      const int sxn = (sx + XS - 1 >= XS) ? sx - 1 : sx + XS - 1;     // (b + XS - 1) % XS
      const int swn = (sw + 2 >= WS) ? sw - 1 : sw + 2;               // (b + 2) % 3
      x_issue(b + XS - 1, sxn);
      w_issue(b + 2, swn);
      // Row sums of b+1 first: their LDS reads and dependent MFMAs overlap the decode of b.
      const int sx1 = (sx + 1 == XS) ? 0 : sx + 1;
      if (b + 1 < KB) s_compute(xs + sx1 * XSTAGE, (int)((b + 1) & 1));
      compute(xs + sx * XSTAGE, wsm + sw * WSTAGE, ss[b & 1], b);
      sx = sx1;
      sw = (sw + 1 == WS) ? 0 : sw + 1;
    }
  }
  // No copy may still be writing this workgroup's LDS when it ends.
  __builtin_amdgcn_s_waitcnt(0);

  const float fin = (FMT == 0) ? 4.f : 16.f;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] *= fin;

  if (LR) {
    __syncthreads();                   // every wave's copies of the low-rank operands have landed
    const int r = a.r;
    const int ks = (3 * r + 31) / 32;
    for (int t = 0; t < ks; ++t) {
      const int q0 = 32 * t + 8 * g;
      const bool live = q0 < 3 * r;
      const int part = q0 / r, jj = q0 - part * r;
      q2_u32x4 bq[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int col = wv * (BN / 4) + 16 * j + c;
        q2_u32x4 v = q2_u32x4{0u, 0u, 0u, 0u};
        if (live) {
          const q2_u32x4 raw = *reinterpret_cast<const q2_u32x4*>(&lb[col * r + jj]);
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            uint16_t h0, l0, h1, l1;
            f16_split_bf16((uint16_t)(raw[d] & 0xFFFFu), h0, l0);
            f16_split_bf16((uint16_t)(raw[d] >> 16), h1, l1);
            v[d] = (part == 1) ? ((uint32_t)l0 | ((uint32_t)l1 << 16)) : ((uint32_t)h0 | ((uint32_t)h1 << 16));
          }
        }
        bq[j] = v;
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const q2_u32x4 aq = live ? *reinterpret_cast<const q2_u32x4*>(&lt[(16 * i + c) * 2 * r + (part == 2 ? r : 0) + jj])
                                 : q2_u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma(aq, bq[j], acc[i][j]);
      }
    }
  } else if (a.r > 0) {
    const int ks = (3 * a.r + 31) / 32;
    for (int t = 0; t < ks; ++t) {
      const int q0 = 32 * t + 8 * g;
      q2_u32x4 bq[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        int64_t n = nw + 16 * j + c;
        n = n < N ? n : N - 1;
        bq[j] = lr_bfrag(a.lr_b, n, a.r, q0, lr_vec != 0);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        int64_t mr = m0 + 16 * i + c;
        mr = mr < M ? mr : M - 1;
        const q2_u32x4 aq = lr_afrag(a.lr_t, mr, a.r, q0, lr_vec != 0);
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma(aq, bq[j], acc[i][j]);
      }
    }
  }

  if (a.acc) {                            // every old value in flight at once, then added
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t m = m0 + 16 * i + 4 * g + e, n = nw + 16 * j + c;
          acc[i][j][e] += y_old(&a.y[m * N + n], m < M && n < N);
        }
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t n = nw + 16 * j + c;
      if (n < N) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t m = m0 + 16 * i + 4 * g + e;
          if (m < M) __builtin_nontemporal_store(acc[i][j][e], &a.y[m * N + n]);
        }
      }
    }
  }
}

// ============================================================================
// GEMM: KG groups of four waves split the K blocks
// ============================================================================
// One wave per SIMD would expose every LDS, matrix-core and barrier latency of
// a block in turn, and with few activation rows a tile carries little
// matrix-core work per block.  Here a workgroup of KG groups of four
// waves owns a BM x BN tile (BM = 16 MT, BN = 64 NT); wave w computes the
// BM x 16 NT columns w & 3 from the blocks KG s + (w >> 2) of each set s of KG
// consecutive blocks, so a SIMD runs KG independent waves on the same output
// columns while every block's weights are still decoded once per workgroup.
// The KG partial sums are added in group order, through LDS, at the end.
// A ring of NSET sets: the copies of set s + NSET - 1 are issued during set s
// (handed out a few per row tile; the compiler may issue them together at the
// top of the set), so with three sets a copy has two sets' time to land.  Each wave copies whole 16-row activation tiles and computes their row
// sums once its own copies have landed; one barrier per set publishes them.
// Rows past M are clamped on the copy side and dropped at the store.
// s_waitcnt vmcnt(n) for a uniform n in [LO, HI], by binary search over
// compile-time counts (the count is an immediate of the instruction).
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));   // vmcnt(N) only
  asm volatile("" ::: "memory");
}
template <int LO, int HI>
__device__ __forceinline__ void vm_wait_range(int n) {
  if constexpr (LO == HI) {
    vm_wait<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) vm_wait_range<LO, MID>(n);
    else vm_wait_range<MID + 1, HI>(n);
  }
}

template <int FMT, int MT, int NT, int KG, int NSET, bool LR>
__global__ __launch_bounds__(256 * KG) void gemm_kgroup_kernel(LinearArgs a, int tiles_m, int group_m, int kpart) {
  constexpr int W = 4 * KG;                                   // waves
  constexpr int BM = 16 * MT, BN = 64 * NT;
  constexpr int DW = WFmt<FMT>::LANE_DW;
  constexpr int BBYTES = WFmt<FMT>::BLOCK_BYTES;
  constexpr int XSTAGE = BM * 256;                            // one activation block
  constexpr int CPB = (FMT == 0) ? 2 * BN : 4 * BN;           // 16-byte code chunks per block
  constexpr int CODE_SLOT = CPB * 16;
  constexpr int SWORDS = 4 * BN;                              // bytes of scale (zero) words per block
  constexpr int WSTAGE = CODE_SLOT + ((FMT == 0) ? SWORDS : 2 * SWORDS);
  constexpr int NST = NSET * KG;                              // block stages of the ring
  constexpr int OFF_W = NST * XSTAGE;
  constexpr int OFF_S = OFF_W + NST * WSTAGE;
  // With the rank-r branch (r <= LR_RMAX): the tile's columns of B in a region
  // of their own, copied at the start; the tile's rows of the x A^T limbs go
  // to the ring slot that is free during the last set.
  constexpr int OFF_B = (OFF_S + NST * BM * 4 + 15) & ~15;
  constexpr int SMEM = OFF_B + (LR ? BN * (2 * LR_RMAX + 16) + 32 : 0);
  constexpr int NTASK = KG * MT;                              // 16-row activation tiles per set
  constexpr int XT = (NTASK + W - 1) / W;                     // tasks per wave (at most)
  constexpr int XUM = 4 * XT;                                 // activation copy units per wave
  constexpr int CINS = KG * CPB / 64;                         // 64-chunk code copies per set
  constexpr int CU = (CINS + W - 1) / W;                      // code copies per wave
  constexpr int NWU = CU + ((FMT == 0) ? 1 : 2);              // weight copies per wave
  constexpr int NU = XUM + NWU;
  constexpr int UPT = (NU + MT - 1) / MT;                     // copy units issued per row tile
  static_assert(NSET == 2 || NSET == 3, "ring depth");
  static_assert((NSET - 1) * (4 * XT + NWU) <= 63, "copies in flight fit the vmcnt field");
  static_assert(XT <= 2, "activation tasks per wave");
  static_assert(CPB % 64 == 0, "a code copy must not straddle two blocks");
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert((KG - 1) * BM * BN * 4 <= OFF_S, "reduction buffer");
  static_assert(!LR || (FMT == 0 && BM * (4 * LR_RMAX + 16) <= KG * XSTAGE), "low-rank limbs fit one ring slot");
  __shared__ __align__(16) uint8_t smem[SMEM];
  float (*const ss)[KG][BM] = reinterpret_cast<float (*)[KG][BM]>(smem + OFF_S);   // [slot][block of set][row]

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
  // Block and set indices in 32 bits (K <= 2^24): uniform 64-bit compares would run on the vector ALU.
  // This workgroup takes blocks kb0 .. kb - 1.
  const int kb0 = part * kpart;
  const int kb = kpart > 0 ? min((int)KB, kb0 + kpart) : (int)KB;
  const int NS = kb > kb0 ? (kb - kb0 + KG - 1) / KG : 0;    // sets
  const int64_t row_bytes = (FMT == 0) ? K / 4 : K / 2;
  const NatConsts kc = (FMT == 0) ? q2_nat_consts() : q4_nat_consts();

  // ---- copy sources.  Task t of a set is row tile t % MT of block t / MT;
  // wave wv owns tasks wv, wv + W, ...  Copy kk (0..3) of a task fills tile
  // rows 4kk .. 4kk+3; lane l covers row 4kk + (l >> 4), chunk position l & 15,
  // which holds chunk (l & 15) ^ row_swz(row).  The lane's byte offset from
  // the tile's block base (row clamped to M - 1) fits 32 bits since BM <= 128
  // and K <= 2^24.
  int xtasks = 0;
#pragma unroll
  for (int k2 = 0; k2 < XT; ++k2) xtasks += (wv + W * k2 < NTASK) ? 1 : 0;
  const int set_units = 4 * xtasks + NWU;                     // copies this wave issues per set
  uint32_t xoff[XT][4];
#pragma unroll
  for (int k2 = 0; k2 < XT; ++k2) {
    const int it = (wv + W * k2) % MT;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int rin = 4 * kk + (lane >> 4);
      int64_t gr = m0 + 16 * it + rin;
      gr = gr < M ? gr : M - 1;
      xoff[k2][kk] = (uint32_t)((gr - m0) * K * 2) | (uint32_t)(((lane & 15) ^ row_swz(rin)) << 4);
    }
  }
  // Code copy v of wave wv: copy index ci = v * W + wv of the set (clamped to
  // the last one, which is then copied twice with identical bytes), block
  // ci * 64 / CPB, chunks from (ci * 64) % CPB of that block.
  uint32_t woff[CU];
#pragma unroll
  for (int v = 0; v < CU; ++v) {
    int ci = v * W + wv;
    ci = ci < CINS ? ci : CINS - 1;
    const int pos = (ci * 64) % CPB + lane;
    int col, unit;
    if constexpr (FMT == 0) {
      col = pos >> 1;
      unit = ((pos & 1) ^ ((col >> 2) & 1)) << 4;
    } else {
      col = pos >> 2;
      unit = ((pos & 3) ^ ((col >> 1) & 3)) << 4;
    }
    const int64_t gc = (n0 + col < N) ? col : N - 1 - n0;
    woff[v] = (uint32_t)(gc * row_bytes + unit);
  }
  // Scale / zero words: the waves of group kg cover block kg of the set, wave
  // wn the columns sq * 64 + lane with sq = min(wn, NT - 1) (waves past NT
  // repeat the last group's copy, identical bytes to the same place).  Each is
  // copied as the aligned word that holds it, through a resource based 4 bytes
  // below the tile's first scale (zero point): with h the half-word position
  // of the column's block-0 value, the word of block blk sits at so_e (blk
  // even) or so_o (blk odd) plus 2 blk.
  const int sq = wn < NT ? wn : NT - 1;
  const int64_t ncols = (N - n0) < BN ? (N - n0) : BN;
  int64_t sgc = sq * 64 + lane;                               // column from n0
  sgc = sgc < ncols ? sgc : ncols - 1;
  const uint32_t svl = (uint32_t)(2 * sgc * KB);
  const uint32_t sbytes = (uint32_t)(2 * ncols * KB + 8);
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(reinterpret_cast<const uint8_t*>(a.s + n0 * KB) - 4, sbytes);
  const uint32_t sh = (uint32_t)(((uintptr_t)(a.s + n0 * KB) + svl) >> 1) & 1u;
  const uint32_t so_e = svl + 4 - 2 * sh, so_o = svl + 2 + 2 * sh;
  __amdgpu_buffer_rsrc_t rz = rs;
  uint32_t zo_e = 0, zo_o = 0;
  if constexpr (FMT == 1) {
    rz = buf_rsrc(reinterpret_cast<const uint8_t*>(a.z + n0 * KB) - 4, sbytes);
    const uint32_t zh = (uint32_t)(((uintptr_t)(a.z + n0 * KB) + svl) >> 1) & 1u;
    zo_e = svl + 4 - 2 * zh;
    zo_o = svl + 2 + 2 * zh;
  }
  // Activation and code resources over the tile's valid rows and columns.
  const int64_t nrows = (M - m0) < BM ? (M - m0) : BM;
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(a.x + m0 * K, (uint32_t)(nrows * K * 2));
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(a.w + n0 * row_bytes, (uint32_t)(ncols * row_bytes));

  // ---- read side
  int aoff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) aoff[t] = c * 256 + (((4 * g + t) ^ row_swz(c)) << 4);
  const int coff = (FMT == 0) ? c * 32 + ((((g >> 1) ^ ((c >> 2) & 1)) << 4) | ((g & 1) << 3))
                              : c * 64 + ((g ^ ((c >> 1) & 3)) << 4);
  uint32_t shalf = 0, zhalf = 0;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int64_t r = nw + 16 * j + c;
    r = r < N ? r : N - 1;
    shalf |= (uint32_t)((((uintptr_t)(a.s + r * KB)) >> 1) & 1) << j;
    if constexpr (FMT == 1) zhalf |= (uint32_t)((((uintptr_t)(a.z + r * KB)) >> 1) & 1) << j;
  }

  // Copies of set `set` into ring slot `slot`, one unit at a time: units
  // 0 .. XUM-1 the activation copies of this wave's tasks, then the codes, the
  // scale words [and zero words].  Blocks past the end re-copy the last one.
  auto issue_unit = [&](int unit, int set, int slot) {
    const int b0 = kb0 + KG * set;
    if (unit < XUM) {
      const int k2 = unit >> 2, kk = unit & 3;
      if (k2 < xtasks) {
        const int task = wv + W * k2;
        const int q = task / MT, it = task - q * MT;
        int blk = b0 + q;
        blk = blk < kb ? blk : kb - 1;
        // Offsets go through locals: with an array element as the operand the
        // host compilation pass drops the kernel's launch stub.
        const uint32_t xo = xoff[k2][kk];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (lds_void*)(smem + (slot * KG + q) * XSTAGE + (16 * it + 4 * kk) * 256), 16, xo,
            (uint32_t)blk * 256u, 0, 0);
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
          (uint32_t)blk * (uint32_t)BBYTES, 0, 0);
    } else {
      int blk = b0 + kg;
      blk = blk < kb ? blk : kb - 1;
      const int dst = OFF_W + (slot * KG + kg) * WSTAGE + CODE_SLOT + sq * 256;
      const bool odd = (blk & 1) != 0;
      if (unit == XUM + CU) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(smem + dst), 4, odd ? so_o : so_e,
                                                 2u * (uint32_t)blk, 0, 0);
      } else if constexpr (FMT == 1) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_void*)(smem + dst + SWORDS), 4, odd ? zo_o : zo_e,
                                                 2u * (uint32_t)blk, 0, 0);
      }
    }
  };
  auto issue_set = [&](int set, int slot) {
    for (int un = 0; un < NU; ++un) issue_unit(un, set, slot);
  };
  auto afrag = [&](const uint8_t* st, int i, int t) -> q2_u32x4 {
    return *reinterpret_cast<const q2_u32x4*>(st + i * 4096 + aoff[t]);
  };

  const uint32_t sone = (FMT == 0) ? 0xBFA0BFA0u : 0xBF80BF80u;   // bf16 -1.25 / -1 pairs
  const q2_u32x4 sones = q2_u32x4{sone, sone, sone, sone};
  // Row sums of this wave's tasks of set `set` (slot `slot`).
  auto row_sums = [&](int set, int slot) {
#pragma unroll
    for (int k2 = 0; k2 < XT; ++k2) {
      if (k2 < xtasks) {
        const int task = wv + W * k2;
        const int q = task / MT, it = task - q * MT;
        if (kb0 + KG * set + q < kb) {
          const uint8_t* st = smem + (slot * KG + q) * XSTAGE;
          q2_f32x4 s4 = q2_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) s4 = mfma(afrag(st, it, t), sones, s4);
          if (c == 0) *reinterpret_cast<q2_f32x4*>(&ss[slot][q][16 * it + 4 * g]) = s4;
        }
      }
    }
  };
  // Wait until at most n of this wave's copies are in flight (n is uniform and
  // one of the per-set counts).
  auto wait_copies = [&](int n) {
    asm volatile("" ::: "memory");
    if (n == 0) {
      __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));
    } else if (n == NWU) {
      __builtin_amdgcn_s_waitcnt((NWU & 15) | (7 << 4) | (15 << 8) | ((NWU >> 4) << 14));
    } else if (n == NWU + 4) {
      __builtin_amdgcn_s_waitcnt(((NWU + 4) & 15) | (7 << 4) | (15 << 8) | (((NWU + 4) >> 4) << 14));
    } else {
      __builtin_amdgcn_s_waitcnt(((NWU + 8) & 15) | (7 << 4) | (15 << 8) | (((NWU + 8) >> 4) << 14));
    }
    asm volatile("" ::: "memory");
  };

  // ---- the rank-r branch (LR; of a split tile, part 0 carries it).  Its
  // operands are copied first: B's rows n0 .. n0 + BN - 1 into a region of
  // their own (with r % 8 == 0 and an aligned start, r / 8 chunks per row plus
  // one of padding; otherwise the row range as one byte run, from the 16-byte
  // boundary b_off bytes below its start), and the tile's rows of the x A^T
  // limbs (4 r8 bytes, r8 / 4 16-byte chunks each, one chunk of padding after
  // each row so the sixteen rows one fragment read touches fall in different
  // banks; rows past M left to the resource's bounds) into ring slot NSET - 1,
  // which no set occupies before set NSET - 1 is copied during set 0.  The
  // branch's matrix-core steps then run while the first set's copies land.
  const int lr_r = LR ? a.r : 0;
  const int lr_rs = lr_pad(lr_r);
  const int t_cr = lr_rs / 4 + 1;                        // LDS chunks per limb row, padding included
  const uint32_t b_off = LR ? (uint32_t)(reinterpret_cast<uintptr_t>(a.lr_b + n0 * lr_r) & 15u) : 0u;
  const bool bvec = LR && (lr_r & 7) == 0 && b_off == 0;
  const int b_cr = lr_r / 8 + 1;                         // LDS chunks per row of B when bvec
  if (LR && part == 0) {
    const uint8_t* bsrc = reinterpret_cast<const uint8_t*>(a.lr_b + n0 * lr_r) - b_off;
    const uint32_t bavail = (uint32_t)(ncols * 2 * lr_r) + b_off;
    const __amdgpu_buffer_rsrc_t rb = buf_rsrc(bsrc, bavail);
    const int bchunks = bvec ? BN * b_cr : (int)((bavail + 15) / 16);
    for (int base = wv * 64; base < bchunks; base += 64 * W) {
      const int idx = base + lane;
      uint32_t src = (uint32_t)idx * 16u;
      if (bvec) {
        const int row = idx / b_cr, q = idx - row * b_cr;
        src = (uint32_t)(row * (b_cr - 1) + min(q, b_cr - 2)) * 16u;   // the padding chunk repeats the last
      }
      if (idx < bchunks)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(smem + OFF_B + base * 16), 16, src, 0, 0, 0);
    }
  }
  auto issue_limbs = [&](int tslot) {
    const __amdgpu_buffer_rsrc_t rt = buf_rsrc(a.lr_t + m0 * 2 * lr_rs, (uint32_t)(nrows * 4 * lr_rs));
    const int tchunks = BM * t_cr;
    for (int base = wv * 64; base < tchunks; base += 64 * W) {
      const int idx = base + lane;
      const int row = idx / t_cr, q = idx - row * t_cr;
      const uint32_t src = (uint32_t)(row * (t_cr - 1) + min(q, t_cr - 2)) * 16u;
      if (idx < tchunks)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (lds_void*)(smem + tslot * KG * XSTAGE + base * 16), 16, src, 0,
                                                 0, 0);
    }
  };

  q2_f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = q2_f32x4{0.f, 0.f, 0.f, 0.f};

  // The branch (x A^T) B^T into acc, from the limbs in ring slot tslot and B
  // in its region, then divided by the final scale factor (a power of two, so
  // exactly) since the block sums are added in those units.  Its K steps are
  // shared out over the groups.
  auto lr_branch = [&](int tslot) {
    const uint8_t* tls = smem + tslot * KG * XSTAGE;
    const uint8_t* bls = smem + OFF_B + b_off;          // (aligned rows when bvec)
    const int ks = (3 * lr_rs + 31) / 32;
    if (bvec && (lr_rs & 31) == 0) {
      // Every K step lies inside one part (T_hi B_hi, T_hi B_lo, T_lo B_hi),
      // the same for all lanes: all of a step's fragments are read first,
      // then only the needed half of B's split is formed.
      const int spp = lr_rs / 32;                        // steps per part
      for (int t = kg; t < ks; t += KG) {
        const int prt = t / spp;                         // uniform
        const int jj = (t - prt * spp) * 32 + 8 * g;
        const int tq = ((prt == 2 ? lr_rs : 0) + jj) / 8;
        q2_u32x4 raw[NT], aq[MT];
#pragma unroll
        for (int j = 0; j < NT; ++j)
          raw[j] = *reinterpret_cast<const q2_u32x4*>(bls + ((wn * (BN / 4) + 16 * j + c) * b_cr + jj / 8) * 16);
#pragma unroll
        for (int i = 0; i < MT; ++i)
          aq[i] = *reinterpret_cast<const q2_u32x4*>(tls + ((16 * i + c) * t_cr + tq) * 16);
        q2_u32x4 bq[NT];
        if (prt == 1) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) bq[j][d] = f16x2_bf16_lo(raw[j][d]);
        } else {
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) bq[j][d] = f16x2_bf16_hi(raw[j][d]);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j) acc[i][j] = mfma(aq[i], bq[j], acc[i][j]);
      }
    } else {
      for (int t = kg; t < ks; t += KG) {
        const int q0 = 32 * t + 8 * g;
        const bool live = q0 < 3 * lr_rs;
        const int prt = live ? q0 / lr_rs : 0, jj = q0 - prt * lr_rs;
        q2_u32x4 bq[NT];
  #pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int col = wn * (BN / 4) + 16 * j + c;
          q2_u32x4 raw = q2_u32x4{0u, 0u, 0u, 0u};
          if (live) {
            if (bvec) {
              raw = *reinterpret_cast<const q2_u32x4*>(bls + (col * b_cr + jj / 8) * 16);
            } else {
              // The copy's bounds check drops a dword that is only partly
              // inside B, so an element in such a last dword comes from
              // global memory instead.
              const uint32_t bavail = (uint32_t)(ncols * 2 * lr_r) + b_off;
              uint32_t h[8];
  #pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int jx = jj + e;
                uint32_t hv = 0u;
                if (jx < lr_r) {
                  const uint32_t p = b_off + (uint32_t)(col * lr_r + jx) * 2u;
                  if ((p & ~3u) + 4u <= bavail) hv = *reinterpret_cast<const uint16_t*>(smem + OFF_B + p);
                  else if (p + 2u <= bavail) hv = a.lr_b[(n0 + col) * lr_r + jx];
                }
                h[e] = hv;
              }
              raw = q2_u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
            }
          }
          q2_u32x4 v;
  #pragma unroll
          for (int d = 0; d < 4; ++d) v[d] = (prt == 1) ? f16x2_bf16_lo(raw[d]) : f16x2_bf16_hi(raw[d]);
          bq[j] = v;
        }
        const int tq = ((prt == 2 ? lr_rs : 0) + jj) / 8;     // the limb chunk of this K step
  #pragma unroll
        for (int i = 0; i < MT; ++i) {
          const q2_u32x4 aq = live ? *reinterpret_cast<const q2_u32x4*>(tls + ((16 * i + c) * t_cr + tq) * 16)
                                   : q2_u32x4{0u, 0u, 0u, 0u};
  #pragma unroll
          for (int j = 0; j < NT; ++j) acc[i][j] = mfma(aq, bq[j], acc[i][j]);
        }
      }
    }
    const float inv = (FMT == 0) ? 0.25f : 0.0625f;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] *= inv;
  };
  // Wait until at most the copies of k sets (uniform) of this wave are in flight.
  auto wait_sets = [&](int k) { vm_wait_range<0, 63>(k * set_units); };

  // Decode of one block's weights for this wave's columns (from its weight stage).
  auto decode = [&](const uint8_t* wst, int blk, q2_u32x4 (&bf)[NT][4], float (&dc)[NT], float (&zc)[NT]) {
    const uint32_t pmask = (uint32_t)(blk & 1) ? 0xFFu : 0u;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int col0 = wn * (BN / 4) + 16 * j;
      uint32_t w[DW];
      if constexpr (FMT == 0) {
        const q2_u32x2 v = *reinterpret_cast<const q2_u32x2*>(wst + col0 * 32 + coff);
        w[0] = v[0]; w[1] = v[1];
      } else {
        const q2_u32x4 v = *reinterpret_cast<const q2_u32x4*>(wst + col0 * 64 + coff);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
      }
      decode_block_nat<FMT>(w, bf[j], kc);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(wst + CODE_SLOT + (col0 + c) * 4);
      uint32_t zb = 0;
      if constexpr (FMT == 1) {
        const uint32_t zw = *reinterpret_cast<const uint32_t*>(wst + CODE_SLOT + SWORDS + (col0 + c) * 4);
        zb = zw >> ((((zhalf ^ pmask) >> j) & 1) * 16);
      }
      block_scale<FMT>(w, sw >> ((((shalf ^ pmask) >> j) & 1) * 16), zb, dc[j], zc[j]);
    }
  };
  // MFMAs of one block over the staged activations `st`, row sums `sb`; the
  // copies of set `cset` (if >= 0) are issued UPT units per row tile.
  auto mainblk = [&](const uint8_t* st, const float* sb, const q2_u32x4 (&bf)[NT][4], const float (&dc)[NT],
                     const float (&zc)[NT], int cset, int cslot) {
    q2_u32x4 a0[4], a1[4];
    q2_f32x4 s0, s1;
    auto rd = [&](int i, q2_u32x4 (&av)[4], q2_f32x4& s4) {
      s4 = *reinterpret_cast<const q2_f32x4*>(&sb[16 * i + 4 * g]);
#pragma unroll
      for (int t = 0; t < 4; ++t) av[t] = afrag(st, i, t);
    };
    auto tile = [&](int i, const q2_u32x4 (&av)[4], q2_f32x4 s4) {
      q2_f32x4 tmp[NT];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          tmp[j] = mfma(av[t], bf[j][t], t == 0 ? block_cinit<FMT>(s4, zc[j]) : tmp[j]);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(dc[j], tmp[j][e], acc[i][j][e]);
    };
    rd(0, a0, s0);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (cset >= 0) {
#pragma unroll
        for (int un = UPT * i; un < UPT * i + UPT; ++un)
          if (un < NU) issue_unit(un, cset, cslot);
      }
      if (i & 1) {
        if (i + 1 < MT) rd(i + 1, a0, s0);
        tile(i, a1, s1);
      } else {
        if (i + 1 < MT) rd(i + 1, a1, s1);
        tile(i, a0, s0);
      }
    }
  };

  // Set s sits in ring slot s % NSET.  Before the top barrier of set s, every
  // wave has waited for its own copies of set s and written their row sums;
  // the barrier publishes them and marks set s - 1 done, so its slot receives
  // the copies of set s + NSET - 1 during set s.  With NSET = 2 a set's weight
  // copies are the last ones waited for (vmcnt(0) at its top barrier); with
  // a deeper ring each wave has waited for all of set s's copies at the end
  // of set s - 1, leaving the copies of up to NSET - 2 later sets in flight.
  // The first NSET - 1 sets are issued at the start.
  const int pre = NS < NSET - 1 ? NS : NSET - 1;         // sets issued before the loop
  if constexpr (LR) {
    if (part == 0) issue_limbs(NSET - 1);
  }
  for (int q = 0; q < pre; ++q) issue_set(q, q);
  if constexpr (LR) {
    if (part == 0) {
      // B and the limbs were issued before the sets' copies, so they have
      // landed once only those may be in flight.
      wait_sets(pre);
      __syncthreads();
      lr_branch(NSET - 1);
    }
  }
  if (NS > 0) {
    if constexpr (NSET >= 3) wait_sets(pre - 1);
    else wait_copies(NWU);
    row_sums(0, 0);
    int slot = 0;
    for (int s = 0; s < NS; ++s) {
      if constexpr (NSET >= 3) stage_barrier<63>();
      else stage_barrier<0>();
      const int cset = (s + NSET - 1 < NS) ? s + NSET - 1 : -1;       // the set copied during this one
      const int cslot = (slot + NSET - 1 >= NSET) ? slot - 1 : slot + NSET - 1;   // (s + NSET - 1) % NSET
      const int bp = kb0 + KG * s + kg;
      if (bp < kb) {
        q2_u32x4 bf[NT][4];
        float dc[NT], zc[NT];
        decode(smem + OFF_W + (slot * KG + kg) * WSTAGE, bp, bf, dc, zc);
        mainblk(smem + (slot * KG + kg) * XSTAGE, ss[slot][kg], bf, dc, zc, cset, cslot);
      } else if (cset >= 0) {
        issue_set(cset, cslot);
      }
      const int nslot = (slot + 1 == NSET) ? 0 : slot + 1;
      if (s + 1 < NS) {
        // The copies of set s + 1 have landed once only those issued after
        // them may be in flight: with two sets its own weight copies, with
        // more the copies of the sets s + 2 .. s + NSET - 1 issued so far.
        if constexpr (NSET >= 3) {
          const int last = (s + NSET - 1 < NS) ? s + NSET - 1 : NS - 1;   // last set issued
          wait_sets(last - (s + 1));
        } else {
          wait_copies(NWU);
        }
        row_sums(s + 1, nslot);
      }
      slot = nslot;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);          // every copy of this wave has landed
  __syncthreads();                        // and every wave is done reading the stages

  const float fin_red = (FMT == 0) ? 4.f : 16.f;   // the scale still to apply after the group sum

  // Under accumulation the old y values of the row-major stores are loaded
  // now, while the tile is reduced.  A split tile adds its part into y with
  // one atomic add per element, in the matrix-core layout (16 consecutive
  // columns of a row per instruction and row group).
  const bool split = kpart > 0;
  const bool rows16 = !split && (N & 3) == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
  constexpr int RP = (BM * (BN / 4) + 64 * W - 1) / (64 * W);
  q2_f32x4 yo4[RP];
  if (a.acc && rows16) {
#pragma unroll
    for (int t = 0; t < RP; ++t) {
      int row, q;
      const bool v = row_piece<BM, BN, 64 * W>(t, tid, (int)nrows, (int)ncols, row, q);
      yo4[t] = y_old4(reinterpret_cast<const q2_f32x4*>(&a.y[(m0 + row) * N + n0 + 4 * q]), v);
    }
  }

  // Partial sums of groups 1 .. KG-1 -> LDS -> added in group order by group 0.
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
  if (rows16) {
    // The finished tile goes through LDS (rows padded to OS floats) and is
    // stored as 16-byte pieces of contiguous rows.
    constexpr int OS = BN + 4;
    static_assert(BM * OS * 4 <= SMEM, "output tile");
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
            acc[i][j][e] = v * fin_red;
          }
    }
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
        if (a.acc) v += yo4[t];
        __builtin_nontemporal_store(v, reinterpret_cast<q2_f32x4*>(&a.y[(m0 + row) * N + n0 + 4 * q]));
      }
    }
  } else if (kg == 0) {
    // Tile-relative 32-bit row and column indices against the tile's valid
    // counts (no 64-bit index is then live across the main loop).
    float* const yt = a.y + m0 * N + n0;
    const int nr = (int)nrows, nc = (int)ncols;
    float yo[MT][NT][4];
    if (a.acc) {                          // every old value in flight at once, then added
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int mr = 16 * i + 4 * g + e, cr = wn * (BN / 4) + 16 * j + c;
            yo[i][j][e] = y_old(&yt[(int64_t)mr * N + cr], mr < nr && cr < nc);
          }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int cr = wn * (BN / 4) + 16 * j + c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = acc[i][j][e];
#pragma unroll
          for (int q = 1; q < KG; ++q) v += red[(((q - 1) * 4 + wn) * PART) + ((i * NT + j) * 4 + e) * 64 + lane];
          v *= fin_red;
          const int mr = 16 * i + 4 * g + e;
          if (a.acc) v += yo[i][j][e];
          if (mr < nr && cr < nc) {
            if (split) unsafeAtomicAdd(&yt[(int64_t)mr * N + cr], v);
            else __builtin_nontemporal_store(v, &yt[(int64_t)mr * N + cr]);
          }
        }
      }
    }
  }
}

// ============================================================================
// GEMV, M <= 16
// ============================================================================
constexpr int GEMV_XQ = 2;                        // 16-activation staging chunks per thread per pass
constexpr int GEMV_X_BYTES = 40 * 1024;          // LDS for staged activations and block sums per chunk

// A unit (16 weight rows x 4 consecutive 128-blocks) is loaded with quad-coalesced
// accesses: lane l reads the 32 bytes of block (l & 3) of row (l >> 2), so four
// consecutive lanes cover one row's 128 contiguous bytes.  It is then
// transposed through a per-wave LDS tile into the matrix-core layout, where
// lane (c, g) needs dwords 2g, 2g+1 of each block of row c.
template <int FMT, int QMAX, int GEMV_WAVES>
__global__ __launch_bounds__(GEMV_WAVES * 64) void gemv_kernel(LinearArgs a, int cb, int lr_vec) {
  constexpr int DW = WFmt<FMT>::LANE_DW;          // dwords per lane per block in the MFMA layout
  constexpr int BBYTES = WFmt<FMT>::BLOCK_BYTES;  // 32 (2-bit) or 64 (4-bit)
  constexpr int UDW = 16 * 4 * BBYTES / 4;        // dwords per unit
  extern __shared__ __align__(16) uint32_t smem[];
  const int M = (int)a.M;
  const int rs = cb * 64 + 4;                     // dwords per staged activation row
  uint32_t* xs = smem;
  float* ss = reinterpret_cast<float*>(smem + M * rs);   // [cb][16] pre-scaled block sums
  uint32_t* ws = smem + M * rs + cb * 16;                // per wave: one unit of codes, then its scales

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t n = n0 + c;                              // weight row of this lane's MFMA column
  const int64_t K = a.K, KB = K / BLOCK_K;
  const int crow = c < M ? c : M - 1;                    // activation rows past M duplicate row M-1
  const DecodeConsts kc = (FMT == 0) ? q2_consts() : q4_consts();
  // loader layout
  const int lrow = lane >> 2, lblk = lane & 3;
  int64_t ln = n0 + lrow;
  ln = ln < a.N ? ln : a.N - 1;                          // rows past N reload row N-1, never stored
  const uint8_t* wrow = a.w + ln * ((FMT == 0) ? K / 4 : K / 2) + lblk * BBYTES;
  const uint16_t* srow = a.s + ln * KB + lblk;
  const uint16_t* zrow = (FMT == 1) ? a.z + ln * KB + lblk : nullptr;
  uint32_t* wt = ws + wv * (UDW + 64);                  // this wave's transpose tile

  q2_f32x4 acc = q2_f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.r > 0 && wv == GEMV_WAVES - 1) {
    // The last wave adds the low-rank term first, divided by the final scale
    // factor (a power of two, so exactly), while the other waves stream codes.
    const int64_t nc = n < a.N ? n : a.N - 1;
    const int ks = (3 * a.r + 31) / 32;
    for (int t = 0; t < ks; ++t) {
      const int q0 = 32 * t + 8 * g;
      acc = mfma(lr_afrag(a.lr_t, crow, a.r, q0, lr_vec != 0), lr_bfrag(a.lr_b, nc, a.r, q0, lr_vec != 0), acc);
    }
    const float inv = (FMT == 0) ? 0.25f : 0.0625f;
    acc = q2_f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  }

  for (int64_t cb0 = 0; cb0 < KB; cb0 += cb) {
    const int nb = (int)((KB - cb0) < cb ? (KB - cb0) : cb);
    const int nunits = (nb + 3) / 4;
    const int mine = (nunits - wv + GEMV_WAVES - 1) / GEMV_WAVES;   // units wv, wv + WAVES, ...
    const int nchunks = M * nb * 8;
    // activation loads of the first staging pass go out first, so that
    // staging waits on them only; then every weight unit of this wave
    constexpr int XP = GEMV_WAVES * 64 * GEMV_XQ;          // chunks per staging pass
    uint32_t nx[GEMV_XQ][8];
    auto x_issue = [&](int base) {
#pragma unroll
      for (int u = 0; u < GEMV_XQ; ++u) {
        const int idx = base + tid + u * GEMV_WAVES * 64;
        if (idx < nchunks) {                     // masked lanes issue no memory traffic
          const int row = idx / (nb * 8);
          const int rem = idx - row * nb * 8;
          load_x16(a.x, row, K, (cb0 + (rem >> 3)) * BLOCK_K + (rem & 7) * 16, nx[u]);
        }
      }
    };
    auto x_stage = [&](int base) {
#pragma unroll
      for (int u = 0; u < GEMV_XQ; ++u) {
        const int idx = base + tid + u * GEMV_WAVES * 64;
        if (base + u * GEMV_WAVES * 64 >= nchunks) break;   // uniform: no chunk left for any thread
        const int row = idx / (nb * 8);
        const int rem = idx - row * nb * 8;
        const int bl = rem >> 3, prt = rem & 7;
        uint32_t pr[8];
        stage_pairs<FMT>(nx[u], pr);
        const float sm = sum8_lanes(bf16_sum16(nx[u]));
        if (idx < nchunks) {
          q2_u32x4* dst = reinterpret_cast<q2_u32x4*>(&xs[row * rs + bl * 64 + prt * 8]);
          dst[0] = q2_u32x4{pr[0], pr[1], pr[2], pr[3]};
          dst[1] = q2_u32x4{pr[4], pr[5], pr[6], pr[7]};
          if (prt == 0) ss[bl * 16 + row] = sm * ((FMT == 0) ? -1.25f : -1.f);
        }
      }
    };
    x_issue(0);
    q2_u32x4 wq[QMAX][BBYTES / 16];
    uint32_t sq[QMAX], zq[QMAX];
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      int unit = wv + GEMV_WAVES * q;
      unit = unit < nunits ? unit : nunits - 1;
      int blk = unit * 4 + lblk;
      blk = blk < nb ? blk : nb - 1;                   // a partial last unit re-reads a valid block
      const int64_t gb = cb0 + blk;
      const q2_u32x4* p = reinterpret_cast<const q2_u32x4*>(wrow + (gb - lblk) * BBYTES);
#pragma unroll
      for (int h = 0; h < BBYTES / 16; ++h) wq[q][h] = p[h];
      sq[q] = srow[gb - lblk];
      zq[q] = (FMT == 1) ? zrow[gb - lblk] : 0u;
    }
    x_stage(0);
    for (int base = XP; base < nchunks; base += XP) {
      x_issue(base);
      x_stage(base);
    }
    for (int idx = tid; idx < nb * 16; idx += GEMV_WAVES * 64)
      if ((idx & 15) >= M) ss[idx] = 0.f;
    __syncthreads();

#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      if (q < mine) {
        const int unit = wv + GEMV_WAVES * q;
        // transpose through the wave's own LDS tile: codes [row][blk][dwords],
        // then scales and zero points [row][blk] as u16 (one wave, in order)
        uint32_t* t = wt;
        {
          q2_u32x4* dst = reinterpret_cast<q2_u32x4*>(t + (lrow * 4 + lblk) * (BBYTES / 4));
#pragma unroll
          for (int h = 0; h < BBYTES / 16; ++h) dst[h] = wq[q][h];
          uint16_t* stw = reinterpret_cast<uint16_t*>(t + UDW);
          stw[lrow * 4 + lblk] = (uint16_t)sq[q];
          if (FMT == 1) stw[64 + lrow * 4 + lblk] = (uint16_t)zq[q];
        }
        const uint16_t* st = reinterpret_cast<const uint16_t*>(t + UDW);
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int bl = unit * 4 + b4;
          if (bl < nb) {
            uint32_t w[DW];
            if constexpr (DW == 2) {
              const q2_u32x2 v = *reinterpret_cast<const q2_u32x2*>(t + (c * 4 + b4) * 8 + 2 * g);
              w[0] = v[0]; w[1] = v[1];
            } else {
              const q2_u32x4 v = *reinterpret_cast<const q2_u32x4*>(t + (c * 4 + b4) * 16 + 4 * g);
              w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
            }
            float dsc, zp;
            block_scale<FMT>(w, st[c * 4 + b4], (FMT == 1) ? st[64 + c * 4 + b4] : 0u, dsc, zp);
            q2_u32x4 bf[4];
            decode_block<FMT>(w, bf, kc);
            const q2_f32x4 s4 = *reinterpret_cast<const q2_f32x4*>(&ss[bl * 16 + 4 * g]);
            q2_f32x4 tmp = block_cinit<FMT>(s4, zp);
#pragma unroll
            for (int tk = 0; tk < 4; ++tk)
              tmp = mfma(*reinterpret_cast<const q2_u32x4*>(&xs[crow * rs + bl * 64 + 16 * g + 4 * tk]), bf[tk], tmp);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(dsc, tmp[e], acc[e]);
          }
        }
        __builtin_amdgcn_wave_barrier();              // tile reads done before the next unit's writes
      }
    }
    __syncthreads();
  }

  // Under accumulation wave 0 loads its old y values before the reduction.
  float yo[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.acc && wv == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * g + e;
      yo[e] = (n < a.N && m < M) ? a.y[(int64_t)m * a.N + n] : 0.f;
    }
  }

  // fixed-order reduction over the waves' K partitions
  q2_f32x4* red = reinterpret_cast<q2_f32x4*>(smem);
  red[wv * 64 + lane] = acc;
  __syncthreads();
  if (wv == 0) {
    q2_f32x4 s = red[lane];
#pragma unroll
    for (int w = 1; w < GEMV_WAVES; ++w) {
      const q2_f32x4 o = red[w * 64 + lane];
      s = q2_f32x4{s[0] + o[0], s[1] + o[1], s[2] + o[2], s[3] + o[3]};
    }
    const float fin = (FMT == 0) ? 4.f : 16.f;
    s = q2_f32x4{s[0] * fin, s[1] * fin, s[2] * fin, s[3] * fin};
    if (n < a.N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * g + e;
        if (m < M) {
          a.y[(int64_t)m * a.N + n] = a.acc ? s[e] + yo[e] : s[e];
        }
      }
    }
  }
}

// ============================================================================
// x A^T for the low-rank branch: bf16 limbs [M, 2 r8] = (hi | lo), r8 = r
// rounded up to a multiple of 8, padding columns zero
// ============================================================================
constexpr int LR_WAVES = 16;
constexpr int LR_UNROLL = 6;     // k-steps per wave whose loads are issued together

// A workgroup owns 16 rows of x and 16 columns of A (one MFMA tile); its waves
// split K in 32-wide steps, issue all their loads first, and are reduced in a
// fixed order.  A (f16) is split exactly into bf16 hi + lo, two MFMAs per step.
__global__ __launch_bounds__(LR_WAVES * 64) void lowrank_t_kernel(const uint16_t* x, const uint16_t* A, uint16_t* tl,
                                                                  int64_t M, int64_t K, int r) {
  __shared__ __align__(16) q2_f32x4 red[LR_WAVES][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  int64_t m = (int64_t)blockIdx.x * 16 + c;                // A-operand row of this lane
  m = m < M ? m : M - 1;
  int col = blockIdx.y * 16 + c;                           // B-operand column (row of A)
  col = col < r ? col : r - 1;
  const int64_t KS = K / 32;
  q2_f32x4 acc = q2_f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t s0 = wv; s0 < KS; s0 += (int64_t)LR_WAVES * LR_UNROLL) {
    q2_u32x4 av[LR_UNROLL], bv[LR_UNROLL];
#pragma unroll
    for (int u = 0; u < LR_UNROLL; ++u) {
      int64_t s = s0 + (int64_t)LR_WAVES * u;
      s = s < KS ? s : KS - 1;
      const int64_t k0 = s * 32 + 8 * g;
      av[u] = *reinterpret_cast<const q2_u32x4*>(x + m * K + k0);
      bv[u] = *reinterpret_cast<const q2_u32x4*>(A + (int64_t)col * K + k0);
    }
#pragma unroll
    for (int u = 0; u < LR_UNROLL; ++u) {
      if (s0 + (int64_t)LR_WAVES * u < KS) {
        q2_u32x4 bh, bl;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          bh[d] = f16x2_bf16_hi(bv[u][d]);
          bl[d] = f16x2_bf16_lo(bv[u][d]);
        }
        acc = mfma(av[u], bh, acc);
        acc = mfma(av[u], bl, acc);
      }
    }
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    q2_f32x4 sm = red[0][lane];
#pragma unroll
    for (int w = 1; w < LR_WAVES; ++w) {
      const q2_f32x4 o = red[w][lane];
      sm = q2_f32x4{sm[0] + o[0], sm[1] + o[1], sm[2] + o[2], sm[3] + o[3]};
    }
    const int oc = blockIdx.y * 16 + c;                    // C layout: column = lane % 16
    const int rs = lr_pad(r);
    if (oc < rs) {                                         // columns r .. rs-1 are the zero padding
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = (int64_t)blockIdx.x * 16 + 4 * g + e;
        if (row < M) {
          const float t = oc < r ? sm[e] : 0.f;
          const uint16_t hi = f32_to_bf16_rn(t);
          const uint16_t lo = f32_to_bf16_rn(t - bf16_to_f32(hi));
          tl[row * 2 * rs + oc] = hi;
          tl[row * 2 * rs + rs + oc] = lo;
        }
      }
    }
  }
}

// ============================================================================
// launchers
// ============================================================================
static int lowrank_vec(const LinearArgs& a) {
  return (a.r > 0 && a.r % 8 == 0 && (reinterpret_cast<uintptr_t>(a.lr_b) % 16) == 0) ? 1 : 0;
}

template <int FMT, int BM, int BN>
static hipError_t run_gemm(const LinearArgs& a, hipStream_t stream) {
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (a.N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const int vec = lowrank_vec(a);
  // The low-rank branch only exists for Q2_0 weights.
  if constexpr (FMT == 0) {
    if (vec && a.r <= LR_RMAX) {
      hipLaunchKernelGGL((gemm_kernel<FMT, BM, BN, true>), dim3((unsigned)tiles), dim3(256), 0, stream, a,
                         (int)tiles_m, vec);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<FMT, BM, BN, false>), dim3((unsigned)tiles), dim3(256), 0, stream, a, (int)tiles_m,
                     vec);
  return hipGetLastError();
}

template <int FMT, int QMAX, int WAVES>
static hipError_t launch_gemv(const LinearArgs& a, int64_t cb, hipStream_t stream) {
  constexpr int UDW = 16 * 4 * WFmt<FMT>::BLOCK_BYTES / 4;
  size_t bytes = (size_t)a.M * (cb * 64 + 4) * 4 + (size_t)cb * 16 * 4 + (size_t)WAVES * (UDW + 64) * 4;
  const size_t red = (size_t)WAVES * 64 * 16;
  if (bytes < red) bytes = red;
  const int64_t grid = (a.N + 15) / 16;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemv_kernel<FMT, QMAX, WAVES>), dim3((unsigned)grid), dim3(WAVES * 64), bytes, stream, a,
                     (int)cb, lowrank_vec(a));
  return hipGetLastError();
}

template <int FMT, int WAVES>
static hipError_t run_gemv_w(const LinearArgs& a, hipStream_t stream) {
  const int64_t KB = a.K / BLOCK_K;
  const int M = (int)a.M;
  // Blocks staged per chunk: activations within GEMV_X_BYTES of LDS, and at
  // most QMAX four-block units per wave.
  const int64_t units = (KB + 3) / 4;
  const int qmax = units <= WAVES ? 1 : units <= 2 * WAVES ? 2 : units <= 3 * WAVES ? 3 : 6;
  int64_t cb = GEMV_X_BYTES / (M * 256 + 64);
  if (cb > (int64_t)WAVES * qmax * 4) cb = (int64_t)WAVES * qmax * 4;
  if (cb > KB) cb = KB;
  if (cb < 1) cb = 1;
  if (qmax == 1) return launch_gemv<FMT, 1, WAVES>(a, cb, stream);
  if (qmax == 2) return launch_gemv<FMT, 2, WAVES>(a, cb, stream);
  if (qmax == 3) return launch_gemv<FMT, 3, WAVES>(a, cb, stream);
  return launch_gemv<FMT, 6, WAVES>(a, cb, stream);
}

// Eight waves per workgroup while the grid fits in one dispatch round at two
// workgroups per CU, four waves (four workgroups per CU) beyond that.
template <int FMT>
static hipError_t run_gemv(const LinearArgs& a, hipStream_t stream) {
  const int64_t grid = (a.N + 15) / 16;
  if (grid <= 384) return run_gemv_w<FMT, 8>(a, stream);
  return run_gemv_w<FMT, 4>(a, stream);
}

// Row tiles per group of the K-group tile order.  Cutting the tile grid into
// p row parts times 8 / p column parts, one block per XCD, makes the XCDs
// together read the weights p times and x 8 / p times, the latter only while
// an XCD's rows of x stay in its 4 MB L2: an XCD runs one tile per CU (32 at
// once), row-fastest through its block, so when the block takes several such
// rounds and its rows of x exceed ~2.5 MB, every round reads them again.  p is
// the power of two (at most the row-tile count) with the least modelled sum.
template <int FMT>
static int kgroup_group_rows(const LinearArgs& a, int bm, int tiles_m, int tiles_n, int nparts) {
  const double xrow = 2.0 * (double)std::min<int64_t>(bm, a.M) * (double)a.K;   // one row tile of x
  const double wb = (double)a.N * (double)a.K * (FMT == 0 ? 0.265625 : 0.53125);
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

// y = 0 before a K-split GEMM adds its two parts into it: 16-byte stores
// from the first 16-byte boundary of y on, single floats before it and after
// the last whole piece.
__global__ __launch_bounds__(256) void zero_y_kernel(float* y, int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t head = (int64_t)(((16u - (uint32_t)(reinterpret_cast<uintptr_t>(y) & 15u)) & 15u) >> 2);
  head = head < count ? head : count;
  const int64_t pieces = (count - head) >> 2;
  q2_f32x4* v = reinterpret_cast<q2_f32x4*>(y + head);
  for (int64_t i = t0; i < pieces; i += stride) v[i] = q2_f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t tail = head + 4 * pieces;
  if (t0 < head) y[t0] = 0.0f;
  if (t0 < count - tail) y[tail + t0] = 0.0f;
}

hipError_t launch_zero_y(float* y, int64_t count, hipStream_t stream) {
  const int64_t blocks = std::min<int64_t>((count / 4 + 255) / 256 + 1, 4096);
  hipLaunchKernelGGL(zero_y_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y, count);
  return hipGetLastError();
}

// ksplit 2: the K blocks in two parts, each tile's two workgroups adding
// into y (zeroed first).  Two fp32 additions onto zero give the same result in
// either order, so a split call is still run-to-run deterministic; it cannot
// accumulate onto an existing y for the same reason.
template <int FMT, int MT, int NT, int KG, int NSET>
static hipError_t run_gemm_kgroup(const LinearArgs& a, int ksplit, hipStream_t stream) {
  constexpr int BM = 16 * MT, BN = 64 * NT;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles = tiles_m * ((a.N + BN - 1) / BN);
  const int64_t KB = a.K / BLOCK_K;
  // The rank-r branch (Q2_0, r <= LR_RMAX) rides in the prologue; of a split
  // tile only the first part adds it.
  if ((a.r > 0 && (FMT != 0 || a.r > LR_RMAX)) || (ksplit == 2 && a.acc) || (ksplit != 1 && ksplit != 2))
    return hipErrorInvalidValue;
  const int kpart = (ksplit == 2) ? (int)((KB + 1) / 2) : 0;
  const int64_t grid = tiles * (kpart > 0 ? 2 : 1);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (kpart > 0) {
    const hipError_t e = launch_zero_y(a.y, a.M * a.N, stream);
    if (e != hipSuccess) return e;
  }
  const int group_m = kgroup_group_rows<FMT>(a, BM, (int)tiles_m, (int)((a.N + BN - 1) / BN), kpart > 0 ? 2 : 1);
  if constexpr (FMT == 0) {
    if (a.r > 0) {
      hipLaunchKernelGGL((gemm_kgroup_kernel<FMT, MT, NT, KG, NSET, true>), dim3((unsigned)grid), dim3(256 * KG), 0,
                         stream, a, (int)tiles_m, group_m, kpart);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kgroup_kernel<FMT, MT, NT, KG, NSET, false>), dim3((unsigned)grid), dim3(256 * KG), 0,
                     stream, a, (int)tiles_m, group_m, kpart);
  return hipGetLastError();
}

// GEMM kernel configurations.  The automatic choice picks one of them; tests
// can force any by name (gemm_config_id), so every configuration is exercised
// whatever shapes the automatic choice gives it.
static const char* const kGemmCfgNames[] = {"auto",    "w48x192", "w96x192", "w64x128", "w32x128",
                                            "w32x64",  "kg2x1x4", "kg4x2x2", "kg2x1x2", "kg2x2x4",
                                            "kg2x2x2", "kg2x1x4r3", "kg6x3x2"};
enum GemmCfg { CFG_AUTO, CFG_W48x192, CFG_W96x192, CFG_W64x128, CFG_W32x128, CFG_W32x64, CFG_KG2x1x4, CFG_KG4x2x2,
               CFG_KG2x1x2, CFG_KG2x2x4, CFG_KG2x2x2, CFG_KG2x1x4R3, CFG_KG6x3x2, CFG_COUNT };
static_assert(sizeof kGemmCfgNames / sizeof kGemmCfgNames[0] == CFG_COUNT, "configuration names");

int gemm_config_id(const char* name) {
  for (int i = 0; i < CFG_COUNT; ++i)
    if (std::strcmp(name, kGemmCfgNames[i]) == 0) return i;
  return -1;
}

template <int FMT>
static hipError_t run_gemm_cfg(const LinearArgs& a, int cfg, int ksplit, hipStream_t stream) {
  if (cfg < CFG_KG2x1x4 && ksplit != 1) return hipErrorInvalidValue;   // only K-group tiles split K
  switch (cfg) {
    case CFG_W48x192: return run_gemm<FMT, 48, 192>(a, stream);
    case CFG_W96x192: return run_gemm<FMT, 96, 192>(a, stream);
    case CFG_W64x128: return run_gemm<FMT, 64, 128>(a, stream);
    case CFG_W32x128: return run_gemm<FMT, 32, 128>(a, stream);
    case CFG_W32x64: return run_gemm<FMT, 32, 64>(a, stream);
    case CFG_KG2x1x4: return run_gemm_kgroup<FMT, 2, 1, 4, 2>(a, ksplit, stream);
    case CFG_KG4x2x2: return run_gemm_kgroup<FMT, 4, 2, 2, 2>(a, ksplit, stream);
    case CFG_KG2x1x2: return run_gemm_kgroup<FMT, 2, 1, 2, 2>(a, ksplit, stream);
    case CFG_KG2x2x4: return run_gemm_kgroup<FMT, 2, 2, 4, 2>(a, ksplit, stream);
    case CFG_KG2x2x2: return run_gemm_kgroup<FMT, 2, 2, 2, 2>(a, ksplit, stream);
    case CFG_KG2x1x4R3: return run_gemm_kgroup<FMT, 2, 1, 4, 3>(a, ksplit, stream);
    case CFG_KG6x3x2: return run_gemm_kgroup<FMT, 6, 3, 2, 2>(a, ksplit, stream);
    default: return hipErrorInvalidValue;
  }
}

// A GEMM launch: kernel configuration and K parts (1 or 2).
struct GemmChoice {
  int cfg, ksplit;
};

template <int FMT>
static int gemm_auto_cfg(const LinearArgs& a) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  const bool lr_lds = FMT == 0 && a.r > 0 && a.r <= LR_RMAX && lowrank_vec(a);
  // The K-group kernels carry the rank-r branch (Q2_0, any r <= LR_RMAX) in
  // their prologue, so they take those calls as they take plain ones.
  const bool kg_ok = a.r == 0 || (FMT == 0 && a.r <= LR_RMAX);
  const int64_t KB = a.K / BLOCK_K;
  // Up to 384 rows: K-group tiles, the widest whose workgroup count still
  // covers a good part of the chip (measured on the 3072 / 9216 / 12288 and
  // 2560 / 9728 shapes); Q2_0 with long K keeps a third set in flight.
  if (kg_ok && a.M <= 384) {
    const int narrow = (FMT == 0 && KB >= 64) ? CFG_KG2x1x4R3 : CFG_KG2x1x4;
    if (a.M <= 64) return tiles(32, 128) >= 128 ? CFG_KG2x2x4 : narrow;
    if (a.M <= 128) return tiles(64, 128) >= 128 ? CFG_KG4x2x2 : narrow;
    if (a.M <= 256) return tiles(32, 128) >= 400 ? (FMT == 0 ? CFG_KG2x2x2 : CFG_KG2x1x2) : CFG_KG2x2x4;
    if (tiles(96, 192) >= 128) return CFG_KG6x3x2;
    return tiles(64, 128) >= 128 ? CFG_KG4x2x2 : CFG_KG2x2x4;
  }
  if (kg_ok) {
    if (a.M <= 640) return tiles(32, 128) >= 400 ? CFG_KG2x2x2 : CFG_KG4x2x2;
    // The 96 x 192 K-group tile for any M once it gives enough workgroups,
    // else two 48 x 192 workgroups per CU.
    if (tiles(96, 192) >= 160) return CFG_KG6x3x2;
    if (a.M >= 48 && tiles(48, 192) >= 256) return CFG_W48x192;
  }
  // Otherwise (a branch of rank above LR_RMAX or with the 4-bit format, or
  // few tiles) the four-wave kernel, with the largest tile that still gives a
  // few waves of workgroups over the 256 compute units.  48 x 192 tiles run
  // two workgroups (eight waves) per CU; with the low-rank
  // operands staged in LDS the tile no longer fits twice, so that case keeps 96 x 192.
  if (!lr_lds && a.M >= 48 && tiles(48, 192) >= 512) return CFG_W48x192;
  if (a.M >= 96 && tiles(96, 192) >= 256) return CFG_W96x192;
  if (a.M >= 64 && tiles(64, 128) >= 256) return CFG_W64x128;
  if (tiles(32, 128) >= 256) return CFG_W32x128;
  return CFG_W32x64;
}

// Long K over few tiles (K >= 8192, without the branch or accumulation): the
// K blocks in two parts, so twice the workgroups share the chip.  Measured at
// K = 9728 / 12288, N = 2560 / 3072: 20-27 % off at M <= 64, 7-8 % at
// M = 128, 11-14 % for Q2_0 at 384 and 512 rows; at 256 rows, and for the
// 4-bit format beyond 128 rows, no configuration gained enough to switch.
template <int FMT>
static GemmChoice gemm_auto_choice(const LinearArgs& a) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  if ((a.r == 0 || (FMT == 0 && a.r <= LR_RMAX)) && !a.acc && a.K / BLOCK_K >= 64) {
    if (a.M <= 64 && tiles(32, 64) < 256) return {FMT == 0 ? CFG_KG2x1x4R3 : CFG_KG2x1x4, 2};
    if (a.M <= 128 && tiles(32, 128) < 256) return {CFG_KG2x2x4, 2};
    if (FMT == 0 && a.M > 256 && a.M <= 640 && tiles(96, 192) < 128) return {CFG_KG6x3x2, 2};
  }
  return {gemm_auto_cfg<FMT>(a), 1};
}

template <int FMT>
static hipError_t run_gemm_auto(const LinearArgs& a, int force_cfg, int force_ksplit, hipStream_t stream) {
  GemmChoice ch = force_cfg > 0 ? GemmChoice{force_cfg, 1} : gemm_auto_choice<FMT>(a);
  if (force_ksplit > 0) ch.ksplit = force_ksplit;
  return run_gemm_cfg<FMT>(a, ch.cfg, ch.ksplit, stream);
}

hipError_t launch_linear(const LinearArgs& a, int fmt, int force_path, int force_cfg, int force_ksplit,
                         hipStream_t stream) {
  const bool gemv = force_path == 1 || (force_path == 0 && a.M <= 16);
  if (gemv && a.M > 16) return hipErrorInvalidValue;
  if (gemv) {
    if (force_ksplit > 1) return hipErrorInvalidValue;
    return fmt == 0 ? run_gemv<0>(a, stream) : run_gemv<1>(a, stream);
  }
  return fmt == 0 ? run_gemm_auto<0>(a, force_cfg, force_ksplit, stream)
                  : run_gemm_auto<1>(a, force_cfg, force_ksplit, stream);
}

hipError_t launch_lowrank_t(const uint16_t* x, const uint16_t* A, uint16_t* tl, int64_t M, int64_t K, int r,
                            hipStream_t stream) {
  const int64_t gx = (M + 15) / 16;
  const int gy = (lr_pad(r) + 15) / 16;
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lowrank_t_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(LR_WAVES * 64), 0, stream, x, A, tl, M,
                     K, r);
  return hipGetLastError();
}

}  // namespace q2dev
