// q2_linear.hip - the Q2_0 ternary linear (and the 4-bit variant) on CDNA4.
//
// Two kernels compute y = x W^T for packed weights:
//  * gemm_kernel (M > 16): a workgroup owns a BM x BN output tile; its four
//    waves split the tile along N.  Per 128-wide K block the workgroup stages
//    the activation rows into LDS (in the weight decoder's pair order, plus the
//    per-row block sum), each wave loads its rows' packed codes straight from
//    HBM into registers, decodes them into bf16 matrix-core operands and runs
//    16x16x32 bf16 MFMAs into a per-block accumulator that is scaled by the
//    block's f16 scale into the fp32 result.  Activations of block b+1 and
//    weights of block b+1 are fetched while block b computes.
//  * gemv_kernel (M <= 16): a workgroup owns 16 weight rows (one MFMA column
//    tile); its waves split K block by block, stream the packed codes with
//    coalesced loads and finish with a fixed-order cross-wave reduction, so
//    there is one HBM pass over the weights and no atomics.
// The rank-r side branch y += (x A^T) B^T is added in both epilogues with
// extra MFMA steps over the bf16 limbs of x A^T (computed once per call by
// lowrank_t_kernel) and the exact bf16 hi/lo split of B.
//
// Every summation order is fixed, so results are bitwise reproducible.
#include "q2_device.h"
#include "q2_internal.h"

namespace q2dev {
#ifndef SCHED_FENCE
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
#endif

template <int FMT> struct WFmt;
template <> struct WFmt<0> {           // Q2_0: 32 bytes of codes per row and block
  static constexpr int BLOCK_BYTES = 32;
  static constexpr int LANE_DW = 2;    // lane group g holds dwords 2g, 2g+1
};
template <> struct WFmt<1> {           // 4-bit: 64 bytes per row and group
  static constexpr int BLOCK_BYTES = 64;
  static constexpr int LANE_DW = 4;    // lane group g holds dwords 4g .. 4g+3
};

// Packed codes, scale and zero point of one block of one weight row.  The row
// index must already be clamped to a valid row: rows past N load row N-1,
// whose outputs are computed but never stored, so loads never branch.
template <int FMT>
__device__ __forceinline__ void load_wblock(const LinearArgs& a, int64_t row, int64_t blk, int g,
                                            uint32_t (&out)[WFmt<FMT>::LANE_DW], float& sc, float& zp) {
  constexpr int DW = WFmt<FMT>::LANE_DW;
  const int64_t row_bytes = (FMT == 0) ? a.K / 4 : a.K / 2;
  const uint8_t* p = a.w + row * row_bytes + blk * WFmt<FMT>::BLOCK_BYTES + g * DW * 4;
  if constexpr (DW == 2) {
    const q2_u32x2 v = *reinterpret_cast<const q2_u32x2*>(p);
    out[0] = v[0]; out[1] = v[1];
  } else {
    const q2_u32x4 v = *reinterpret_cast<const q2_u32x4*>(p);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  }
  const int64_t si = row * (a.K / BLOCK_K) + blk;
  sc = f16_to_f32(a.s[si]);
  zp = (FMT == 1) ? f16_to_f32(a.z[si]) : 0.f;
}

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

// ---- low-rank epilogue operands -------------------------------------------
// A'' = [T_hi, T_hi, T_lo] (row m of the limbs), B'' = [B_hi, B_lo, B_hi] (row n of B),
// so sum_q A''[m,q] B''[n,q] = T_hi B_hi + T_hi B_lo + T_lo B_hi.  With r % 8 == 0 the
// eight elements of a lane group lie in one part and one aligned 16-byte run.
__device__ __forceinline__ q2_u32x4 lr_afrag(const uint16_t* tl, int64_t m, int r, int q0, bool vec) {
  if (q0 >= 3 * r) return q2_u32x4{0u, 0u, 0u, 0u};
  if (vec) {
    const int part = q0 / r, jj = q0 - part * r;
    return *reinterpret_cast<const q2_u32x4*>(tl + m * 2 * r + (part == 2 ? r : 0) + jj);
  }
  uint32_t e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = q0 + k;
    uint32_t v = 0;
    if (q < 3 * r) {
      const int part = q / r, jj = q - part * r;
      v = tl[m * 2 * r + (part == 2 ? r : 0) + jj];
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
constexpr int XSTRIDE = 68;   // dwords per staged row-block: 64 pair dwords + 4 pad (bank spread)

template <int FMT, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_kernel(LinearArgs a, int tiles_m, int lr_vec) {
  constexpr int MT = BM / 16;            // 16-row tiles per wave
  constexpr int NT = BN / 64;            // 16-column tiles per wave (4 waves along N)
  constexpr int CPT = BM / 32;           // 16-element staging chunks per thread per block
  constexpr int DW = WFmt<FMT>::LANE_DW;
  static_assert(BM % 32 == 0 && BN % 64 == 0, "tile shape");

  __shared__ __align__(16) uint32_t xs[2][BM * XSTRIDE];
  __shared__ __align__(16) float ss[2][BM];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t nw = (int64_t)tn * BN + wv * (BN / 4);   // first row of W for this wave
  const int64_t M = a.M, K = a.K, KB = K / BLOCK_K;
  const DecodeConsts kc = (FMT == 0) ? q2_consts() : q4_consts();

  const int part = tid & 7;
  const int row0 = tid >> 3;
  int64_t xrow[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int64_t r = m0 + row0 + 32 * q;
    xrow[q] = r < M ? r : M - 1;
  }
  int64_t wrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t r = nw + 16 * j + c;
    wrow[j] = r < a.N ? r : a.N - 1;
  }

  auto x_load = [&](uint32_t (&xr)[CPT][8], int64_t blk) {
    blk = blk < KB ? blk : KB - 1;
#pragma unroll
    for (int q = 0; q < CPT; ++q) load_x16(a.x, xrow[q], K, blk * BLOCK_K + part * 16, xr[q]);
  };
  auto x_store = [&](const uint32_t (&xr)[CPT][8], int buf) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int row = row0 + 32 * q;
      uint32_t pr[8];
      stage_pairs<FMT>(xr[q], pr);
      q2_u32x4* dst = reinterpret_cast<q2_u32x4*>(&xs[buf][row * XSTRIDE + part * 8]);
      dst[0] = q2_u32x4{pr[0], pr[1], pr[2], pr[3]};
      dst[1] = q2_u32x4{pr[4], pr[5], pr[6], pr[7]};
      const float sm = sum8_lanes(bf16_sum16(xr[q]));
      if (part == 0) ss[buf][row] = sm * ((FMT == 0) ? -1.25f : -1.f);
    }
  };
  auto w_load = [&](uint32_t (&w)[NT][DW], float (&d)[NT], float (&z)[NT], int64_t blk) {
    blk = blk < KB ? blk : KB - 1;
#pragma unroll
    for (int j = 0; j < NT; ++j) load_wblock<FMT>(a, wrow[j], blk, g, w[j], d[j], z[j]);
  };

  q2_f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = q2_f32x4{0.f, 0.f, 0.f, 0.f};

  // One block: decode this wave's weights, refill their registers with the
  // block two ahead, then run the MFMAs over the staged activations.
  auto compute = [&](int buf, uint32_t (&w)[NT][DW], float (&d)[NT], float (&z)[NT], int64_t next_blk) {
    q2_u32x4 bf[NT][4];
    float dc[NT], zc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      decode_block<FMT>(w[j], bf[j], kc);
      dc[j] = d[j];
      zc[j] = z[j];
    }
    w_load(w, d, z, next_blk);
    // A fragments of tile i+1 are read from LDS while tile i's MFMAs run;
    // tile i's MFMAs are issued before tile i-1's rescale so the FMAs run in
    // the matrix core's shadow; two temporaries keep everything in VGPRs.
    q2_f32x4 t0[NT], t1[NT];
    q2_u32x4 a0[4], a1[4];
    q2_f32x4 s0, s1;
    auto rd = [&](int i, q2_u32x4 (&av)[4], q2_f32x4& s4) {
      s4 = *reinterpret_cast<const q2_f32x4*>(&ss[buf][16 * i + 4 * g]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        av[t] = *reinterpret_cast<const q2_u32x4*>(&xs[buf][(16 * i + c) * XSTRIDE + 16 * g + 4 * t]);
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
      SCHED_FENCE();
    }
    if ((MT - 1) & 1) rescale(MT - 1, t1);
    else rescale(MT - 1, t0);
  };

  if (KB > 0) {
    uint32_t xA[CPT][8], xB[CPT][8];
    uint32_t wA[NT][DW], wB[NT][DW];
    float dA[NT], dB[NT], zA[NT], zB[NT];
    x_load(xA, 0);
    w_load(wA, dA, zA, 0);
    x_load(xB, 1);
    w_load(wB, dB, zB, 1);
    x_store(xA, 0);
    x_load(xA, 2);
    __syncthreads();
    // Steady state at block b: LDS[b&1] holds X(b); the other X registers
    // hold X(b+1) (to be staged after this block) and X(b+2) (in flight).
    for (int64_t b = 0; b < KB; b += 2) {
      compute(0, wA, dA, zA, b + 2);
      if (b + 1 < KB) x_store(xB, 1);
      x_load(xB, b + 3);
      __syncthreads();
      if (b + 1 >= KB) break;
      compute(1, wB, dB, zB, b + 3);
      if (b + 2 < KB) x_store(xA, 0);
      x_load(xA, b + 4);
      __syncthreads();
    }
  }

  const float fin = (FMT == 0) ? 4.f : 16.f;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] *= fin;

  if (a.r > 0) {
    const int ks = (3 * a.r + 31) / 32;
    for (int t = 0; t < ks; ++t) {
      const int q0 = 32 * t + 8 * g;
      q2_u32x4 bq[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) bq[j] = lr_bfrag(a.lr_b, wrow[j], a.r, q0, lr_vec != 0);
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

#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t n = nw + 16 * j + c;
      if (n < a.N) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t m = m0 + 16 * i + 4 * g + e;
          if (m < M) a.y[m * a.N + n] = acc[i][j][e];
        }
      }
    }
  }
}

// ============================================================================
// GEMV, M <= 16
// ============================================================================
#ifndef Q2_GEMV_WAVES
#define Q2_GEMV_WAVES 8
#endif
constexpr int GEMV_WAVES = Q2_GEMV_WAVES;
constexpr int GEMV_XQ = 2048 / (GEMV_WAVES * 64);   // 16-activation staging chunks per thread per chunk of K
constexpr int GEMV_X_ROWBLOCKS = 256;             // (row, block) pairs staged per chunk: 64 KB of LDS

template <int FMT, int QMAX>
__global__ __launch_bounds__(GEMV_WAVES * 64) void gemv_kernel(LinearArgs a, int cb, int lr_vec) {
  constexpr int DW = WFmt<FMT>::LANE_DW;
  extern __shared__ __align__(16) uint32_t smem[];
  const int M = (int)a.M;
  const int rs = cb * 64 + 4;                     // dwords per staged row
  uint32_t* xs = smem;
  float* ss = reinterpret_cast<float*>(smem + M * rs);   // [cb][16]

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t n = (int64_t)blockIdx.x * 16 + c;        // weight row of this lane's MFMA column
  const int64_t nc = n < a.N ? n : a.N - 1;              // rows past N recompute row N-1, never stored
  const int64_t K = a.K, KB = K / BLOCK_K;
  const int crow = c < M ? c : M - 1;                    // activation rows past M duplicate row M-1
  const DecodeConsts kc = (FMT == 0) ? q2_consts() : q4_consts();
  const uint8_t* wbase = a.w + nc * ((FMT == 0) ? K / 4 : K / 2) + g * DW * 4;
  const uint16_t* sbase = a.s + nc * KB;
  const uint16_t* zbase = (FMT == 1) ? a.z + nc * KB : nullptr;

  q2_f32x4 acc = q2_f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t cb0 = 0; cb0 < KB; cb0 += cb) {
    const int nb = (int)((KB - cb0) < cb ? (KB - cb0) : cb);
    const int mine = (nb - wv + GEMV_WAVES - 1) / GEMV_WAVES;   // blocks wv, wv + 8, ... of this chunk
    const int nchunks = M * nb * 8;
    // activation loads first, so that staging waits on them only
    uint32_t nx[GEMV_XQ][8];
#pragma unroll
    for (int u = 0; u < GEMV_XQ; ++u) {
      const int idx = tid + u * GEMV_WAVES * 64;
      if (idx < nchunks) {                       // masked lanes issue no memory traffic
        const int row = idx / (nb * 8);
        const int rem = idx - row * nb * 8;
        load_x16(a.x, row, K, (cb0 + (rem >> 3)) * BLOCK_K + (rem & 7) * 16, nx[u]);
      }
    }
    // then every weight load of this wave's share of the chunk
    uint32_t wq[QMAX][DW];
    float dq[QMAX], zq[QMAX];
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      int bl = wv + GEMV_WAVES * q;
      bl = bl < nb ? bl : nb - 1;
      const uint32_t blk = (uint32_t)(cb0 + bl);
      const uint8_t* p = wbase + (uint64_t)blk * WFmt<FMT>::BLOCK_BYTES;
      if constexpr (DW == 2) {
        const q2_u32x2 v = *reinterpret_cast<const q2_u32x2*>(p);
        wq[q][0] = v[0]; wq[q][1] = v[1];
      } else {
        const q2_u32x4 v = *reinterpret_cast<const q2_u32x4*>(p);
        wq[q][0] = v[0]; wq[q][1] = v[1]; wq[q][2] = v[2]; wq[q][3] = v[3];
      }
      dq[q] = f16_to_f32(sbase[blk]);
      zq[q] = (FMT == 1) ? f16_to_f32(zbase[blk]) : 0.f;
    }
    // stage the activations in the decoder's pair order, with pre-scaled block sums
#pragma unroll
    for (int u = 0; u < GEMV_XQ; ++u) {
      const int idx = tid + u * GEMV_WAVES * 64;
      if (u * GEMV_WAVES * 64 >= nchunks) break;          // uniform: no chunk left for any thread
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
    for (int idx = tid; idx < nb * 16; idx += GEMV_WAVES * 64)
      if ((idx & 15) >= M) ss[idx] = 0.f;
    __syncthreads();

#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      if (q < mine) {
        const int bl = wv + GEMV_WAVES * q;
        q2_u32x4 bf[4];
        decode_block<FMT>(wq[q], bf, kc);
        const q2_f32x4 s4 = *reinterpret_cast<const q2_f32x4*>(&ss[bl * 16 + 4 * g]);
        q2_f32x4 tmp = block_cinit<FMT>(s4, zq[q]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          tmp = mfma(*reinterpret_cast<const q2_u32x4*>(&xs[crow * rs + bl * 64 + 16 * g + 4 * t]), bf[t], tmp);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(dq[q], tmp[e], acc[e]);
      }
    }
    __syncthreads();
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
    if (a.r > 0) {
      const int ks = (3 * a.r + 31) / 32;
      for (int t = 0; t < ks; ++t) {
        const int q0 = 32 * t + 8 * g;
        s = mfma(lr_afrag(a.lr_t, crow, a.r, q0, lr_vec != 0), lr_bfrag(a.lr_b, nc, a.r, q0, lr_vec != 0), s);
      }
    }
    if (n < a.N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * g + e;
        if (m < M) a.y[(int64_t)m * a.N + n] = s[e];
      }
    }
  }
}

// ============================================================================
// x A^T for the low-rank branch: bf16 limbs [M, 2r] = (hi | lo)
// ============================================================================
constexpr int LR_WAVES = 16;
constexpr int LR_UNROLL = 2;     // k-steps whose loads are issued together

__global__ __launch_bounds__(LR_WAVES * 64) void lowrank_t_kernel(const uint16_t* x, const uint16_t* A, uint16_t* tl,
                                                                  int64_t M, int64_t K, int r) {
  __shared__ __align__(16) q2_f32x4 red[LR_WAVES][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  int64_t m = (int64_t)blockIdx.x * 16 + c;                // A-operand row of this lane
  m = m < M ? m : M - 1;
  const int col0 = blockIdx.y * 64;
  const int ntl = (r - col0 + 15) / 16 < 4 ? (r - col0 + 15) / 16 : 4;   // live 16-column tiles
  const int64_t KS = K / 32;
  q2_f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = q2_f32x4{0.f, 0.f, 0.f, 0.f};
  int colc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = col0 + 16 * j + c;
    colc[j] = col < r ? col : r - 1;
  }

  for (int64_t s0 = wv; s0 < KS; s0 += (int64_t)LR_WAVES * LR_UNROLL) {
    q2_u32x4 av[LR_UNROLL], bv[LR_UNROLL][4];
#pragma unroll
    for (int u = 0; u < LR_UNROLL; ++u) {
      int64_t s = s0 + (int64_t)LR_WAVES * u;
      s = s < KS ? s : KS - 1;
      const int64_t k0 = s * 32 + 8 * g;
      av[u] = *reinterpret_cast<const q2_u32x4*>(x + m * K + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < ntl) bv[u][j] = *reinterpret_cast<const q2_u32x4*>(A + (int64_t)colc[j] * K + k0);
    }
#pragma unroll
    for (int u = 0; u < LR_UNROLL; ++u) {
      if (s0 + (int64_t)LR_WAVES * u < KS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < ntl) {
            q2_u32x4 bh, bl;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              uint16_t h0, l0, h1, l1;
              f16_split_bf16((uint16_t)(bv[u][j][d] & 0xFFFFu), h0, l0);
              f16_split_bf16((uint16_t)(bv[u][j][d] >> 16), h1, l1);
              bh[d] = (uint32_t)h0 | ((uint32_t)h1 << 16);
              bl[d] = (uint32_t)l0 | ((uint32_t)l1 << 16);
            }
            acc[j] = mfma(av[u], bh, acc[j]);
            acc[j] = mfma(av[u], bl, acc[j]);
          }
        }
      }
    }
  }
  for (int j = 0; j < 4; ++j) {
    if (j >= ntl) break;
    red[wv][lane] = acc[j];
    __syncthreads();
    if (wv == 0) {
      q2_f32x4 sm = red[0][lane];
#pragma unroll
      for (int w = 1; w < LR_WAVES; ++w) {
        const q2_f32x4 o = red[w][lane];
        sm = q2_f32x4{sm[0] + o[0], sm[1] + o[1], sm[2] + o[2], sm[3] + o[3]};
      }
      const int col = col0 + 16 * j + c;            // C layout: column = lane % 16
      if (col < r) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = (int64_t)blockIdx.x * 16 + 4 * g + e;
          if (row < M) {
            const float t = sm[e];
            const uint16_t hi = f32_to_bf16_rn(t);
            const uint16_t lo = f32_to_bf16_rn(t - bf16_to_f32(hi));
            tl[row * 2 * r + col] = hi;
            tl[row * 2 * r + r + col] = lo;
          }
        }
      }
    }
    __syncthreads();
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
  hipLaunchKernelGGL((gemm_kernel<FMT, BM, BN>), dim3((unsigned)tiles), dim3(256), 0, stream, a, (int)tiles_m,
                     lowrank_vec(a));
  return hipGetLastError();
}

template <int FMT>
static hipError_t run_gemv(const LinearArgs& a, hipStream_t stream) {
  const int64_t KB = a.K / BLOCK_K;
  const int M = (int)a.M;
  // blocks staged per chunk: at most 256 (row, block) pairs of activations, and
  // at most QMAX blocks per wave
  const int qmax = KB <= (int64_t)GEMV_WAVES * 4 ? 4 : (KB <= (int64_t)GEMV_WAVES * 8 ? 8 : 12);
  int64_t cb = GEMV_X_ROWBLOCKS / M;
  if (cb > (int64_t)GEMV_WAVES * qmax) cb = (int64_t)GEMV_WAVES * qmax;
  if (cb > KB) cb = KB;
  if (cb < 1) cb = 1;
  size_t bytes = (size_t)M * (cb * 64 + 4) * 4 + (size_t)cb * 16 * 4;
  const size_t red = (size_t)GEMV_WAVES * 64 * 16;
  if (bytes < red) bytes = red;
  const int64_t grid = (a.N + 15) / 16;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (qmax == 4)
    hipLaunchKernelGGL((gemv_kernel<FMT, 4>), dim3((unsigned)grid), dim3(GEMV_WAVES * 64), bytes, stream, a,
                       (int)cb, lowrank_vec(a));
  else if (qmax == 8)
    hipLaunchKernelGGL((gemv_kernel<FMT, 8>), dim3((unsigned)grid), dim3(GEMV_WAVES * 64), bytes, stream, a,
                       (int)cb, lowrank_vec(a));
  else
    hipLaunchKernelGGL((gemv_kernel<FMT, 12>), dim3((unsigned)grid), dim3(GEMV_WAVES * 64), bytes, stream, a,
                       (int)cb, lowrank_vec(a));
  return hipGetLastError();
}

template <int FMT>
static hipError_t run_gemm_auto(const LinearArgs& a, hipStream_t stream) {
  // Prefer the largest tile that still gives a few waves of workgroups over
  // the 256 compute units.
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  if (a.M >= 96 && tiles(96, 192) >= 256) return run_gemm<FMT, 96, 192>(a, stream);
  if (a.M >= 64 && tiles(64, 128) >= 256) return run_gemm<FMT, 64, 128>(a, stream);
  if (tiles(32, 128) >= 256) return run_gemm<FMT, 32, 128>(a, stream);
  return run_gemm<FMT, 32, 64>(a, stream);
}

hipError_t launch_linear(const LinearArgs& a, int fmt, int force_path, hipStream_t stream) {
  const bool gemv = force_path == 1 || (force_path == 0 && a.M <= 16);
  if (gemv && a.M > 16) return hipErrorInvalidValue;
  if (fmt == 0) return gemv ? run_gemv<0>(a, stream) : run_gemm_auto<0>(a, stream);
  return gemv ? run_gemv<1>(a, stream) : run_gemm_auto<1>(a, stream);
}

hipError_t launch_lowrank_t(const uint16_t* x, const uint16_t* A, uint16_t* tl, int64_t M, int64_t K, int r,
                            hipStream_t stream) {
  const int64_t gx = (M + 15) / 16;
  const int gy = (r + 63) / 64;
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lowrank_t_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(LR_WAVES * 64), 0, stream, x, A, tl, M,
                     K, r);
  return hipGetLastError();
}

}  // namespace q2dev
