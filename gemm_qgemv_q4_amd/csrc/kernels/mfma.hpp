// Prefill-M products on the gfx950 matrix cores, for every weight format
// whose values are a per-group affine map of small integer codes:
//
// y[m, n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k]  +  sum_g b[n,g] * X_g[m]
// with X_g[m] = sum_{k in g} x[m,k]:
//   affine (u8 or packed codes): s, b from the scale and bias tensors
//                                         [mlx-native qmm_affine.rs]
//   Q4_0: groups of 32 with the signed codes 16 (q - 8), s = d / 16, no bias
//                                         [mlx-native fused_dual_proj_q4_0.rs]
//   Q4_K: groups of 32 (sub-blocks), s = d * sc_j, b = -dmin * m_j
//                                         [ferrum-kernels q4_k_gemv_v2.rs]
//
// Precision: the codes (0..255, or -128..112 for Q4_0) are exact in bf16, so
// a Q4_0 block of codes 8 adds exactly 0.  x is split once into
// x_hi = bf16(x) and x_lo = bf16(x - x_hi), so x_hi + x_lo carries 16
// significant bits (relative error <= 2^-17); bf16 x bf16 products are exact
// in the f32 MFMA accumulator.  Each group's partial product P_g = (x_hi +
// x_lo) . q is accumulated by two v_mfma_f32_16x16x32_bf16 per 32 columns and
// scaled in f32 (acc += s * P_g).  The bias term is a product over the group
// index with X and b both split into bf16 hi + lo (the lo*lo part, below
// 2^-16 relative, is dropped).  Together this keeps |y - y_exact| well inside
// 1e-5 * sum|x w|, which a single bf16 or f16 operand does not.
//
// Kernels:
//   affine_prep_kernel : x [M,K] f32 -> x_hi, x_lo [M,K] bf16 and X [M, K/gs]
//                        as bf16 hi, lo.
//   qmm_mfma_kernel<F, MULTI, SM, SN, TI> : a (16 TI SM) x (64 SN) output
//                        tile per workgroup of 2*SM*SN waves: SM x SN
//                        sub-tiles of (16 TI) x 64, each shared by two waves
//                        that split every 64-wide K stage.  Column tiles are
//                        numbered part after part (up to kMaxParts weight
//                        tensors sharing x), so a tile's part is uniform.
#pragma once
#include "common.hpp"

namespace qg {

// ---------------------------------------------------------------------------
// x -> (x_hi, x_lo) bf16 and per-group sums X_g, the sums also split into
// bf16 hi/lo (they feed the bias product on the matrix cores; sh == nullptr:
// no sums, for formats without a bias).  Each thread converts 8 consecutive
// elements; the gs/8 threads of a group (gs <= 512) combine their partial sums
// with a fixed-order DPP reduction.  Every store comes after all arithmetic:
// the vector memory counter also counts stores, so arithmetic placed after a
// store would wait for that store to complete.
__global__ void __launch_bounds__(256) affine_prep_kernel(const float* __restrict__ x,
                                                          __bf16* __restrict__ xh,
                                                          __bf16* __restrict__ xl,
                                                          __bf16* __restrict__ sh,
                                                          __bf16* __restrict__ sl,
                                                          int m_rows, int k, int gs) {
  const int per_row = k / 8;
  const int item = blockIdx.x * blockDim.x + threadIdx.x;  // < 2^31: M*K/8 is checked on the host
  const bool ok = item < m_rows * per_row;
  const int m = ok ? item / per_row : 0;
  const int c8 = ok ? item - m * per_row : 0;
  const size_t base = (size_t)m * k + (size_t)c8 * 8;
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (ok) {
    const bool vec = (reinterpret_cast<uintptr_t>(x + base) & 15u) == 0;
    if (vec) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(x + base);
      const f32x4 b = *reinterpret_cast<const f32x4*>(x + base + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = x[base + i];
    }
  }
  const bool sums = sh != nullptr;  // uniform across the grid
  const int lanes = gs / 8;         // threads per group (4..64)
  float s = 0.0f;
  __bf16 s_hi = (__bf16)0.0f, s_lo = (__bf16)0.0f;
  if (sums) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
    s = group_sum(s, lanes);
    s_hi = (__bf16)s;
    s_lo = (__bf16)(s - (float)s_hi);
  }
  bf16x8 hv, lv;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)v[i];
    hv[i] = h;
    lv[i] = (__bf16)(v[i] - (float)h);
  }
  if (ok) {
    *reinterpret_cast<bf16x8*>(xh + base) = hv;
    *reinterpret_cast<bf16x8*>(xl + base) = lv;
    if (sums && (c8 % lanes) == 0) {
      const size_t gi = (size_t)m * (k / gs) + c8 / lanes;
      sh[gi] = s_hi;
      sl[gi] = s_lo;
    }
  }
}

// One weight tensor of a product and where its outputs go.
struct MfmaPart {
  const uint8_t* w;       // row r at w + r * row_bytes
  const float* scales;    // affine formats: [n, K/gs]
  const float* biases;    // affine formats: [n, K/gs]
  float* y;               // output (m, r) at y[m * ldy + r]
  long long ldy;
  int n;                  // rows
  int tile0;              // first column tile of this part
};

struct MfmaParams {
  const __bf16* xh;      // [M, K]
  const __bf16* xl;      // [M, K]
  const __bf16* sh;      // [M, K/gs] group sums of x, hi
  const __bf16* sl;      // [M, K/gs] group sums of x, lo
  MfmaPart part[kMaxParts];
  int parts;
  long long row_bytes;   // bytes per weight row
  int m, k, gs;
  int tiles_m, tiles_n;  // tiles_n over all parts
  int xcd_mb;            // > 0: each XCD takes a block of xcd_mb row tiles by
                         // tiles/(8 xcd_mb) column tiles; 0: consecutive tiles
};

constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // bf16 elements per LDS row (144 bytes)

// Scale s[row, g] and bias b[row, g] of group g (group size 32 for the block
// formats) of weight row `row` of part `pt`.
template <int F>
__device__ __forceinline__ float group_scale(const MfmaPart& pt, long long row_bytes, int groups, int row,
                                             int g) {
  if constexpr (F == FMT_AFF || F == FMT_AFF4) {
    return pt.scales[(size_t)row * groups + g];
  } else if constexpr (F == FMT_Q40) {
    // the codes enter as 16 (q - 8): d / 16 is exact
    const uint16_t d = *(const uint16_t*)(pt.w + (size_t)row * row_bytes + 18 * (size_t)g);
    return f16_bits_to_f32(d) * 0.0625f;
  } else {
    const uint8_t* sb = pt.w + (size_t)row * row_bytes + 144 * (size_t)(g >> 3);
    int sc, mn;
    q4k_sc_m(sb + 4, g & 7, sc, mn);
    return f16_bits_to_f32(*(const uint16_t*)sb) * (float)sc;  // exact: 11 x 6 bits
  }
}
template <int F>
__device__ __forceinline__ float group_bias(const MfmaPart& pt, long long row_bytes, int groups, int row,
                                            int g) {
  static_assert(F != FMT_Q40, "Q4_0 has no bias term");
  if constexpr (F == FMT_AFF || F == FMT_AFF4) {
    return pt.biases[(size_t)row * groups + g];
  } else {
    const uint8_t* sb = pt.w + (size_t)row * row_bytes + 144 * (size_t)(g >> 3);
    int sc, mn;
    q4k_sc_m(sb + 4, g & 7, sc, mn);
    return -(f16_bits_to_f32(*(const uint16_t*)(sb + 2)) * (float)mn);
  }
}

// One 32-wide K step of the wave's (16 TI) x 64 sub-tile: P += (A_hi + A_lo) * B.
// All 16 hi products are issued before the 16 lo products, so consecutive
// MFMAs never wait on each other's accumulator.
template <bool FIRST, int TI>
__device__ __forceinline__ void mfma_substep(const __bf16* sAh, const __bf16* sAl, const __bf16* sB,
                                             int kq, int wm, int wn, int lane, f32x4 (&P)[TI][4]) {
  const int r16 = lane & 15;
  const int kk = (lane >> 4) * 8 + kq;
  bf16x8 bfrag[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bfrag[j] = *(const bf16x8*)(sB + (wn * 64 + j * 16 + r16) * kPitch + kk);
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const bf16x8 ah = *(const bf16x8*)(sAh + (wm * 16 * TI + i * 16 + r16) * kPitch + kk);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (FIRST) {
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        P[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bfrag[j], z, 0, 0, 0);
      } else {
        P[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bfrag[j], P[i][j], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const bf16x8 al = *(const bf16x8*)(sAl + (wm * 16 * TI + i * 16 + r16) * kPitch + kk);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      P[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bfrag[j], P[i][j], 0, 0, 0);
  }
}

// One workgroup computes a (16*TI*SM) x (64*SN) output tile: SM x SN
// sub-tiles of (16*TI) x 64, each owned by a pair of waves (TI x 4 MFMA tiles
// each), so the workgroup has 2*SM*SN waves.  With TI = 2 a wave holds 32
// accumulator tiles' worth of registers (acc and P), which leaves room for
// four waves per SIMD; the measured alternative, TI = 4 at two waves per
// SIMD, is 10-20% slower on every workload.  The two waves of a pair split
// every 64-wide K stage: wave half 0 takes columns 0..31, half 1 columns
// 32..63; their partial sums meet in LDS at the end.  K runs through two LDS
// buffers; each stage's global loads are issued one stage ahead into
// registers (one barrier per stage).  When a group of gs columns is complete,
// a wave scales its partial product: acc += s[n, g] * P.  The bias term
// sum_g b[n,g] * X_g[m] is one more small matrix product at the end, with
// both factors split into bf16 hi + lo (three MFMAs per 32 groups).  The
// arithmetic of one output element is the same for every (SM, SN, TI), so
// the host picks the tile shape from the tile count alone.
//
// BKS: 64-column K steps per barrier (1 or 2).  With 2, a stage is two
// consecutive steps, loaded, converted and multiplied together, in twice the
// LDS; each step's arithmetic is unchanged, so the bits are the same.
template <int F, bool MULTI, int SM, int SN, int TI, int BKS = 1>
__global__ void __launch_bounds__(128 * SM * SN, BKS == 1 ? 8 / TI : 2) qmm_mfma_kernel(MfmaParams p) {
  constexpr int T = 128 * SM * SN;  // threads
  constexpr int NSUB = SM * SN;
  constexpr int SUBM = 16 * TI;     // rows of a wave pair's sub-tile
  constexpr int BM = SUBM * SM, BN = 64 * SN;
  constexpr int A_ELEMS = BM * kPitch, B_ELEMS = BN * kPitch;
  constexpr int RA = BM * 8 / T;    // x rows each thread moves per stage (8 elements each, hi and lo)
  constexpr int NB = BN * 4;        // 16-code pieces of weights per stage
  constexpr int IB = NB >= T ? NB / T : 1;  // pieces per thread (threads past NB move none)
  static_assert(RA >= 1 && BM * 8 == RA * T, "x pieces must divide evenly over the threads");
  static_assert(BKS == 1 || BKS == 2, "one or two 64-column steps per stage");
  __shared__ __attribute__((aligned(16))) __bf16 sA[2 * BKS][2 * A_ELEMS];  // [buf][hi | lo]
  __shared__ __attribute__((aligned(16))) __bf16 sB[2 * BKS][B_ELEMS];
  __shared__ float sS[2 * BKS][2][BN];  // [buf][group in step][n]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int kh = wid / NSUB;  // which 32-column half of each stage
  const int sub = wid % NSUB;
  const int wm = sub / SN, wn = sub % SN;

  // The dispatcher spreads consecutive workgroup ids over the 8 XCDs, each
  // with its own L2.  With xcd_mb set, XCD x = id % 8 takes a block of xcd_mb
  // row tiles by nb column tiles, so that its L2 holds the x rows and the
  // weight rows of that block only (the host picks the block shape that
  // fetches the fewest bytes).  Otherwise each XCD takes a contiguous range of
  // tiles (row tiles fastest) when the count allows it.
  const int total = p.tiles_m * p.tiles_n;
  int tm, tn;  // tn: column tile over all parts
  if (p.xcd_mb > 0) {
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    const int rms = p.tiles_m / p.xcd_mb;  // blocks along the rows
    const int nb = (total >> 3) / p.xcd_mb;
    tm = (x % rms) * p.xcd_mb + i % p.xcd_mb;
    tn = (x / rms) * nb + i / p.xcd_mb;
  } else {
    int tile = blockIdx.x;
    if ((total & 7) == 0) tile = (tile & 7) * (total >> 3) + (tile >> 3);
    tm = tile % p.tiles_m;
    tn = tile / p.tiles_m;
  }
  // a single-part launch (MULTI false) reads part 0 at fixed argument offsets
  MfmaPart pt = p.part[0];
  if constexpr (MULTI) {
    // unused slots start past every tile (set by the host): fixed-offset
    // loads that leave together, no read of the part count
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxParts; ++i) pi = tn >= p.part[i].tile0 ? i : pi;
    pi = __builtin_amdgcn_readfirstlane(pi);
    pt = p.part[pi];
  }
  const int n_rows = pt.n;
  const int m0 = tm * BM, n0 = (tn - pt.tile0) * BN;  // n0: row of the part
  const int groups = p.k / p.gs;
  const int stages = p.k / kBK;
  const int ng = p.gs < kBK ? kBK / p.gs : 1;  // groups per stage: 2 when gs == 32

  f32x4 acc[TI][4], P[TI][4];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      P[i][j] = acc[i][j];
    }

  // Pieces this thread moves per stage: 8-element pieces of x_hi/x_lo rows
  // a_row0 + i*(T/8), and 16 codes of weight rows b_n[i] (codes 16*b_kc[i] ..
  // 16*b_kc[i]+15 of the stage's 64 columns).  Offsets are 32-bit offsets
  // from the uniform base pointers (M*K elements and the part's weight bytes
  // are below 2^31, checked on the host).  Rows past M or the part's rows read
  // nothing (zeros).
  const int a_row0 = tid >> 3, a_kc = tid & 7;
  bool a_ok[RA];
  uint32_t a_off[RA];
#pragma unroll
  for (int i = 0; i < RA; ++i) {
    const int r = m0 + a_row0 + i * (T / 8);
    a_ok[i] = r < p.m;
    a_off[i] = (uint32_t)(a_ok[i] ? r : 0) * (uint32_t)p.k + (uint32_t)(a_kc * 8);
  }
  int b_n[IB], b_kc[IB];
  bool b_ok[IB];
  uint32_t b_row[IB];
  const bool b_mine = NB >= T || tid < NB;  // threads past NB move no weight piece
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int it = b_mine ? tid + i * T : 0;
    b_n[i] = it >> 2;
    b_kc[i] = it & 3;
    b_ok[i] = b_mine && n0 + b_n[i] < n_rows;
    b_row[i] = (uint32_t)(b_ok[i] ? n0 + b_n[i] : 0) * (uint32_t)p.row_bytes;
  }
  const int s_row = n0 + (tid % BN) < n_rows ? n0 + (tid % BN) : n_rows - 1;

  struct Regs { u32x4 ah[RA], al[RA], b[IB]; uint32_t b4[IB]; };
  auto load = [&](int st, Regs& r) {
    const uint32_t k0 = (uint32_t)(st * kBK);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      r.ah[i] = a_ok[i] ? *(const u32x4*)(p.xh + (a_off[i] + k0)) : z;
      r.al[i] = a_ok[i] ? *(const u32x4*)(p.xl + (a_off[i] + k0)) : z;
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      r.b[i] = z;
      r.b4[i] = 0u;
      if (b_ok[i]) {
        if constexpr (F == FMT_AFF) {
          r.b[i] = *(const u32x4*)(pt.w + (b_row[i] + k0 + 16u * b_kc[i]));
        } else if constexpr (F == FMT_AFF4) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          const u32x2 v = *(const u32x2*)(pt.w + (b_row[i] + k0 / 2u + 8u * b_kc[i]));
          r.b[i].x = v.x;
          r.b[i].y = v.y;
        } else if constexpr (F == FMT_Q40) {
          // the stage's two blocks are 36 contiguous bytes at 36*st; block
          // b_kc/2 has its 16 nibble bytes at 2 (block 0) or 20 (block 1): read
          // the 20 bytes from 16*(b_kc/2) (4-byte aligned, inside the 36)
          const uint8_t* base = pt.w + (b_row[i] + 36u * st + 16u * (b_kc[i] >> 1));
          r.b[i] = *(const u32x4a4*)base;
          r.b4[i] = *(const uint32_t*)(base + 16);
        } else {
          // Q4_K: stage st is 64-column chunk (st & 3) of super-block st / 4;
          // its 32 nibble bytes sit at 16 + 32*(st & 3); b_kc & 1 picks the half
          r.b[i] = *(const u32x4*)(pt.w + (b_row[i] + 144u * (st >> 2) + 16u + 32u * (st & 3) + 16u * (b_kc[i] & 1)));
        }
      }
    }
  };
  // The 16 codes of a B piece as bytes in element order.
  auto code_words = [&](const u32x4& b, uint32_t b4, int kc, uint32_t (&cw)[4]) {
    if constexpr (F == FMT_AFF) {
      cw[0] = b.x; cw[1] = b.y; cw[2] = b.z; cw[3] = b.w;
    } else if constexpr (F == FMT_AFF4) {
      const uint32_t w2[2] = {b.x, b.y};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t ev = w2[i] & 0x0F0F0F0Fu, od = (w2[i] >> 4) & 0x0F0F0F0Fu;
        cw[2 * i] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
        cw[2 * i + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
      }
    } else {
      uint32_t nb[4];
      if constexpr (F == FMT_Q40) {
        const uint32_t d[5] = {b.x, b.y, b.z, b.w, b4};
#pragma unroll
        for (int i = 0; i < 4; ++i) nb[i] = (kc >> 1) ? d[i + 1] : __builtin_amdgcn_alignbyte(d[i + 1], d[i], 2);
      } else {
        nb[0] = b.x; nb[1] = b.y; nb[2] = b.z; nb[3] = b.w;
      }
      // Q4_0: low nibbles are elements 0..15 of the block, high ones 16..31,
      // as int8 bytes 16 (q - 8); Q4_K: low nibbles are the first sub-block of
      // the chunk, high the second
      if constexpr (F == FMT_Q40) {
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[i] = (kc & 1) ? q40_hi16(nb[i]) : q40_lo16(nb[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[i] = (kc >> 1) ? (nb[i] >> 4) & 0x0F0F0F0Fu : nb[i] & 0x0F0F0F0Fu;
      }
    }
  };
  auto store = [&](int st, const Regs& r, int buf) {
    __bf16* ah = sA[buf];
    __bf16* al = sA[buf] + A_ELEMS;
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      *(u32x4*)(ah + (a_row0 + i * (T / 8)) * kPitch + a_kc * 8) = r.ah[i];
      *(u32x4*)(al + (a_row0 + i * (T / 8)) * kPitch + a_kc * 8) = r.al[i];
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      if (!b_mine) break;
      // 16 codes -> 16 bf16 (exact: integers below 256, or the int8 Q4_0 codes)
      uint32_t cw[4];
      code_words(r.b[i], r.b4[i], b_kc[i], cw);
      bf16x8 lo, hi;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wlo = cw[e >> 2] >> (8 * (e & 3)), whi = cw[2 + (e >> 2)] >> (8 * (e & 3));
        if constexpr (F == FMT_Q40) {
          lo[e] = (__bf16)(float)(int8_t)wlo;
          hi[e] = (__bf16)(float)(int8_t)whi;
        } else {
          lo[e] = (__bf16)(float)(wlo & 0xFFu);
          hi[e] = (__bf16)(float)(whi & 0xFFu);
        }
      }
      *(bf16x8*)(sB[buf] + b_n[i] * kPitch + b_kc[i] * 16) = lo;
      *(bf16x8*)(sB[buf] + b_n[i] * kPitch + b_kc[i] * 16 + 8) = hi;
    }
    const int g0 = st * kBK / p.gs;
    if (tid < ng * BN) sS[buf][tid / BN][tid % BN] = group_scale<F>(pt, p.row_bytes, groups, s_row, g0 + tid / BN);
  };
  auto scale_into_acc = [&](int buf, int gi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sv = sS[buf][gi][wn * 64 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(sv, P[i][j][e], acc[i][j][e]);
    }
  };
  // this wave's 32-column half of stage st
  auto compute = [&](int st, int buf) {
    const __bf16* ah = sA[buf];
    const __bf16* al = sA[buf] + A_ELEMS;
    if (p.gs == 32) {  // the half is a whole group
      mfma_substep<true, TI>(ah, al, sB[buf], kh * 32, wm, wn, lane, P);
      scale_into_acc(buf, kh);
      return;
    }
    const int c0 = st * kBK;
    if (c0 % p.gs == 0) mfma_substep<true, TI>(ah, al, sB[buf], kh * 32, wm, wn, lane, P);
    else mfma_substep<false, TI>(ah, al, sB[buf], kh * 32, wm, wn, lane, P);
    if ((c0 + kBK) % p.gs == 0) scale_into_acc(buf, 0);
  };

  // stage sb holds steps BKS sb .. BKS sb + BKS - 1 in buffers BKS (sb & 1) + u
  Regs rg[BKS];
#pragma unroll
  for (int u = 0; u < BKS; ++u) load(u, rg[u]);
#pragma unroll
  for (int u = 0; u < BKS; ++u) store(u, rg[u], u);
  __syncthreads();
  const int nsb = stages / BKS;  // the host launches BKS = 2 for K % 128 == 0 only
  for (int sb = 0; sb < nsb; ++sb) {
    const int buf = (sb & 1) * BKS, nbuf = BKS - buf;
    if (sb + 1 < nsb) {
#pragma unroll
      for (int u = 0; u < BKS; ++u) load((sb + 1) * BKS + u, rg[u]);
    }
#pragma unroll
    for (int u = 0; u < BKS; ++u) compute(sb * BKS + u, buf + u);
    if (sb + 1 < nsb) {
#pragma unroll
      for (int u = 0; u < BKS; ++u) store((sb + 1) * BKS + u, rg[u], nbuf + u);
    }
    __syncthreads();
  }

  // ---- combine the two K halves: half 1 hands its partial sums to half 0
  float* red = reinterpret_cast<float*>(&sA[0][0]);  // NSUB sub-tiles x 64 x 64 floats
  float* mine = red + (size_t)sub * (SUBM * 64);
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) *(f32x4*)(mine + ((i * 4 + j) * 64 + lane) * 4) = acc[i][j];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 o = *(const f32x4*)(mine + ((i * 4 + j) * 64 + lane) * 4);
        acc[i][j] += o;
      }
  }
  __syncthreads();

  // ---- bias term: acc += X[m, g] * b[n, g] over all groups, as a K = groups
  // product on the matrix cores with X and b split into bf16 hi + lo (Q4_0
  // has none)
  constexpr int BR = BM > BN ? BM : BN;
  if constexpr (F != FMT_Q40) for (int g0 = 0; g0 < groups; g0 += 32) {
    __bf16* xh_s = sA[1];  // [BM m][32 g], pitch kPitch
    __bf16* xl_s = sA[1] + A_ELEMS;
    __bf16* bh_s = sB[0];  // [BN n][32 g]
    __bf16* bl_s = sB[1];
    for (int i = tid; i < BR * 32; i += T) {
      const int r = i >> 5, g = i & 31;
      const int gm = m0 + r, gn = n0 + r, gg = g0 + g;
      if (r < BM) {
        __bf16 xhv = (__bf16)0.0f, xlv = (__bf16)0.0f;
        if (gg < groups && gm < p.m) {
          xhv = p.sh[(size_t)gm * groups + gg];
          xlv = p.sl[(size_t)gm * groups + gg];
        }
        xh_s[r * kPitch + g] = xhv;
        xl_s[r * kPitch + g] = xlv;
      }
      if (r < BN) {
        __bf16 bhv = (__bf16)0.0f, blv = (__bf16)0.0f;
        if (gg < groups && gn < n_rows) {
          const float b = group_bias<F>(pt, p.row_bytes, groups, gn, gg);
          bhv = (__bf16)b;
          blv = (__bf16)(b - (float)bhv);
        }
        bh_s[r * kPitch + g] = bhv;
        bl_s[r * kPitch + g] = blv;
      }
    }
    __syncthreads();
    if (kh == 0) {
      const int r16 = lane & 15;
      const int kk = (lane >> 4) * 8;
      bf16x8 bh[4], bl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bh[j] = *(const bf16x8*)(bh_s + (wn * 64 + j * 16 + r16) * kPitch + kk);
        bl[j] = *(const bf16x8*)(bl_s + (wn * 64 + j * 16 + r16) * kPitch + kk);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const bf16x8 ah = *(const bf16x8*)(xh_s + (wm * SUBM + i * 16 + r16) * kPitch + kk);
        const bf16x8 al = *(const bf16x8*)(xl_s + (wm * SUBM + i * 16 + r16) * kPitch + kk);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // store: lane holds rows 4*(lane/16)+e, column lane%16 of each 16x16 tile
  if (kh == 0) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gm = m0 + wm * SUBM + i * 16 + (lane >> 4) * 4 + e;
          const int gn = n0 + wn * 64 + j * 16 + (lane & 15);
          if (gm < p.m && gn < n_rows) pt.y[(size_t)gm * pt.ldy + gn] = acc[i][j][e];
        }
  }
}

}  // namespace qg
