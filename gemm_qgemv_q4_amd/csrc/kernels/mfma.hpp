// Prefill-M affine product on the gfx950 matrix cores.
//
// y[m, n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k]  +  sum_g b[n,g] * X_g[m]
// with X_g[m] = sum_{k in g} x[m,k]  (the affine value s*q + b of
// mlx-native qmm_affine.rs, regrouped per group g of group_size columns).
//
// Precision: the codes q (0..255) are exact in bf16.  x is split once into
// x_hi = bf16(x) and x_lo = bf16(x - x_hi), so x_hi + x_lo carries 16
// significant bits (relative error <= 2^-18); bf16 x bf16 products are exact
// in the f32 MFMA accumulator.  Each group's partial product P_g = (x_hi +
// x_lo) . q is accumulated by two v_mfma_f32_16x16x32_bf16 per 32 columns,
// then scaled in f32: acc += s * P_g and acc += b * X_g.  This keeps
// |y - y_exact| well inside 1e-5 * sum|x w| (a single bf16 or f16 operand
// does not).
//
// Kernels:
//   affine_prep_kernel : x [M,K] f32 -> x_hi, x_lo [M,K] bf16 and X [M, K/gs] f32.
//   affine_mfma_kernel : 128x128 output tile per 256-thread workgroup (2x2
//       waves of 64x64 = 4x4 MFMA tiles), K in stages of 64 staged through
//       LDS (rows padded to 144 bytes so the 16-byte operand reads of a wave
//       are bank-conflict free).  Workgroup ids are remapped so the tiles of
//       one weight column block land on the same XCD (shared L2).
#pragma once
#include "common.hpp"

namespace qg {

// ---------------------------------------------------------------------------
// x -> (x_hi, x_lo) bf16 and per-group sums.  One wave per (row, group); the
// lanes walk the group with stride 64 and the group sum is a fixed butterfly.
__global__ void __launch_bounds__(256) affine_prep_kernel(const float* __restrict__ x,
                                                          __bf16* __restrict__ xh,
                                                          __bf16* __restrict__ xl,
                                                          float* __restrict__ xsum,
                                                          int m_rows, int k, int gs) {
  const int groups = k / gs;
  const long long item = (long long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (item >= (long long)m_rows * groups) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int m = (int)(item / groups);
  const int g = (int)(item - (long long)m * groups);
  const size_t base = (size_t)m * k + (size_t)g * gs;
  float s = 0.0f;
  for (int i = lane; i < gs; i += kWave) {
    const float v = x[base + i];
    const __bf16 h = (__bf16)v;
    const __bf16 l = (__bf16)(v - (float)h);
    xh[base + i] = h;
    xl[base + i] = l;
    s += v;
  }
  s = wave_sum_xor(s, kWave);
  if (lane == 0) xsum[(size_t)m * groups + g] = s;
}

struct MfmaParams {
  const __bf16* xh;      // [M, K]
  const __bf16* xl;      // [M, K]
  const float* xsum;     // [M, K/gs]
  const uint8_t* q;      // [N, K]
  const float* scales;   // [N, K/gs]
  const float* biases;   // [N, K/gs]
  float* y;              // [M, N]
  int m, n, k, gs;
  int tiles_m, tiles_n;
};

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kPitch = kBK + 8;  // bf16 elements per LDS row (144 bytes)

template <bool FIRST>
__device__ __forceinline__ void mfma_substep(const __bf16* sAh, const __bf16* sAl, const __bf16* sB,
                                             int sub, int wm, int wn, int lane, f32x4 (&P)[4][4]) {
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 8 + sub * 32;
  bf16x8 bfrag[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bfrag[j] = *(const bf16x8*)(sB + (wn * 64 + j * 16 + r16) * kPitch + kq);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x8 ah = *(const bf16x8*)(sAh + (wm * 64 + i * 16 + r16) * kPitch + kq);
    const bf16x8 al = *(const bf16x8*)(sAl + (wm * 64 + i * 16 + r16) * kPitch + kq);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (FIRST) {
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        P[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bfrag[j], z, 0, 0, 0);
      } else {
        P[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bfrag[j], P[i][j], 0, 0, 0);
      }
      P[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bfrag[j], P[i][j], 0, 0, 0);
    }
  }
}

__global__ void __launch_bounds__(256) affine_mfma_kernel(MfmaParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 sAh[kBM * kPitch];
  __shared__ __attribute__((aligned(16))) __bf16 sAl[kBM * kPitch];
  __shared__ __attribute__((aligned(16))) __bf16 sB[kBN * kPitch];
  __shared__ float sS[2][kBN];
  __shared__ float sBi[2][kBN];
  __shared__ __attribute__((aligned(16))) float sX[2][kBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // Tile order: tiles of one column block (same weights) are consecutive, and
  // consecutive ids are spread over the 8 XCDs by the dispatcher, so give each
  // XCD a contiguous range of tiles when the count allows it.
  const int total = p.tiles_m * p.tiles_n;
  int tile = blockIdx.x;
  if ((total & 7) == 0) tile = (tile & 7) * (total >> 3) + (tile >> 3);
  const int tm = tile % p.tiles_m;
  const int tn = tile / p.tiles_m;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int groups = p.k / p.gs;

  f32x4 acc[4][4], P[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      P[i][j] = acc[i][j];
    }

  // global -> register staging of one K stage
  u32x4 ra_h[4], ra_l[4], rb[2];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = tid + it * 256;  // 1024 chunks of 8 bf16
      const int row = c >> 3, kc = c & 7;
      const int gm = m0 + row;
      u32x4 vh = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
      if (gm < p.m) {
        const size_t off = (size_t)gm * p.k + k0 + kc * 8;
        vh = *(const u32x4*)(p.xh + off);
        vl = *(const u32x4*)(p.xl + off);
      }
      ra_h[it] = vh;
      ra_l[it] = vl;
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + it * 256;  // 512 chunks of 16 codes
      const int n = c >> 2, kc = c & 3;
      const int gn = n0 + n;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gn < p.n) v = *(const u32x4*)(p.q + (size_t)gn * p.k + k0 + kc * 16);
      rb[it] = v;
    }
  };
  auto store_stage = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = tid + it * 256;
      const int row = c >> 3, kc = c & 7;
      *(u32x4*)(sAh + row * kPitch + kc * 8) = ra_h[it];
      *(u32x4*)(sAl + row * kPitch + kc * 8) = ra_l[it];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + it * 256;
      const int n = c >> 2, kc = c & 3;
      // 16 codes -> 16 bf16 (exact: integers below 256)
      bf16x8 lo, hi;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wlo = rb[it][e >> 2], whi = rb[it][2 + (e >> 2)];
        lo[e] = (__bf16)(float)((wlo >> (8 * (e & 3))) & 0xFFu);
        hi[e] = (__bf16)(float)((whi >> (8 * (e & 3))) & 0xFFu);
      }
      *(bf16x8*)(sB + n * kPitch + kc * 16) = lo;
      *(bf16x8*)(sB + n * kPitch + kc * 16 + 8) = hi;
    }
    // scales / biases / x sums of the group(s) this stage touches
    const int g0 = k0 / p.gs;
    const int ng = p.gs < kBK ? kBK / p.gs : 1;  // 2 when gs == 32
    for (int i = tid; i < ng * kBN; i += 256) {
      const int gi = i / kBN, n = i - gi * kBN;
      const int gn = n0 + n;
      float sv = 0.0f, bv = 0.0f;
      if (gn < p.n) {
        sv = p.scales[(size_t)gn * groups + g0 + gi];
        bv = p.biases[(size_t)gn * groups + g0 + gi];
      }
      sS[gi][n] = sv;
      sBi[gi][n] = bv;
    }
    for (int i = tid; i < ng * kBM; i += 256) {
      const int gi = i / kBM, r = i - gi * kBM;
      const int gm = m0 + r;
      sX[gi][r] = gm < p.m ? p.xsum[(size_t)gm * groups + g0 + gi] : 0.0f;
    }
  };
  auto epilogue = [&](int gi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 64 + j * 16 + (lane & 15);
      const float sv = sS[gi][col], bv = sBi[gi][col];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 xs4 = *(const f32x4*)(&sX[gi][wm * 64 + i * 16 + (lane >> 4) * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float a = acc[i][j][e];
          a = __builtin_fmaf(sv, P[i][j][e], a);
          a = __builtin_fmaf(bv, xs4[e], a);
          acc[i][j][e] = a;
        }
      }
    }
  };

  load_stage(0);
  for (int k0 = 0; k0 < p.k; k0 += kBK) {
    __syncthreads();
    store_stage(k0);
    __syncthreads();
    if (k0 + kBK < p.k) load_stage(k0 + kBK);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kk = k0 + sub * 32;  // first column of this 32-wide step
      const bool first = (kk % p.gs) == 0;
      if (first) mfma_substep<true>(sAh, sAl, sB, sub, wm, wn, lane, P);
      else mfma_substep<false>(sAh, sAl, sB, sub, wm, wn, lane, P);
      if (((kk + 32) % p.gs) == 0) epilogue(p.gs < kBK ? sub : 0);
    }
  }

  // store: lane holds rows 4*(lane/16)+e, column lane%16 of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gm = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        const int gn = n0 + wn * 64 + j * 16 + (lane & 15);
        if (gm < p.m && gn < p.n) p.y[(size_t)gm * p.n + gn] = acc[i][j][e];
      }
}

}  // namespace qg
