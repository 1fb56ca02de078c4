// Small-M products (2..8 rows of x) of the affine formats on the gfx950
// matrix cores, streamed like the GEMV.
//
// y[m, n] = sum_pairs ( s[n, g] * P[m, n, pr] + b[n, g] * X[m, pr] ),
//   P[m, n, pr] = sum_{k in pr} x[m, k] q[n, k],  X[m, pr] = sum_{k in pr} x[m, k]
// over 64-column pairs of blocks pr, each inside one group g (group sizes of
// 64 and more) [mlx-native qmm_affine.rs: the affine map s*q + b per group].
//
// At M <= 8 the FMA path spends about M FMAs and one LDS read per weight and
// row of x; here the per-weight work is the code conversion, and the
// products run on v_mfma_f32_16x16x32_bf16 with the x rows as the MFMA rows
// and 16 weight rows as its columns.  x is split into x_hi = bf16(x) and
// x_lo = bf16(x - x_hi) as in the prefill path (relative error <= 2^-17 per
// element, codes exact in bf16, products exact in the f32 accumulator); the
// column sums X stay in f32.
//
// Operand layout.  The MFMA takes, in lane l, 8 consecutive "K" values of A
// row l % 16 and of B column l % 16, K piece l / 16.  The K order inside one
// group does not matter, so a lane loads 16 consecutive codes of its weight
// row (64 bytes per row and instruction for u8 codes) and feeds their first
// eight to one MFMA and the other eight to a second; x is laid out in LDS in
// the same order.  MFMA rows 8..15 repeat rows 0..7 and are not stored.
//
// Work: a workgroup of 8 waves owns a group of 16 weight rows; wave w owns
// the w-th eighth of K (NP pairs of 32-column blocks).  Each wave splits its
// slice of x into LDS once, loads all NP pairs of its 16 rows before the
// first MFMA, and keeps an f32 accumulator per (m, n); the 8 partial sums of
// an output are added in a fixed order through LDS.  Workgroups walk row
// groups (x stays in LDS), issuing the next group's loads before the barrier.
#pragma once
#include "common.hpp"
#include "gemv.hpp"

namespace qg {

constexpr int kMmaMaxM = 8;  // x rows per launch

// LDS bytes of gemv_mma_kernel<NP>: per wave x_hi and x_lo [NP][2][4][8][8]
// bf16 and X [NP][8] f32; then the partial sums [8 waves][8][16] f32.
__host__ __device__ constexpr int mma_lds_bytes(int np) {
  return 8 * (np * 2 * 4 * kMmaMaxM * 8 * 2 * 2 + np * kMmaMaxM * 4) + 8 * kMmaMaxM * 16 * 4;
}

// Sixteen codes of one weight row as two MFMA operands of eight bf16 (the
// codes are exact in bf16; v_cvt_pk_bf16_f32 packs two per register).
__device__ __forceinline__ void codes_bf16(const u32x4& v, bf16x8& lo, bf16x8& hi) {  // u8 codes
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lo[4 * i + 0] = (__bf16)ubyte_f32<0>(v[i]);
    lo[4 * i + 1] = (__bf16)ubyte_f32<1>(v[i]);
    lo[4 * i + 2] = (__bf16)ubyte_f32<2>(v[i]);
    lo[4 * i + 3] = (__bf16)ubyte_f32<3>(v[i]);
    hi[4 * i + 0] = (__bf16)ubyte_f32<0>(v[2 + i]);
    hi[4 * i + 1] = (__bf16)ubyte_f32<1>(v[2 + i]);
    hi[4 * i + 2] = (__bf16)ubyte_f32<2>(v[2 + i]);
    hi[4 * i + 3] = (__bf16)ubyte_f32<3>(v[2 + i]);
  }
}
__device__ __forceinline__ void codes_bf16(const uint2& v, bf16x8& lo, bf16x8& hi) {  // 4-bit codes, element j of a word in bits 4j..4j+3
  float e[16];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t w = i == 0 ? v.x : v.y;
    small_codes_f32(w & 0x0F0F0F0Fu, e[8 * i + 0], e[8 * i + 2], e[8 * i + 4], e[8 * i + 6]);
    small_codes_f32((w >> 4) & 0x0F0F0F0Fu, e[8 * i + 1], e[8 * i + 3], e[8 * i + 5], e[8 * i + 7]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo[i] = (__bf16)e[i];
    hi[i] = (__bf16)e[8 + i];
  }
}

template <int FMT> struct MmaCodes;
template <> struct MmaCodes<FMT_AFF> { using T = u32x4; };
template <> struct MmaCodes<FMT_AFF4> { using T = uint2; };

template <int FMT, int NP, bool MULTI>
__global__ void __launch_bounds__(512) gemv_mma_kernel(GemvParams p) {
  static_assert(FMT == FMT_AFF || FMT == FMT_AFF4, "affine codes only");
  constexpr int WV = 8;
  constexpr int ROWS = 16;
  constexpr int MM = kMmaMaxM;
  constexpr int XW = NP * 2 * 4 * MM * 8;  // bf16 per wave and half (hi or lo)
  using Codes = typename MmaCodes<FMT>::T;

  extern __shared__ f32x4 smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int r16 = lane & 15;  // MFMA row of A (x row m) and column of B (weight row n)
  const int kp = lane >> 4;   // 16-column piece of a 64-column pair
  const int mrows = p.m_rows;
  const int k0 = wv * NP * 64;  // this wave's K slice
  __bf16* xh = reinterpret_cast<__bf16*>(smem) + wv * (2 * XW);  // [NP][2][4][MM][8]
  __bf16* xl = xh + XW;
  float* xb = reinterpret_cast<float*>(reinterpret_cast<__bf16*>(smem) + WV * 2 * XW) + wv * (NP * MM);  // [NP][MM]
  float* red = reinterpret_cast<float*>(reinterpret_cast<__bf16*>(smem) + WV * 2 * XW) + WV * NP * MM;  // [WV][MM][16]

  struct View {
    const uint8_t* w;   // codes of this lane's row at column k0 + 16 kp
    const float* sc;    // scale and bias of the group holding column k0
    const float* bi;
    int row;
  };
  const int groups = p.k / p.gs;
  const int gsh = __builtin_ctz((unsigned)p.gs) - 6;  // log2(gs / 64): pairs per group
  auto view_of = [&](int g, View& v) {
    PartLoad pt;
    if constexpr (MULTI) {
      pt = part_load(p, part_of_group(p, g));
    } else {
      const GemvPart& p0 = p.part0;
      pt = PartLoad{p0.w[0], p0.scales, p0.biases, p0.n, p0.group0};
    }
    const int rr = (g - pt.group0) * ROWS + r16;
    v.row = rr < pt.n ? rr : pt.n - 1;  // clamped for the loads; not stored
    const int kc = FMT == FMT_AFF ? k0 + 16 * kp : (k0 + 16 * kp) / 2;
    v.w = pt.w + (size_t)v.row * (size_t)p.row_bytes + kc;
    const size_t gi = (size_t)v.row * groups + (k0 >> (gsh + 6));
    v.sc = pt.scales + gi;
    v.bi = pt.biases + gi;
  };

  // 16 codes of every pair of the slice, and the scale and bias of its group.
  Codes cq[NP];
  float cs[NP], cb[NP];
  auto fetch_all = [&](const View& v) {
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      if constexpr (FMT == FMT_AFF) cq[pr] = *reinterpret_cast<const u32x4*>(v.w + 64 * pr);
      else cq[pr] = *reinterpret_cast<const uint2*>(v.w + 32 * pr);
      cs[pr] = v.sc[pr >> gsh];
      cb[pr] = v.bi[pr >> gsh];
    }
  };

  int g = blockIdx.x;
  if (g >= p.n_groups) return;
  if constexpr (MULTI) prefetch_part_table<true>(p);
  View cv;
  view_of(g, cv);

  // x slice of this wave: item f = lane + 64 i covers float4 q4 (0..15) of
  // pair pr of row m (f = (m * NP + pr) * 16 + q4): columns 16 (q4/4) + 4 (q4%4)
  // .. +3 of the pair go to piece kp = q4/4, MFMA half (q4%4)/2, slot 4 (q4%2).
  {
    // Every load is one dword-aligned float4 (any x alignment gives the same
    // values); rows past m_rows load row 0 and are zeroed, so the loads are
    // unconditional and the compiler counts them exactly.
    f32x4 xv[2 * NP];
#pragma unroll
    for (int i = 0; i < 2 * NP; ++i) {
      const int f = lane + kWave * i;
      const int m = f / (NP * 16);
      const int rem = f % (NP * 16);
      xv[i] = *reinterpret_cast<const f32x4a4*>(p.x + (size_t)(m < mrows ? m : 0) * p.k + k0 + 4 * rem);
    }
    fetch_all(cv);
#pragma unroll
    for (int i = 0; i < 2 * NP; ++i) {
      const int f = lane + kWave * i;
      const int m = f / (NP * 16);
      const int rem = f % (NP * 16);
      const int pr = rem / 16;
      const int q4 = rem % 16;
      if (m >= mrows) xv[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const int at = (((pr * 2 + (q4 % 4) / 2) * 4 + q4 / 4) * MM + m) * 8 + 4 * (q4 % 2);
      const float v4[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
      bf16x4 hv, lv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hv[e] = (__bf16)v4[e];
        lv[e] = (__bf16)(v4[e] - (float)hv[e]);
      }
      *reinterpret_cast<bf16x4*>(xh + at) = hv;
      *reinterpret_cast<bf16x4*>(xl + at) = lv;
      const float sm = group_sum(((xv[i].x + xv[i].y) + xv[i].z) + xv[i].w, 16);
      if (q4 == 0) xb[pr * MM + m] = sm;
    }
    // LDS operations of one wave complete in order; this only keeps the
    // compiler from moving the reads above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  const int am = r16 & (MM - 1);  // MFMA rows 8..15 repeat rows 0..7 (not stored)
  // One row group: the arithmetic on the loaded pairs, then the next group's
  // loads, then the sum over the waves and the store.
  auto group = [&]() {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      bf16x8 b0, b1;
      codes_bf16(cq[pr], b0, b1);
      const __bf16* a = xh + ((pr * 2 * 4 + kp) * MM + am) * 8;
      const __bf16* a2 = xl + ((pr * 2 * 4 + kp) * MM + am) * 8;
      const bf16x8 ah0 = *reinterpret_cast<const bf16x8*>(a);
      const bf16x8 ah1 = *reinterpret_cast<const bf16x8*>(a + 4 * MM * 8);
      const bf16x8 al0 = *reinterpret_cast<const bf16x8*>(a2);
      const bf16x8 al1 = *reinterpret_cast<const bf16x8*>(a2 + 4 * MM * 8);
      const f32x4 xs4 = *reinterpret_cast<const f32x4*>(xb + pr * MM + 4 * (kp & 1));
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah0, b0, z, 0, 0, 0);
      P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah1, b1, P, 0, 0, 0);
      P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al0, b0, P, 0, 0, 0);
      P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al1, b1, P, 0, 0, 0);
      // P[e] is the pair's product for x row 4 kp + e and weight row r16
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = __builtin_fmaf(cs[pr], P[e], acc[e]);
        acc[e] = __builtin_fmaf(cb[pr], xs4[e], acc[e]);
      }
    }
    if (kp < MM / 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(wv * MM + 4 * kp + e) * 16 + r16] = acc[e];
    }
    const int g_done = g;
    g += (int)gridDim.x;
    if (g < p.n_groups) {
      view_of(g, cv);
      fetch_all(cv);
    }
    __syncthreads();
    if (threadIdx.x < MM * 16) {
      const int m = threadIdx.x / 16;
      const int n = threadIdx.x % 16;
      const float* a = red + m * 16 + n;
      constexpr int WS = MM * 16;  // stride between waves
      const float t = ((a[0 * WS] + a[1 * WS]) + (a[2 * WS] + a[3 * WS])) +
                      ((a[4 * WS] + a[5 * WS]) + (a[6 * WS] + a[7 * WS]));
      PartStore pt;
      if constexpr (MULTI) {
        pt = part_store(p, part_of_group(p, g_done));
      } else {
        const GemvPart& p0 = p.part0;
        pt = PartStore{p0.y[0], p0.ldy, p0.n, p0.group0};
      }
      const int rr = (g_done - pt.group0) * ROWS + n;
      if (m < mrows && rr < pt.n) pt.y[(size_t)m * pt.ldy + rr] = t;
    }
    // the partial sums are read before the next group writes them
    __syncthreads();
  };
  group();
  while (g < p.n_groups) group();
}

}  // namespace qg
