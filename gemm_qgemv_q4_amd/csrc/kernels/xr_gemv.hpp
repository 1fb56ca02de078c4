// Q4_0, Q4_K and affine-code products at 3..8 rows of x on the gfx950 matrix
// cores, with x held in registers for the whole launch.
//
// Q4_0: y[m, n] = sum_b d[n, b] P[m, n, b] with P over x (q - 8)
//                                               [GGML block_q4_0: w = d (q - 8)]
// Q4_K: y[m, n] = sum_j (d sc_j)[n] P[m, n, j] - (dmin m_j)[n] X[m, j]
//                                               [GGML block_q4_K: w = d sc_j q - dmin m_j]
// affine: y[m, n] = sum_b s[n, g(b)] P[m, n, b] + b[n, g(b)] X[m, b]
//                                               [MLX affine groups: w = s q + b]
// with P = sum over a 32-weight block (Q4_0, affine) or sub-block (Q4_K) of
// x q and X the sum of x over it.
//
// Each 32-weight block is one v_mfma_f32_16x16x32_bf16 whose 16 columns are
// 16 weight rows and whose 16 rows are x: rows 0..7 hold bf16(x) of the (up
// to) 8 rows of x, rows 8..15 hold bf16(x - bf16(x)).  Both halves of x thus
// ride in one MFMA, and the output's two partial sums are added at the end
// (x carries 16 significant bits, relative error <= 2^-17 per element; the
// codes are exact in bf16 -- Q4_0 as 16 (q - 8), -128..112, the others as
// 0..15 or 0..255 -- and the products exact in the f32 accumulator).  A Q4_0
// block of codes 8 therefore adds exactly 0.  The block sums of x that Q4_K
// and the affine formats need come from the same MFMA unit (x times a column
// of ones).
//
// Work split: a workgroup of K/512 waves owns 16 weight rows at a time; wave
// w owns columns 512 w .. 512 w + 511, i.e. NB = 16 blocks (288 bytes of each
// row for the block formats, 512 for u8 and 256 for packed codes).  The wave
// keeps its slice of x as 16 MFMA A operands (64 VGPRs) and the block sums
// (64 VGPRs) for the whole launch, so after the first load x costs no memory
// or LDS traffic; that first load reads x row by row and is moved to the MFMA
// lanes through LDS.  The MFMA wants, in lane l, 4 code bytes of
// weight row l % 16; loads that narrow touch 16 rows per instruction and
// stream poorly, so the wave reads its 16 rows with 16-byte loads along the
// rows (18 lanes per row for the block formats), writes them to its own LDS
// region and reads the MFMA operands from there.  The loads of the next row
// group leave before the arithmetic on the current one.  The wave partials of
// an output are added in a fixed order through LDS, one barrier per up to
// four row groups (XrSlots).
#pragma once
#include "common.hpp"
#include "gemv.hpp"

namespace qg {

constexpr int kXrNB = 16;        // 32-weight blocks per wave
constexpr int kXrMaxWaves = 8;   // K <= 4096
constexpr int kXrMaxM = 8;       // x rows per launch
// Row groups whose wave partials are added after one barrier: 4, or 1 for u8
// codes, whose larger row groups, loaded early by the waves that run ahead,
// delayed the x loads of the others (12288 x 4096 at M = 8: 16.9 -> 17.6 us).
template <int FMT> struct XrSlots { static constexpr int n = FMT == FMT_AFF ? 1 : 4; };

// Bytes of one weight row in a wave's 512-column slice, and the LDS stride of
// its copy: a stride of 2 mod 32 dwords puts the 16 rows of one MFMA operand
// read (one or two dwords per lane) in distinct banks for every 16 or 32
// lanes that the LDS serves together.
template <int FMT> struct XrRow;
template <> struct XrRow<FMT_Q40> { static constexpr int bytes = 288, lds = 392; };
template <> struct XrRow<FMT_Q4K> { static constexpr int bytes = 288, lds = 392; };
template <> struct XrRow<FMT_AFF> { static constexpr int bytes = 512, lds = 520; };
template <> struct XrRow<FMT_AFF4> { static constexpr int bytes = 256, lds = 264; };

// LDS of one wave: its copy of a row group (16 rows of XrRow::lds bytes), its partial sums of
// up to XrSlots::n row groups in each of two buffers, and for the affine
// formats the staged scales and biases of a row group.
template <int FMT> struct XrLds {
  static constexpr int rows = 16 * XrRow<FMT>::lds;
  static constexpr int red = 2 * XrSlots<FMT>::n * 16 * 16 * 4;
  static constexpr int sb = (FMT == FMT_AFF || FMT == FMT_AFF4) ? 2 * 16 * 8 * 4 : 0;
  static constexpr int wave = rows + red + sb;
  static_assert(rows % 16 == 0 && wave % 16 == 0, "wave regions stay 16-byte aligned");
  static_assert(kXrMaxWaves * wave <= 160 * 1024, "a workgroup's LDS exceeds the CU's");
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two bytes holding codes 0..15 (byte pair `hiword` of v) as two exact bf16:
// read as OCP e4m3 the bytes 0..15 are q / 512, scaled back by 2^9.
template <bool HIWORD>
__device__ __forceinline__ uint32_t codes2_bf16(uint32_t v) {
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 512.0f, HIWORD);
  return __builtin_bit_cast(uint32_t, c);
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf16x2 c = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, c);
}

// LDS operations of one wave complete in order; this only keeps the compiler
// from moving a wave's LDS accesses across each other.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t dpp_row_ror8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);  // row_ror:8
}

// WV: the most waves a launch of this instance has (8, or 4 for K <= 2048,
// whose workgroups then fit twice in a CU's LDS).  The LDS is static:
// the same layout as dynamic shared memory measured 0.3-0.5 us slower on
// u8 codes at 8 rows of x.
template <int FMT, bool MULTI, int WV>
__global__ void __launch_bounds__(64 * kXrMaxWaves) gemv_xr_kernel(const float* ax, const uint8_t* aw0, int ak,
                                                                  int am_rows, int an_groups, int an, int agroup0,
                                                                  int arow_bytes, GemvParams p) {
  // The leading scalar arguments repeat what the x loads and a single-part
  // launch's weight loads need from p (x, part 0's weights, K, the x rows of
  // the tile, the tile count, part 0's rows and first tile, the row stride):
  // the hardware preloads them into scalar registers before the wave starts,
  // so those loads leave without waiting for a kernel-argument load.
  constexpr bool K4 = FMT == FMT_Q4K;
  constexpr bool AF = FMT == FMT_AFF || FMT == FMT_AFF4;
  constexpr int SLICE = XrRow<FMT>::bytes;
  constexpr int kRowLds = XrRow<FMT>::lds;
  constexpr int NB = kXrNB;
  using LW = XrLds<FMT>;
  static_assert(WV == 4 || WV == kXrMaxWaves, "instances for 4 and 8 waves");
  __shared__ u32x4 xr_lds[WV * LW::wave / 16];
  uint8_t* const lds = reinterpret_cast<uint8_t*>(xr_lds);

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int waves = ak >> 9;  // the launch has K / 512 waves (no hidden-argument load)
  const int r = lane & 15;  // MFMA row of A (x row r & 7; bf16(x) for r < 8, the remainder for r >= 8) and column of B
  const int kp = lane >> 4;  // K piece: weights 4kp..4kp+3, 16+4kp..16+4kp+3 of a Q4_0 block, 8kp..8kp+7 of a Q4_K sub-block
  const bool lo_row = r >= 8;
  const int kb0 = wv * NB;  // first block of this wave

  // No range check on the first tile: the host never launches more
  // workgroups than tiles, and a tile past the last one would only load
  // clamped rows and store nothing.  Without it the x loads need one
  // scalar-memory round trip less.
  int t = blockIdx.x;

  // ---- x slice.  The MFMA layout wants, for every block, in lane r < 8 the
  // first four of its K piece's x values (row r & 7) and in lane r + 8 the
  // last four; the two then trade halves.  Loaded that way, the 8 lanes of
  // a quad pair sit on 8 rows of x, and the slice (16 KB per wave at 8 rows)
  // arrived 1-3 us after the launch.  So the loads read x row by row instead
  // (lane l: float4 l % 8 of row l / 8 of every block, one 128-byte line per
  // 8 lanes), and the wave moves the values to the MFMA lanes through its
  // LDS region, XB blocks at a time.
  const int mx = r & 7;
  const bool live = mx < am_rows;
  const int e0 = FMT == FMT_Q40 ? 4 * kp + (lo_row ? 16 : 0) : 8 * kp + (lo_row ? 4 : 0);
  // Up to 4 rows of x (x4): each load covers two blocks of 4 rows (lane l:
  // block l / 32 of the pair, row l / 8 % 4), 8 loads instead of 16.
  const bool x4 = am_rows <= 4;  // uniform
  const int xrow = x4 ? (lane >> 3) & 3 : lane >> 3;  // row of x this lane loads (rows past the tile load row 0, unused)
  const int xblk = x4 ? lane >> 5 : 0;                // block of the pair (x4)
  const float* xp = ax + (size_t)(xrow < am_rows ? xrow : 0) * ak + 32 * (kb0 + xblk) + 4 * (lane & 7);
  f32x4 xv[NB];
  if (x4) {
#pragma unroll
    for (int j = 0; j < NB / 2; ++j) xv[j] = *reinterpret_cast<const f32x4a4*>(xp + 64 * j);
  } else {
#pragma unroll
    for (int s = 0; s < NB; ++s) xv[s] = *reinterpret_cast<const f32x4a4*>(xp + 32 * s);
  }
  // the x loads leave before anything that waits for a kernel-argument load
  // (the part lookup of a multi-part launch)
  __builtin_amdgcn_sched_barrier(0);

  // ---- weight loads of one row group: 16 rows x SLICE bytes (288 for the
  // block formats) as pieces of 16 bytes (piece i: row i / (SLICE / 16), bytes
  // 16 (i % (SLICE / 16)) of the wave's slice); lane l loads pieces l + 64 j
  // (past the last piece: the last one again).  Rows are whole multiples of
  // SLICE bytes, so every piece is 16-byte aligned when the weights are.
  // what the loads of a tile need from its part
  auto part_of = [&](int tile) -> PartLoad {
    if constexpr (MULTI) return part_load(p, part_of_group(p, tile));
    return PartLoad{aw0, p.part0.scales, p.part0.biases, an, agroup0};
  };
  constexpr int PPR = SLICE / 16;  // pieces per row
  constexpr int PIECES = 16 * PPR;
  constexpr int LOADS = (PIECES + kWave - 1) / kWave;  // 5, 8 (u8 codes) or 4 (packed)
  // affine: the groups of the wave's 512-column slice, from g0 (8 groups or
  // fewer; past the wave's last group a lane loads the last one again)
  const int gsh = AF ? __builtin_ctz((unsigned)p.gs) : 0;
  const int wgroups = AF ? (p.gs >= 512 ? 1 : 512 >> gsh) : 0;
  const int g0 = AF ? (512 * wv) >> gsh : 0;
  u32x4 ga[LOADS];  // the next row group in flight
  float gsb[AF ? 4 : 1];  // affine: its scales or biases
  auto fetch = [&](u32x4 (&gq)[LOADS], int tile) {
    const PartLoad pt = part_of(tile);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int i = lane + kWave * j < PIECES ? lane + kWave * j : PIECES - 1;
      const int rr = (tile - pt.group0) * 16 + i / PPR;
      const int row = rr < pt.n ? rr : pt.n - 1;  // clamped for the loads; not stored
      gq[j] = *reinterpret_cast<const u32x4*>(pt.w + (size_t)row * (size_t)arow_bytes + SLICE * wv + 16 * (i % PPR));
    }
    if constexpr (AF) {
      // load e: rows 4e .. 4e + 3, lane l takes group l % 8 of array (l / 8) % 2
      // (scales, biases) of row 4e + l / 16, so that each load touches 8 row
      // segments of 32 bytes (with lanes 0..31 on the scales of 16 rows and
      // 32..63 on the biases, every load touched 32)
      const float* base = (((lane >> 3) & 1) ? pt.biases : pt.scales) + g0;
      const int g = (lane & 7) < wgroups ? lane & 7 : wgroups - 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = (tile - pt.group0) * 16 + 4 * e + (lane >> 4);
        const int row = rr < pt.n ? rr : pt.n - 1;
        gsb[e] = base[(size_t)row * (size_t)(ak >> gsh) + g];
      }
    }
  };
  // The wave's LDS copy: row n at byte kRowLds n (stride chosen in XrRow).
  uint8_t* wl = lds + wv * LW::wave;
  // the wave's partial sums: [buffer][slot][MFMA row][column]
  auto red_of = [&](int w, int buf, int slot) -> float* {
    return reinterpret_cast<float*>(lds + w * LW::wave + LW::rows) + (buf * XrSlots<FMT>::n + slot) * 256;
  };
  // affine: scale and bias of 16 rows x 8 groups, [2][16][8]
  float* const sbw = reinterpret_cast<float*>(wl + LW::rows + LW::red);
  auto stage = [&](const u32x4 (&gq)[LOADS]) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      // lanes past piece 287 loaded piece 287 again and write the same bytes there
      const int i = lane + kWave * j < PIECES ? lane + kWave * j : PIECES - 1;
      // rows start 8-byte aligned (the stride is not a multiple of 16): two 8-byte writes
      uint2* d = reinterpret_cast<uint2*>(wl + kRowLds * (i / PPR) + 16 * (i % PPR));
      d[0] = uint2{gq[j][0], gq[j][1]};
      d[1] = uint2{gq[j][2], gq[j][3]};
    }
    if constexpr (AF) {
      float* d = sbw + ((lane >> 3) & 1) * 128 + (lane >> 4) * 8 + (lane & 7);  // [array][row][group]
#pragma unroll
      for (int e = 0; e < 4; ++e) d[32 * e] = gsb[e];  // row 4e + lane / 16
    }
    wave_lds_sync();
  };
  // Row group t is loaded first; group t + G (G workgroups) leaves when group
  // t has been copied to LDS.  Past the last group the loads repeat a group of
  // this workgroup and are not used.  (Two groups in flight measured 4-8%
  // slower.)
  fetch(ga, t);
  // the weight loads leave before the x arithmetic below, behind the x loads only
  __builtin_amdgcn_sched_barrier(0);
  // the grid size (a hidden kernel argument) is read while the loads are in flight
  const int G = (int)gridDim.x;
  asm volatile("" ::"s"(G));

  // ---- A operands and block sums.  Row r < 8 takes bf16(x) of its K piece's
  // 8 weights, row r + 8 takes bf16(x - bf16(x)) of the same.  The block
  // formats take the weights in order; affine codes take them as
  // [0, 2, 4, 6, 1, 3, 5, 7], the order of the even and odd nibbles of a
  // packed word (u8 codes use the same order, so both give the same bits).
  constexpr bool XSUM = FMT != FMT_Q40;  // the format has an offset or bias term
  bf16x8 a[NB];
  f32x4 xs[XSUM ? NB : 1];  // X of this lane's MFMA rows 4kp .. 4kp+3
  {
    const bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                         (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    // XB blocks of the slice in the wave's LDS region as 8 rows of XROW
    // floats (132: the 8 rows of one read fall in distinct banks); the first
    // row group is staged there only after the last pass.
    constexpr int XB = 4;
    constexpr int XROW = 32 * XB + 4;
    static_assert(8 * XROW * 4 <= 16 * kRowLds, "x pass does not fit the wave's LDS region");
    float* xl = reinterpret_cast<float*>(wl);
    f32x4 xm[XB];
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      if (s % XB == 0) {
        if (x4) {  // rows 0..3 of the pass; rows 4..7 are not live
#pragma unroll
          for (int j = 0; j < XB / 2; ++j)
            *reinterpret_cast<f32x4*>(xl + xrow * XROW + 32 * (2 * j + xblk) + 4 * (lane & 7)) = xv[s / 2 + j];
        } else {
#pragma unroll
          for (int b = 0; b < XB; ++b)
            *reinterpret_cast<f32x4*>(xl + xrow * XROW + 32 * b + 4 * (lane & 7)) = xv[s + b];
        }
        wave_lds_sync();
#pragma unroll
        for (int b = 0; b < XB; ++b) xm[b] = *reinterpret_cast<const f32x4*>(xl + mx * XROW + 32 * b + e0);
        wave_lds_sync();
      }
      const f32x4 v = live ? xm[s % XB] : z;
      // pairs of this lane's four values: (0, 1), (2, 3), or (0, 2), (1, 3) for affine codes
      const float u0 = v.x, u1 = AF ? v.z : v.y, u2 = AF ? v.y : v.z, u3 = v.w;
      const uint32_t h01 = pk_bf16(u0, u1), h23 = pk_bf16(u2, u3);
      const float f0 = __builtin_bit_cast(float, h01 << 16), f1 = __builtin_bit_cast(float, h01 & 0xFFFF0000u);
      const float f2 = __builtin_bit_cast(float, h23 << 16), f3 = __builtin_bit_cast(float, h23 & 0xFFFF0000u);
      const uint32_t l01 = pk_bf16(u0 - f0, u1 - f1), l23 = pk_bf16(u2 - f2, u3 - f3);
      // lane r sends the remainders of its half to row r + 8, which sends its bf16(x) back
      const uint32_t r01 = dpp_row_ror8(lo_row ? h01 : l01);
      const uint32_t r23 = dpp_row_ror8(lo_row ? h23 : l23);
      u32x4 av;
      if constexpr (AF)  // [own, received] pairs interleaved: 0 2 | 4 6 | 1 3 | 5 7
        av = lo_row ? u32x4{r01, l01, r23, l23} : u32x4{h01, r01, h23, r23};
      else
        av = lo_row ? u32x4{r01, r23, l01, l23} : u32x4{h01, h23, r01, r23};
      a[s] = __builtin_bit_cast(bf16x8, av);
      if constexpr (XSUM) xs[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], ones, z, 0, 0, 0);
    }
  }

  // One row group from buffer gq: copy it to LDS, send the loads of the next
  // group into gq, multiply, add the wave partials.
  int it = 0;    // partial-sum buffer (alternates after every barrier)
  int slot = 0;  // row groups in it so far
  auto tile = [&](u32x4 (&gq)[LOADS]) {
    stage(gq);
    const int t2 = t + G;
    fetch(gq, t2 < an_groups ? t2 : t);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint8_t* rl = wl + kRowLds * r;
    auto mfma = [&](int s, uint32_t c0, uint32_t c1) -> f32x4 {
      const u32x4 bv = {codes2_bf16<false>(c0), codes2_bf16<true>(c0), codes2_bf16<false>(c1), codes2_bf16<true>(c1)};
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], __builtin_bit_cast(bf16x8, bv), z, 0, 0, 0);
    };
    if constexpr (FMT == FMT_Q40) {
      // Block s of row r sits at byte 18 s of the row's copy.  Even blocks start
      // 4-byte aligned: code bytes 4kp.. at 2 + 4kp, read as two dwords; odd
      // blocks have them in one dword.  The scale is the low (even) or high
      // (odd) half of the dword holding the block start.  The codes enter the
      // MFMA as the exact bf16 values 16 (q - 8) (int8 bytes, q40_lo16 /
      // q40_hi16), and d / 16 scales the block's product.
      // All of the lane's code and scale words of the group are read before
      // the first MFMA (40 registers): read block by block, each MFMA waited
      // for its own LDS round trip.  The scheduling barrier also keeps the
      // next group's loads ahead of the MFMAs.
      uint32_t qw[NB], qe[NB / 2], dw[NB];
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        const uint8_t* blk = rl + 18 * s;
        if (s % 2 == 0) {
          qw[s] = *reinterpret_cast<const uint32_t*>(blk + 4 * kp);
          qe[s / 2] = *reinterpret_cast<const uint32_t*>(blk + 4 * kp + 4);
          dw[s] = *reinterpret_cast<const uint32_t*>(blk);
        } else {
          qw[s] = *reinterpret_cast<const uint32_t*>(blk + 2 + 4 * kp);
          dw[s] = *reinterpret_cast<const uint32_t*>(blk - 2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      auto product = [&](int s, uint32_t& db) -> f32x4 {
        uint32_t v;
        if (s % 2 == 0) {
          v = __builtin_amdgcn_alignbyte(qe[s / 2], qw[s], 2);
          db = dw[s];
        } else {
          v = qw[s];
          db = dw[s] >> 16;
        }
        float c[8];
        signed_codes_f32(q40_lo16(v), c[0], c[1], c[2], c[3]);  // elements 4kp .. 4kp+3
        signed_codes_f32(q40_hi16(v), c[4], c[5], c[6], c[7]);  // elements 16+4kp ..
        const u32x4 bv = {pk_bf16(c[0], c[1]), pk_bf16(c[2], c[3]), pk_bf16(c[4], c[5]), pk_bf16(c[6], c[7])};
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], __builtin_bit_cast(bf16x8, bv), z, 0, 0, 0);
      };
      // block s + 1 is multiplied before block s is scaled into acc
      uint32_t db0;
      f32x4 P0 = product(0, db0);
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        uint32_t db1 = 0;
        f32x4 P1 = P0;
        if (s + 1 < NB) P1 = product(s + 1, db1);
        const float d = f16_bits_to_f32(db0) * 0.0625f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(d, P0[i], acc[i]);
        P0 = P1;
        db0 = db1;
      }
    } else if constexpr (K4) {
      // Super-block b (two per wave) of row r sits at byte 144 b of the row's
      // copy: d, dmin, 12 scale bytes, then 4 runs of 32 code bytes.  Sub-block
      // j takes the low (j even) or high nibbles of run j / 2; K piece kp is
      // its bytes 8kp .. 8kp + 7.
      // both super-blocks' words are read before the first MFMA
      uint2 hw[NB / 8][2], qw[NB / 8][4];
#pragma unroll
      for (int b = 0; b < NB / 8; ++b) {
        const uint8_t* sb = rl + 144 * b;
        hw[b][0] = *reinterpret_cast<const uint2*>(sb);
        hw[b][1] = *reinterpret_cast<const uint2*>(sb + 8);
#pragma unroll
        for (int c = 0; c < 4; ++c) qw[b][c] = *reinterpret_cast<const uint2*>(sb + 16 + 32 * c + 8 * kp);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < NB / 8; ++b) {
        const u32x4 hd = {hw[b][0].x, hw[b][0].y, hw[b][1].x, hw[b][1].y};
        const float d = f16_bits_to_f32(hd[0]), dmin = f16_bits_to_f32(hd[0] >> 16);
        // 6-bit scales and mins of sub-blocks 0..3 and 4..7, one per byte
        const uint32_t sc03 = hd[1] & 0x3F3F3F3Fu, mn03 = hd[2] & 0x3F3F3F3Fu;
        const uint32_t sc47 = (hd[3] & 0x0F0F0F0Fu) | ((hd[1] >> 2) & 0x30303030u);
        const uint32_t mn47 = ((hd[3] >> 4) & 0x0F0F0F0Fu) | ((hd[2] >> 2) & 0x30303030u);
        auto product = [&](int j) -> f32x4 {
          const uint2 v = qw[b][j / 2];
          const int sh = 4 * (j % 2);
          return mfma(8 * b + j, (v.x >> sh) & 0x0F0F0F0Fu, (v.y >> sh) & 0x0F0F0F0Fu);
        };
        f32x4 P0 = product(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          f32x4 P1 = P0;
          if (j + 1 < 8) P1 = product(j + 1);
          const uint32_t scw = j < 4 ? sc03 : sc47, mnw = j < 4 ? mn03 : mn47;
          const float ds = d * (float)((scw >> (8 * (j % 4))) & 0xFFu);
          const float dm = -(dmin * (float)((mnw >> (8 * (j % 4))) & 0xFFu));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i] = __builtin_fmaf(ds, P0[i], acc[i]);
            acc[i] = __builtin_fmaf(dm, xs[8 * b + j][i], acc[i]);
          }
          P0 = P1;
        }
      }
    } else {
      // Affine codes: block s of row r is bytes 32 s (u8) or 16 s (packed) of
      // the row's copy; K piece kp is its bytes 8kp .. 8kp + 7 (u8) or word kp
      // (packed), taken in the order [0, 2, 4, 6, 1, 3, 5, 7].  The scale and
      // bias of its group come from the staged table.
      const float* sr = sbw + r * 8;
      const float* br = sbw + 128 + r * 8;
      auto product = [&](int s) -> f32x4 {
        if constexpr (FMT == FMT_AFF) {
          const uint2 v = *reinterpret_cast<const uint2*>(rl + 32 * s + 8 * kp);
          const u32x4 bv = {pk_bf16(ubyte_f32<0>(v.x), ubyte_f32<2>(v.x)), pk_bf16(ubyte_f32<0>(v.y), ubyte_f32<2>(v.y)),
                            pk_bf16(ubyte_f32<1>(v.x), ubyte_f32<3>(v.x)), pk_bf16(ubyte_f32<1>(v.y), ubyte_f32<3>(v.y))};
          const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
          return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], __builtin_bit_cast(bf16x8, bv), z, 0, 0, 0);
        } else {
          const uint32_t v = *reinterpret_cast<const uint32_t*>(rl + 16 * s + 4 * kp);
          return mfma(s, v & 0x0F0F0F0Fu, (v >> 4) & 0x0F0F0F0Fu);
        }
      };
      f32x4 P0 = product(0);
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        f32x4 P1 = P0;
        if (s + 1 < NB) P1 = product(s + 1);
        const int gi = (32 * s) >> gsh;  // group of block s among the wave's groups
        const float sc = sr[gi], bi = br[gi];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] = __builtin_fmaf(sc, P0[i], acc[i]);
          acc[i] = __builtin_fmaf(bi, xs[s][i], acc[i]);
        }
        P0 = P1;
      }
    }
    // acc[i]: MFMA row 4 kp + i (x row (4kp+i) & 7, high or low part) for weight row r of the group
    float* rb = red_of(wv, it & 1, slot);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[(4 * kp + i) * 16 + r] = acc[i];
    ++slot;
    t += G;
    // The wave partials are added once per XrSlots::n row groups (or after
    // the last one), so a wave whose x arrived early works on ahead instead
    // of waiting at a barrier after every group.
    if (slot == XrSlots<FMT>::n || t >= an_groups) {
      __syncthreads();
      const int t0 = t - slot * G;  // first row group of these slots
      for (int e = threadIdx.x; e < slot * (kXrMaxM * 16); e += blockDim.x) {
        const int si = e >> 7;
        const int m = (e >> 4) & 7;
        const int n = e & 15;
        const int tt = t0 + si * G;
        // every wave's partial read first (slots past the last wave read the
        // last wave's and are not used), then added in wave order: a loop up
        // to `waves` waited for each read before the next one left
        float pw[WV];
#pragma unroll
        for (int w = 0; w < WV; ++w) {
          const float* rw = red_of(w < waves ? w : waves - 1, it & 1, si);
          pw[w] = rw[m * 16 + n] + rw[(m + 8) * 16 + n];
        }
        float sum = pw[0];
#pragma unroll
        for (int w = 1; w < WV; ++w) sum = w < waves ? sum + pw[w] : sum;
        PartStore pt;
        if constexpr (MULTI) {
          pt = part_store(p, part_of_group(p, tt));
        } else {
          pt = PartStore{p.part0.y[0], p.part0.ldy, an, agroup0};
        }
        const int rr = (tt - pt.group0) * 16 + n;
        if (m < am_rows && rr < pt.n) pt.y[(size_t)m * pt.ldy + rr] = sum;
      }
      // this buffer is written again after the next barrier
      ++it;
      slot = 0;
    }
  };
  tile(ga);
  while (t < an_groups) tile(ga);
}

}  // namespace qg
