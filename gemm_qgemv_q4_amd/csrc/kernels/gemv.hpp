// Dequantize-fused GEMV / skinny GEMM kernels for gfx950 (CDNA4, wave64).
//
// y[m, n] = sum_k x[m, k] * w[n, k] for f32 x and 4-bit block-quantized w.
// Formats (byte layouts, see the headers in include/qgemv_q4.h):
//   Q4_0  : 18-byte blocks of 32 weights (fp16 d + 16 nibble bytes),
//           value (nibble - 8) * d            [mlx-native fused_dual_proj_q4_0.rs]
//   Q4_K  : 144-byte super-blocks of 256 weights (fp16 d, fp16 dmin, 12 bytes
//           of 6-bit sub-block scales/mins, 128 nibble bytes),
//           value d*sc*q - dmin*m              [ferrum-kernels q4_k_gemv_v2.rs]
//   affine: u8 codes, f32 scale and bias per group, value s*q + b
//                                              [mlx-native qmm_affine.rs]
//   affine b4: the same with the codes packed eight per u32 word (element
//           8*kp + j in bits 4j..4j+3 of word kp)   [same page, packed kernel]
//
// Work decomposition (chosen for wave64 and HBM streaming, not taken from the
// pages' Metal kernels):
//   * A row of weights is cut into "chunks" of CH weights (64 for Q4_0 = two
//     blocks = 36 contiguous bytes; 64 for Q4_K = one 32-byte nibble run of a
//     super-block plus its 16-byte header; 32 for affine = 32 u8 codes or 16
//     bytes of packed codes, inside one group since group sizes of 32 and up
//     take this kernel).  Consecutive lanes take consecutive chunks, so every
//     wave-wide load instruction covers contiguous memory of one row.
//   * L lanes serve one row; a wave serves P = 64/L rows side by side and R
//     such row sets one after the other; each lane keeps NW*R*MT f32
//     accumulators (NW = 1, or 2 for the dual projection).
//   * x (MT rows of the activation) is staged once per workgroup in LDS as
//     float4 columns [m][e4][chunk] (e4 = which 4 elements of the chunk), so
//     the lanes of a wave read consecutive 16-byte words (no bank conflicts)
//     and every x word read feeds R*NW rows.  The per-32 sums of x are staged
//     too, which lets the block offset (-dmin*m, or the affine bias b) and the
//     scale be applied once per 32 weights instead of once per weight: the
//     inner loop is one code conversion and one FMA per weight.  Q4_0 codes
//     are converted as the signed values q - 8 (times 16, taken out of d), so
//     its blocks need no offset term and a block of codes 8 adds exactly 0.
//   * The lanes of a row are summed with a fixed xor butterfly: no atomics,
//     and the arithmetic of one output does not depend on R, NW, MT, the
//     number of waves or which part a row belongs to, which makes the dual
//     kernel bitwise equal to two single calls, the multi-part product equal
//     to one call per part, and the packed affine format equal to the u8 one.
//   * A launch may have up to kLaunchParts parts: weight tensors of one
//     format that share x, each with its own rows and output slice.  Row
//     groups are numbered part after part, so the part of a workgroup's group
//     is uniform and its pointers live in scalar registers.
#pragma once
#include "common.hpp"

namespace qg {

// One weight tensor of a product and where its outputs go.
struct GemvPart {
  const uint8_t* w[2];    // weights of stream 0 and (dual only) stream 1
  float* y[2];            // output (m, r) of stream s at y[s][m * ldy + r]
  int n;                  // rows
  int group0;             // first row group of this part
  const float* scales;    // affine: [n, K/gs]
  const float* biases;    // affine: [n, K/gs]
  long long ldy;
};

// Parts of one GEMV launch (a call with more parts makes several launches;
// each part's arithmetic does not depend on its launch).
constexpr int kLaunchParts = 4;

// Part table of a multi-part launch, each array of the four parts' fields in
// one 64-byte line: what a group's weight loads need (first group, rows,
// weights), where its outputs go, and the affine scales and biases.  Unused
// slots have their first group past every group.
struct PartQuad {
  int group0[kLaunchParts];  // slot 0 (part 0) is always 0
  int n[kLaunchParts];
  const uint8_t* w[kLaunchParts];
};
struct PartQuadOut {
  float* y[kLaunchParts];    // output (m, r) of part i at y[i][m * ldy[i] + r]
  long long ldy[kLaunchParts];
};
struct PartQuadAff {
  const float* scales[kLaunchParts];
  const float* biases[kLaunchParts];
};

// Kernel arguments.  The wavefront reads them through the scalar cache in
// 64-byte lines, and every line beyond the first costs time before the first
// weight load can leave (about 0.2 us for one more line on a 4096 x 4096 Q4_K
// product).  So:
//   * line 0 holds what a one-part block-format GEMV needs at M = 1: x,
//     row_bytes, k, n_groups and part 0's weights, outputs, rows and first
//     group;
//   * line 1 the rest of part 0 (scales, biases, ldy) and the settings the
//     affine formats, tiles of several x rows and the chunked kernel read;
//   * a multi-part launch finds its parts in one more line, its outputs in
//     another and, for the affine formats, scales and biases in a third.
struct GemvParams {
  const float* x;         // [m_rows, K] of this m-tile
  long long row_bytes;    // bytes per weight row
  int k;
  int n_groups;           // row groups over all parts
  GemvPart part0;         // the only part of a single-part launch
  int kt;                 // K elements staged per LDS tile (multiple of L*CH, or == k)
  int m_rows;             // valid x rows in this tile (<= MT)
  int gs;                 // affine group size
  int parts;
  alignas(64) PartQuad hot;
  PartQuadOut out;
  PartQuadAff aff;
};
static_assert(offsetof(GemvParams, part0) + offsetof(GemvPart, scales) == 64,
              "x, row_bytes, k, n_groups and part 0's w, y, n, group0 share the first 64 bytes");
static_assert(offsetof(GemvParams, parts) + sizeof(int) <= 128, "part 0's rest and the settings fill line 1");
static_assert(sizeof(PartQuad) == 64 && sizeof(PartQuadOut) == 64 && sizeof(PartQuadAff) == 64 &&
                  offsetof(GemvParams, hot) % 64 == 0,
              "each array of the multi-part table fills one 64-byte line");

// Part of row group g in a multi-part launch: compared against the first
// groups of parts 1..3 (fixed offsets, one line; unused slots never match).
// A loop over the parts up to a count read from a later line took one
// scalar-memory round trip per part before the first weight load.
__device__ __forceinline__ int part_of_group(const GemvParams& p, int g) {
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kLaunchParts; ++i) pi = g >= p.hot.group0[i] ? i : pi;
  return __builtin_amdgcn_readfirstlane(pi);
}

// Entry pi of a part-table array, picked by selects among its values, which
// are loaded at fixed offsets (and kept in scalar registers across the row
// groups of a workgroup): an index computed from pi would be a scalar load
// that waits for the lookup, before every group's weight loads.  The empty
// asm hides each value's origin, so that the compiler cannot fold the selects
// back into such a load.
template <typename T>
__device__ __forceinline__ T pick_part(const T (&a)[kLaunchParts], int pi) {
  T v = a[0];
#pragma unroll
  for (int i = 1; i < kLaunchParts; ++i) {
    T e = a[i];
    asm("" : "+s"(e));
    v = pi == i ? e : v;
  }
  return v;
}
// The same for pointers, picked as integers and turned back into pointers to
// global memory: a pointer that went through the asm would lose its address
// space, and its loads and stores would become flat instructions, which
// count against both wait counters and make every wait a full one.
template <typename T>
__device__ __forceinline__ T* pick_part(T* const (&a)[kLaunchParts], int pi) {
  unsigned long long v = reinterpret_cast<unsigned long long>(a[0]);
#pragma unroll
  for (int i = 1; i < kLaunchParts; ++i) {
    unsigned long long e = reinterpret_cast<unsigned long long>(a[i]);
    asm("" : "+s"(e));
    v = pi == i ? e : v;
  }
  using G = __attribute__((address_space(1))) T*;
  return (T*)(G)v;
}

// What the weight loads of a group need from part pi of a multi-part launch
// (fields a format does not use are never loaded).
struct PartLoad {
  const uint8_t* w;
  const float* scales;
  const float* biases;
  int n;
  int group0;
};
__device__ __forceinline__ PartLoad part_load(const GemvParams& p, int pi) {
  return {pick_part(p.hot.w, pi), pick_part(p.aff.scales, pi), pick_part(p.aff.biases, pi),
          pick_part(p.hot.n, pi), pick_part(p.hot.group0, pi)};
}

// Loads line 0 of the arguments with the part table before the lookup: the
// compiler would otherwise issue them one after the other.
template <bool AFFINE>
__device__ __forceinline__ void prefetch_part_table(const GemvParams& p) {
  if constexpr (AFFINE) {
    asm volatile("" ::"s"(p.x), "s"(p.n_groups), "s"(p.hot.group0[1]), "s"(p.aff.scales[0]));
  } else {
    asm volatile("" ::"s"(p.x), "s"(p.n_groups), "s"(p.hot.group0[1]));
  }
}
// The same without line 0, for a kernel that has x and the group count in
// preloaded scalar arguments.
template <bool AFFINE>
__device__ __forceinline__ void prefetch_part_quads(const GemvParams& p) {
  if constexpr (AFFINE) {
    asm volatile("" ::"s"(p.hot.group0[1]), "s"(p.aff.scales[0]));
  } else {
    asm volatile("" ::"s"(p.hot.group0[1]));
  }
}

// Where the outputs of part pi go (a multi-part launch has one stream per part).
struct PartStore {
  float* y;
  long long ldy;
  int n;
  int group0;
};
__device__ __forceinline__ PartStore part_store(const GemvParams& p, int pi) {
  return {pick_part(p.out.y, pi), pick_part(p.out.ldy, pi), pick_part(p.hot.n, pi), pick_part(p.hot.group0, pi)};
}

// CH: weights per chunk; SUMS: the format needs the per-32 sums of x (a
// block offset or bias multiplies them).  Q4_0 decodes its codes as signed
// values (q - 8) and has no offset term.
template <int FMT> struct FmtTraits;
template <> struct FmtTraits<FMT_Q40> { static constexpr int CH = 64; static constexpr bool SUMS = false; };
template <> struct FmtTraits<FMT_Q4K> { static constexpr int CH = 64; static constexpr bool SUMS = true; };
template <> struct FmtTraits<FMT_AFF> { static constexpr int CH = 32; static constexpr bool SUMS = true; };
template <> struct FmtTraits<FMT_AFF4> { static constexpr int CH = 32; static constexpr bool SUMS = true; };

// Raw bytes of one chunk of one row.
struct ChunkQ40 { u32x4a4 a; u32x4a4 b; uint32_t c; };   // 36 bytes: blocks 2t, 2t+1
struct ChunkQ4K { u32x4 h; u32x4 qa; u32x4 qb; };         // header + 32 nibble bytes
struct ChunkAff { u32x4 qa, qb; float s; float b; };     // 32 codes + their group's s, b
struct ChunkAff4 { u32x4 q; float s; float b; };          // 32 packed codes + s, b

template <int FMT> struct ChunkOf;
template <> struct ChunkOf<FMT_Q40> { using T = ChunkQ40; };
template <> struct ChunkOf<FMT_Q4K> { using T = ChunkQ4K; };
template <> struct ChunkOf<FMT_AFF> { using T = ChunkAff; };
template <> struct ChunkOf<FMT_AFF4> { using T = ChunkAff4; };

// Chunk tg of row `row` of a weight tensor starting at w (affine: its scales
// and biases start at sc, bi).
template <int FMT>
__device__ __forceinline__ typename ChunkOf<FMT>::T load_chunk(long long row_bytes, int k, int gs, const uint8_t* w,
                                                               const float* sc, const float* bi, int row,
                                                               int tg, bool with_sb = true) {
  typename ChunkOf<FMT>::T c;
  const uint8_t* rw = w + (size_t)row * (size_t)row_bytes;
  if constexpr (FMT == FMT_Q40) {
    const uint8_t* base = rw + 36 * (size_t)tg;
    c.a = *(const u32x4a4*)(base);
    c.b = *(const u32x4a4*)(base + 16);
    c.c = *(const uint32_t*)(base + 32);
  } else if constexpr (FMT == FMT_Q4K) {
    const uint8_t* base = rw + 144 * (size_t)(tg >> 2);
    c.h = *(const u32x4*)(base);
    c.qa = *(const u32x4*)(base + 16 + 32 * (tg & 3));
    c.qb = *(const u32x4*)(base + 32 + 32 * (tg & 3));
  } else {
    if constexpr (FMT == FMT_AFF) {
      c.qa = *(const u32x4*)(rw + 32 * (size_t)tg);
      c.qb = *(const u32x4*)(rw + 32 * (size_t)tg + 16);
    } else {
      // non-temporal: each 16-byte piece is read once by one lane and the
      // pieces of a wave are contiguous; 12288 x 4096 gs 64 at M = 1 8.15 ->
      // 7.8 us.  (The Q4 formats and u8 codes read a line with two or three
      // instructions; non-temporal loads there measured 4.1 -> 5.0 us on the
      // Q4_K 4096 x 4096 product.)
      c.q = __builtin_nontemporal_load((const u32x4*)(rw + 16 * (size_t)tg));
    }
    c.s = 0.0f;
    c.b = 0.0f;
    if (with_sb) {  // else the caller loads them (load_chunk_sb)
      const int groups = k / gs;
      const size_t gi = (size_t)row * groups + (32 * tg) / gs;
      c.s = sc[gi];
      c.b = bi[gi];
    }
  }
  return c;
}

// The scale and bias of an affine chunk loaded without its codes.
template <typename C>
__device__ __forceinline__ void load_chunk_sb(C& c, int k, int gs, const float* sc, const float* bi, int row, int tg) {
  const int groups = k / gs;
  const size_t gi = (size_t)row * groups + (32 * tg) / gs;
  c.s = sc[gi];
  c.b = bi[gi];
}

// The eight u32 words of byte codes (element order, one code per byte) of an
// affine chunk.  Packed codes: each word holds eight elements as nibbles; the
// even elements are its low nibbles, the odd ones its high nibbles, and a
// byte permute interleaves them back into element order.
__device__ __forceinline__ void aff_words(const ChunkAff& c, uint32_t (&qd)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qd[i] = c.qa[i];
    qd[4 + i] = c.qb[i];
  }
}
__device__ __forceinline__ void aff_words(const ChunkAff4& c, uint32_t (&qd)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = c.q[i];
    const uint32_t ev = w & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6 of the word
    const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
    // v_perm_b32(od, ev, sel): byte selector 0..3 = ev bytes, 4..7 = od bytes
    qd[2 * i] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
    qd[2 * i + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
  }
}

// Four codes 0..15, one per byte, as floats.  Read as OCP fp8 (e4m3), the
// bytes 0..15 are q / 512 exactly (the subnormals and the first binade share
// one spacing), and the scaled pair conversion multiplies by 2^9: two
// conversions give four exact codes.
__device__ __forceinline__ void small_codes_f32(uint32_t v, float& q0, float& q1, float& q2, float& q3) {
  const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 512.0f, false);
  const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 512.0f, true);
  q0 = lo[0];
  q1 = lo[1];
  q2 = hi[0];
  q3 = hi[1];
}

// Per-half (32-weight) scale factors of a chunk: y += A0*dot0 + B0*sumx0 + A1*dot1 + B1*sumx1
// (Q4_0: B = 0, not applied.)
struct HalfScales { float a0, b0, a1, b1; };

__device__ __forceinline__ HalfScales q40_scales(const ChunkQ40& c) {
  // block 2t: d in bytes 0..1; block 2t+1: d in bytes 18..19 (high half of dword 4);
  // the codes are read as 16 (q - 8)
  const float d0 = f16_bits_to_f32(c.a.x) * 0.0625f;
  const float d1 = f16_bits_to_f32(c.b.x >> 16) * 0.0625f;
  return {d0, 0.0f, d1, 0.0f};
}

// Sub-blocks 2c and 2c+1 of a Q4_K super-block.  The 12 scale bytes S0 (bytes
// 0..3), S1 (4..7), S2 (8..11) hold, for sub-block j < 4, scale = S0 byte j & 63
// and min = S1 byte j & 63; for j = 4 + i, scale = (S2 byte i & 15) | (S0 byte i
// >> 6) << 4 and min = (S2 byte i >> 4) | (S1 byte i >> 6) << 4.  Sub-blocks 2c,
// 2c+1 are adjacent bytes, so both are decoded with 16-bit wide masks.
__device__ __forceinline__ HalfScales q4k_scales(const ChunkQ4K& c, int cc) {
  const uint32_t sh = (uint32_t)(cc & 1) * 16u;
  const uint32_t a0 = c.h.y >> sh, a1 = c.h.z >> sh, a2 = c.h.w >> sh;
  const uint32_t sc_lo = a0 & 0x3F3Fu, m_lo = a1 & 0x3F3Fu;
  const uint32_t sc_hi = (a2 & 0x0F0Fu) | ((a0 >> 2) & 0x3030u);
  const uint32_t m_hi = ((a2 >> 4) & 0x0F0Fu) | ((a1 >> 2) & 0x3030u);
  const uint32_t scp = cc < 2 ? sc_lo : sc_hi;
  const uint32_t mp = cc < 2 ? m_lo : m_hi;
  const float d = f16_bits_to_f32(c.h.x);
  const float dmin = f16_bits_to_f32(c.h.x >> 16);
  // d*sc and dmin*m are exact in f32 (11-bit by 6-bit significands)
  return {d * ubyte_f32<0>(scp), -(dmin * ubyte_f32<0>(mp)), d * ubyte_f32<1>(scp), -(dmin * ubyte_f32<1>(mp))};
}

// The 8 dwords of code bytes of half h (32 weights) of a 64-weight chunk, in
// element order: dword i holds elements 4i .. 4i+3 of the half.  Q4_0: int8
// bytes 16 (q - 8); Q4_K: nibble values 0..15.  Unpacking one half at a time
// keeps half the code registers live.
__device__ __forceinline__ void unpack_q40(const ChunkQ40& c, int h, uint32_t (&v)[8]) {
  const uint32_t d[9] = {c.a.x, c.a.y, c.a.z, c.a.w, c.b.x, c.b.y, c.b.z, c.b.w, c.c};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // block 2t: nibble bytes start at byte 2 -> realign across dwords 0..4;
    // block 2t+1: nibbles at bytes 20..35 = dwords 5..8
    const uint32_t q = h == 0 ? __builtin_amdgcn_alignbyte(d[i + 1], d[i], 2) : d[5 + i];
    v[i] = q40_lo16(q);      // elements 4i..4i+3 of the block (low nibbles)
    v[4 + i] = q40_hi16(q);  // elements 16+4i.. of the block (high nibbles)
  }
}

__device__ __forceinline__ void unpack_q4k(const ChunkQ4K& c, int h, uint32_t (&v)[8]) {
  const uint32_t q[8] = {c.qa.x, c.qa.y, c.qa.z, c.qa.w, c.qb.x, c.qb.y, c.qb.z, c.qb.w};
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = opaque(h == 0 ? q[i] & 0x0F0F0F0Fu            // sub-block 2c: low nibbles
                         : (q[i] >> 4) & 0x0F0F0F0Fu);   // sub-block 2c+1: high nibbles
}

// x of one chunk for a single x row and its two per-32 sums, read from LDS
// before any of them is used: all reads are in flight together instead of two
// at a time, so a wave waits for LDS once per chunk.  (Only the timing of the
// reads changes.)
template <int NE4, bool SUMS>
__device__ __forceinline__ void preload_x(const f32x4* xs, const float* xsum, int ctp, int t, f32x4 (&xall)[NE4],
                                          float (&sall)[2]) {
#pragma unroll
  for (int e4 = 0; e4 < NE4; ++e4) xall[e4] = xs[e4 * ctp + t];
  if constexpr (SUMS) {
    sall[0] = xsum[t * 2];
    sall[1] = NE4 > 8 ? xsum[t * 2 + 1] : 0.0f;  // 32-element chunks have one sum
  } else {
    sall[0] = sall[1] = 0.0f;
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Decode one chunk of every (stream, row) and accumulate it.
template <int FMT, int MT, int NW, int R>
__device__ __forceinline__ void compute_chunk(const typename ChunkOf<FMT>::T (&ch)[NW][R], const f32x4* xs,
                                              const float* xsum, int ctp, int ct_max, int t, int tg,
                                              float (&acc)[NW][R][MT]) {
  constexpr int CH = FmtTraits<FMT>::CH;
  constexpr int NE4 = CH / 4;
  if constexpr (FMT == FMT_AFF || FMT == FMT_AFF4) {
    // the chunk lies in one group: acc += s * sum(x q) + b * sum(x)
    uint32_t words[NW][R][8];
#pragma unroll
    for (int s = 0; s < NW; ++s)
#pragma unroll
      for (int r = 0; r < R; ++r) aff_words(ch[s][r], words[s][r]);
    float sub[NW][R][MT];
#pragma unroll
    for (int s = 0; s < NW; ++s)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) sub[s][r][m] = 0.0f;
    f32x4 xall[MT == 1 ? NE4 : 1];
    float sall[2];
    if constexpr (MT == 1) preload_x<NE4, true>(xs, xsum, ctp, t, xall, sall);
#pragma unroll
    for (int e4 = 0; e4 < NE4; ++e4) {
      f32x4 xv[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) xv[m] = MT == 1 ? xall[MT == 1 ? e4 : 0] : xs[(m * NE4 + e4) * ctp + t];
#pragma unroll
      for (int s = 0; s < NW; ++s)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t qd = opaque(words[s][r][e4]);
          float q0, q1, q2, q3;
          if constexpr (FMT == FMT_AFF4) {
            small_codes_f32(qd, q0, q1, q2, q3);
          } else {
            q0 = ubyte_f32<0>(qd), q1 = ubyte_f32<1>(qd);
            q2 = ubyte_f32<2>(qd), q3 = ubyte_f32<3>(qd);
          }
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            float a = sub[s][r][m];
            a = __builtin_fmaf(xv[m].x, q0, a);
            a = __builtin_fmaf(xv[m].y, q1, a);
            a = __builtin_fmaf(xv[m].z, q2, a);
            a = __builtin_fmaf(xv[m].w, q3, a);
            sub[s][r][m] = a;
          }
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float sx = MT == 1 ? sall[0] : xsum[(m * ct_max + t) * 2];
#pragma unroll
      for (int s = 0; s < NW; ++s)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float a = acc[s][r][m];
          a = __builtin_fmaf(ch[s][r].s, sub[s][r][m], a);
          a = __builtin_fmaf(ch[s][r].b, sx, a);
          acc[s][r][m] = a;
        }
    }
  } else {
    HalfScales hs[NW][R];
#pragma unroll
    for (int s = 0; s < NW; ++s)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (FMT == FMT_Q40) hs[s][r] = q40_scales(ch[s][r]);
        else hs[s][r] = q4k_scales(ch[s][r], tg & 3);
      }
    constexpr bool SUMS = FmtTraits<FMT>::SUMS;
    f32x4 xall[MT == 1 ? NE4 : 1];
    float sall[2];
    if constexpr (MT == 1) preload_x<NE4, SUMS>(xs, xsum, ctp, t, xall, sall);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t nib[NW][R][8];
#pragma unroll
      for (int s = 0; s < NW; ++s)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if constexpr (FMT == FMT_Q40) unpack_q40(ch[s][r], h, nib[s][r]);
          else unpack_q4k(ch[s][r], h, nib[s][r]);
        }
      float sub[NW][R][MT];
#pragma unroll
      for (int s = 0; s < NW; ++s)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int m = 0; m < MT; ++m) sub[s][r][m] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int e4 = h * 8 + e;
        f32x4 xv[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) xv[m] = MT == 1 ? xall[MT == 1 ? e4 : 0] : xs[(m * NE4 + e4) * ctp + t];
#pragma unroll
        for (int s = 0; s < NW; ++s)
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float q0, q1, q2, q3;
            if constexpr (FMT == FMT_Q40) signed_codes_f32(nib[s][r][e], q0, q1, q2, q3);
            else small_codes_f32(nib[s][r][e], q0, q1, q2, q3);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              float a = sub[s][r][m];
              a = __builtin_fmaf(xv[m].x, q0, a);
              a = __builtin_fmaf(xv[m].y, q1, a);
              a = __builtin_fmaf(xv[m].z, q2, a);
              a = __builtin_fmaf(xv[m].w, q3, a);
              sub[s][r][m] = a;
            }
          }
      }
      // fold this 32-weight half: acc += A*dot + B*sum(x)  (Q4_0: acc += A*dot)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float sx = 0.0f;
        if constexpr (SUMS) sx = MT == 1 ? sall[h] : xsum[(m * ct_max + t) * 2 + h];
#pragma unroll
        for (int s = 0; s < NW; ++s)
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float A = h == 0 ? hs[s][r].a0 : hs[s][r].a1;
            const float B = h == 0 ? hs[s][r].b0 : hs[s][r].b1;
            float a = acc[s][r][m];
            a = __builtin_fmaf(A, sub[s][r][m], a);
            if constexpr (SUMS) a = __builtin_fmaf(B, sx, a);
            acc[s][r][m] = a;
          }
      }
    }
  }
}

// Workgroup = WV waves.  A "group" is WV*P*R consecutive rows (wave w takes
// P*R of them).  When x fits in LDS (kt == K) a workgroup stages it once and
// then walks groups blockIdx.x, blockIdx.x + gridDim.x, ... ("persistent");
// otherwise it owns one group and stages x tile by tile.  The lane's weight
// loads run one step ahead of its arithmetic across chunk, tile and group
// boundaries.
template <int FMT, int MT, int NW, int L, int R, bool MULTI>
__global__ void __launch_bounds__(512) gemv_kernel(GemvParams p) {
  constexpr int CH = FmtTraits<FMT>::CH;
  constexpr int NE4 = CH / 4;
  constexpr int P = kWave / L;
  constexpr bool SUMS = FmtTraits<FMT>::SUMS;
  constexpr int SB = 16 / MT > 4 ? 4 : 16 / MT;  // float4s of x per row and thread per staging batch
  constexpr int XPRE = 4;   // float4 registers for x loaded ahead of the first weights
  using Chunk = typename ChunkOf<FMT>::T;

  extern __shared__ f32x4 smem[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int lc = lane % L;
  const int rp = lane / L;
  const int rows_per_group = (int)(blockDim.x / kWave) * P * R;  // = the host's row-group size
  const int n_groups = p.n_groups;
  const int n_chunks = p.k / CH;
  const int ct_max = p.kt / CH;
  const int ctp = ct_max + 1;  // LDS pitch in float4s (odd: spreads banks on the staging writes)
  f32x4* xs = smem;                                              // [MT][NE4][ctp]
  float* xsum = reinterpret_cast<float*>(smem + MT * NE4 * ctp);  // [MT][ct_max][2]
  const bool x_vec = (reinterpret_cast<uintptr_t>(p.x) & 15u) == 0;
  // Part of row group g (uniform across the workgroup), copied out of the
  // kernel arguments once per group, and this lane's rows in it, counted from
  // the part's first row.
  struct View {
    const uint8_t* w[NW];
    const float* sc;
    const float* bi;
    float* y[NW];
    long long ldy;
  };
  struct Span {
    int n, group0;
  };
  auto view_of = [&](const GemvPart& pt, View& v, Span& sp) {
#pragma unroll
    for (int s = 0; s < NW; ++s) {
      v.w[s] = pt.w[s];
      v.y[s] = pt.y[s];
    }
    v.sc = pt.scales;
    v.bi = pt.biases;
    v.ldy = pt.ldy;
    sp.n = pt.n;
    sp.group0 = pt.group0;
  };
  // A single-part launch (MULTI false) reads part 0 at fixed argument
  // offsets together with the other arguments; only multi-part launches look
  // the part of each group up.
  auto group_rows = [&](int g, View& v, int (&rows)[R], bool (&valid)[R]) {
    Span sp;
    if constexpr (MULTI) {
      const int pi = part_of_group(p, g);
      const PartLoad pl = part_load(p, pi);
      v.w[0] = pl.w;
      v.sc = pl.scales;
      v.bi = pl.biases;
      sp.n = pl.n;
      sp.group0 = pl.group0;
      const PartStore ps = part_store(p, pi);
      v.y[0] = ps.y;
      v.ldy = ps.ldy;
    } else {
      view_of(p.part0, v, sp);
    }
    const int n = sp.n;
    const int row0 = (g - sp.group0) * rows_per_group + wv * (P * R) + rp;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int rr = row0 + r * P;
      valid[r] = rr < n;
      rows[r] = valid[r] ? rr : n - 1;  // clamp: loads stay in bounds, the store is skipped
    }
  };
  auto fetch = [&](Chunk (&dst)[NW][R], const View& v, const int (&rows)[R], int tg) {
#pragma unroll
    for (int s = 0; s < NW; ++s)
#pragma unroll
      for (int r = 0; r < R; ++r) dst[s][r] = load_chunk<FMT>(p.row_bytes, p.k, p.gs, v.w[s], v.sc, v.bi, rows[r], tg);
  };

  // Stage x[:, k0:k0+ktile] as [m][e4][chunk] float4 columns plus the sums of
  // each 32-element half (8 consecutive float4s = 8 consecutive lanes).  Index
  // math is shifts only (CH is a power of two); loops are uniform so every lane
  // takes part in the shuffles.
  auto xload = [&](int m, int j, int k0, int n4) -> f32x4 {
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if ((MT == 1 || m < p.m_rows) && j < n4) {  // MT = 1: m_rows is 1
      const float* xrow = p.x + (size_t)m * p.k + k0;
      if (x_vec) v = *reinterpret_cast<const f32x4*>(xrow + 4 * j);
      else v = f32x4{xrow[4 * j], xrow[4 * j + 1], xrow[4 * j + 2], xrow[4 * j + 3]};
    }
    return v;
  };
  auto xstore = [&](int m, int j, int n4, const f32x4& v) {
    const int t = j / NE4;   // chunk (NE4 is a power of two)
    const int e4 = j % NE4;  // float4 within the chunk
    if (j < n4) xs[(m * NE4 + e4) * ctp + t] = v;
    if constexpr (SUMS) {
      const float sm = group_sum(((v.x + v.y) + v.z) + v.w, 8);
      if (j < n4 && (e4 & 7) == 0) xsum[(m * ct_max + t) * 2 + (e4 >> 3)] = sm;
    }
  };
  // The loads of a batch cover every x row before any of them is written, so
  // staging MT rows costs one memory round trip per batch, not one per row.
  auto stage = [&](int k0, int ktile) {
    const int n4 = ktile >> 2;
    const int step = SB * (int)blockDim.x;
    for (int j0 = 0; j0 < n4; j0 += step) {
      f32x4 v[MT][SB];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int u = 0; u < SB; ++u) v[m][u] = xload(m, j0 + u * (int)blockDim.x + tid, k0, n4);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int u = 0; u < SB; ++u) xstore(m, j0 + u * (int)blockDim.x + tid, n4, v[m][u]);
    }
    __syncthreads();
  };
  // First staging of a single x row whose share per thread fits in XPRE
  // registers: the x loads are issued before the first weight loads, so
  // writing x to LDS waits only for x (loads retire in order) and the weights
  // stay in flight.  (For MT > 1 the extra registers cost more than it saves.)
  constexpr int XU = XPRE / MT > 0 ? XPRE / MT : 1;
  auto stage_x_first = [&](int ktile, Chunk (&dst)[NW][R], const View& pv, const int (&rws)[R], int tg) {
    const int n4 = ktile >> 2;
    f32x4 v[MT][XU];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int u = 0; u < XU; ++u) v[m][u] = xload(m, u * (int)blockDim.x + tid, 0, n4);
    fetch(dst, pv, rws, tg);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int u = 0; u < XU; ++u)
        if (u * (int)blockDim.x < n4) xstore(m, u * (int)blockDim.x + tid, n4, v[m][u]);
    __syncthreads();
  };

  const bool persistent = p.kt >= p.k;
  int g = blockIdx.x;
  if constexpr (MULTI) prefetch_part_table<FMT == FMT_AFF || FMT == FMT_AFF4>(p);
  View cv;
  int rows[R];
  bool rvalid[R];
  group_rows(g, cv, rows, rvalid);
  Chunk cur[NW][R];
  const int tg0 = lc < n_chunks ? lc : 0;
  bool staged = false;

  while (g < n_groups) {
    float acc[NW][R][MT];
#pragma unroll
    for (int s = 0; s < NW; ++s)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[s][r][m] = 0.0f;
    const int g_next = g + gridDim.x;
    View nv;
    int rows_next[R];
    bool valid_next[R];
    group_rows(g_next < n_groups ? g_next : g, nv, rows_next, valid_next);

    for (int k0 = 0; k0 < p.k; k0 += p.kt) {
      const int ktile = min(p.kt, p.k - k0);
      const int ct = ktile / CH;
      if (!persistent || !staged) {
        if (MT == 1 && !staged && k0 == 0 && (ktile >> 2) <= XU * (int)blockDim.x) {
          if constexpr (MT == 1) stage_x_first(ktile, cur, cv, rows, tg0);
        } else {
          if (staged) __syncthreads();     // the previous tile's readers are done
          else fetch(cur, cv, rows, tg0);  // first weights in flight while x is staged
          stage(k0, ktile);
        }
        staged = true;
      }
      for (int t = lc; t < ct; t += L) {
        const int tg = k0 / CH + t;
        Chunk nxt[NW][R];
        if (tg + L < n_chunks) fetch(nxt, cv, rows, tg + L);
        else if (g_next < n_groups) fetch(nxt, nv, rows_next, tg0);
        compute_chunk<FMT, MT, NW, R>(cur, xs, xsum, ctp, ct_max, t, tg, acc);
#pragma unroll
        for (int s = 0; s < NW; ++s)
#pragma unroll
          for (int r = 0; r < R; ++r) cur[s][r] = nxt[s][r];
      }
    }

    // ---- sum the L lanes of each row and store
#pragma unroll
    for (int s = 0; s < NW; ++s)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float v = group_sum(acc[s][r][m], L);
          if (lc == 0 && rvalid[r] && (MT == 1 || m < p.m_rows)) cv.y[s][(size_t)m * cv.ldy + rows[r]] = v;
        }
    g = g_next;
    cv = nv;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      rows[r] = rows_next[r];
      rvalid[r] = valid_next[r];
    }
    if (!persistent) break;
  }
}

// ---------------------------------------------------------------------------
// K-sliced GEMV for a tile of MT rows of x.  It computes the same additions
// in the same order as gemv_kernel with the same MT, L (lanes per row) and R
// (rows per lane), so both kernels give the same bits; what changes is which
// wave does which of them.
//   * The L lanes of a row in gemv_kernel become "virtual lanes" spread over
//     the WV waves of a workgroup (4, 8 or 16): wave w holds virtual lanes
//     LW*w .. LW*w+LW-1 (LW = L/WV) of 64/LW row sets of R rows each (hardware
//     lane = LW * set + c, virtual lane LW*w + c), so it needs x only at its
//     own chunks LW*w + c + L*j: one WV-th of K.
//   * Each wave stages that slice of x (for each of the MT rows) in its own
//     LDS region and then multiplies: no workgroup barrier stands between the
//     staging and the arithmetic, and all J chunks of a lane are loaded before
//     the first one is used.
//   * The butterfly over the L virtual lanes keeps its pairing: its first
//     log2(LW) levels run inside the wave (DPP), the upper log2(WV) levels
//     combine the waves' partial sums through LDS as (w0 + w1, w2 + w3, ...),
//     then pairs of pairs, and so on.
// A workgroup walks row groups of 64/LW*R rows; x stays in LDS between them.
// PAIR: the two weight streams of part 0 (a dual product, NW = 1) run as one
// stream of twice the row groups, the first half on w[0] / y[0] and the second
// on w[1] / y[1]; each group then holds one stream's rows, as in a single call.
// Scalar arguments of the K-sliced body (the leading, preloaded arguments of
// the two kernels at the end of this section):
//   single part (or MULTI without MPRE, which reads its part table from p):
//     aw0 = part 0's weights, aw1 = its second stream (dual or pair launch),
//     a3 = its first stream's output, an0 = its rows, an1 = the row stride,
//     an2 = the group count; ag1 and ag2 are unused;
//   MULTI && MPRE (up to three parts without scales or biases): aw0, aw1, a3
//     = the parts' weights, an0..an2 their rows, ag1 and ag2 the first
//     groups of parts 1 and 2 (a two-part launch passes a3 = aw1, an2 = 0
//     and ag2 = the group count); the row stride follows from K and the
//     format, the group count from the parts' rows.
// Part 0 starts at group 0.
template <typename T> __device__ __forceinline__ T sel(bool c, T a, T b) { return c ? a : b; }
template <int FMT> __device__ __forceinline__ int row_bytes_for(int k) {
  if constexpr (FMT == FMT_Q40) return k / 32 * 18;
  else if constexpr (FMT == FMT_Q4K) return k / 256 * 144;
  else if constexpr (FMT == FMT_AFF) return k;
  else return k / 2;
}

// The body of both K-sliced kernels below (gemv_ks_kernel and
// gemv_ks_mp_kernel), which differ only in their leading scalar arguments.
template <int FMT, int MT, int NW, int L, int R, int J, int WV, bool MULTI, bool PAIR, bool MPRE>
__device__ __forceinline__ void gemv_ks_body(const float* ax, const uint8_t* aw0, const uint8_t* aw1, const void* a3,
                                             int ak, int an0, int an1, int an2, int ag1, int ag2,
                                             const GemvParams& p) {
  const uint8_t* const aw2 = static_cast<const uint8_t*>(a3);
  static_assert(!MPRE || (MULTI && NW == 1 && FMT != FMT_AFF && FMT != FMT_AFF4),
                "parts from the arguments: one stream per part, no scales or biases");
  // the in-wave part of the butterfly below covers 4 or 8 virtual lanes
  static_assert((L == 32 || L == 64) && (WV == 4 || WV == 8 || WV == 16) && (L / WV == 4 || L / WV == 8),
                "4, 8 or 16 waves of 4 or 8 virtual lanes");
  static_assert(!PAIR || (NW == 1 && !MULTI), "a pair launch has one stream per group and one part");
  constexpr int CH = FmtTraits<FMT>::CH;
  constexpr int NE4 = CH / 4;
  constexpr int LW = L / WV;             // lanes of a row inside one wave
  constexpr int RS = kWave / LW;         // row sets per wave
  constexpr int ROWS = RS * R;           // rows per group
  constexpr int U = LW * J;              // chunks of x held by one wave
  constexpr int XP = U + 1;              // LDS pitch in float4s (odd: spreads banks on the staging writes)
  constexpr int XS = LW * NE4 / kWave;   // float4s of x per lane and chunk slice
  static_assert(XS >= 1 && XS * kWave == LW * NE4, "whole float4s of x per lane");
  constexpr bool SUMS = FmtTraits<FMT>::SUMS;
  constexpr int NSUM = SUMS ? MT * 2 * U : 0;  // per-32 sums of x per wave
  using Chunk = typename ChunkOf<FMT>::T;

  extern __shared__ f32x4 smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int rset = lane / LW;
  const int c = lane % LW;
  const int vl = LW * wv + c;
  const int n_chunks = ak / CH;
  f32x4* xs = smem + wv * (MT * NE4 * XP);                                         // [m][e4][u] of this wave
  float* xsum = reinterpret_cast<float*>(smem + WV * MT * NE4 * XP) + wv * NSUM;  // [m][u][2]
  float* red = reinterpret_cast<float*>(smem + WV * MT * NE4 * XP) + WV * NSUM;   // [2][NW][WV][ROWS][MT]

  // Weights and rows of group g for this lane (rows are clamped for the
  // loads; rows past the part's end are not stored).
  struct View {
    const uint8_t* w[NW];
    const float* sc;
    const float* bi;
    int row[R];
  };
  // groups of one stream of a pair launch
  const int pair_groups = PAIR ? (an0 + ROWS - 1) / ROWS : 0;
  const int arow_bytes = MULTI ? row_bytes_for<FMT>(ak) : an1;
  int an_groups;
  if constexpr (!MULTI) an_groups = an2;
  else if constexpr (MPRE) an_groups = ag2 + (an2 + ROWS - 1) / ROWS;
  else an_groups = p.n_groups;
  auto view_of = [&](int g, View& v) {
    int gl, n;
    if constexpr (MULTI && MPRE) {
      // selects of values: a conditional over the arguments themselves is a
      // select of their addresses, which puts the arguments in scratch memory
      const bool past0 = g >= ag1, past1 = g >= ag2;
      v.w[0] = sel(past1, aw2, sel(past0, aw1, aw0));
      n = sel(past1, an2, sel(past0, an1, an0));
      gl = g - sel(past1, ag2, sel(past0, ag1, 0));
      v.sc = nullptr;
      v.bi = nullptr;
    } else if constexpr (MULTI) {
      const PartLoad pl = part_load(p, part_of_group(p, g));
      v.w[0] = pl.w;
      v.sc = pl.scales;
      v.bi = pl.biases;
      n = pl.n;
      gl = g - pl.group0;
    } else {
      v.w[0] = aw0;
      if constexpr (NW == 2) v.w[1] = aw1;
      v.sc = p.part0.scales;
      v.bi = p.part0.biases;
      n = an0;
      gl = g;  // part 0 starts at group 0
      if constexpr (PAIR) {
        const bool second = gl >= pair_groups;
        v.w[0] = second ? aw1 : aw0;
        gl -= second ? pair_groups : 0;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int rr = gl * ROWS + rset + RS * r;
      v.row[r] = rr < n ? rr : n - 1;
    }
  };

  // Chunk tg = vl + L j of the lane's rows; past the last chunk the last one
  // is loaded again (same cache lines) and not used.
  Chunk ch[J][NW][R];
  constexpr bool AFF = FMT == FMT_AFF || FMT == FMT_AFF4;
  auto fetch_all = [&](const View& v) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int tg = vl + L * j;
      const int tl = tg < n_chunks ? tg : n_chunks - 1;
#pragma unroll
      for (int s = 0; s < NW; ++s)
#pragma unroll
        for (int r = 0; r < R; ++r)
          ch[j][s][r] = load_chunk<FMT>(arow_bytes, ak, p.gs, v.w[s], v.sc, v.bi, v.row[r], tl, !AFF);
    }
    if constexpr (AFF) {
      // The scales and biases after all codes: the vector memory counter
      // completes in order, so a chunk's codes would otherwise wait for the
      // scale loads issued before them.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int tg = vl + L * j;
        const int tl = tg < n_chunks ? tg : n_chunks - 1;
#pragma unroll
        for (int s = 0; s < NW; ++s)
#pragma unroll
          for (int r = 0; r < R; ++r) load_chunk_sb(ch[j][s][r], ak, p.gs, v.sc, v.bi, v.row[r], tl);
      }
    }
  };

  // No range check on the first group: the host never launches more
  // workgroups than groups, and a group past the last one would only load
  // clamped rows and store nothing.  Without the check the compiler issues the
  // group count, x and a multi-part launch's part table together instead of
  // one after the other.
  int g = blockIdx.x;
  if constexpr (MULTI && !MPRE) prefetch_part_quads<FMT == FMT_AFF || FMT == FMT_AFF4>(p);
  View cv;
  view_of(g, cv);
  int grid;
  float* ys[3] = {nullptr, nullptr, nullptr};  // outputs of parts 0..2 (single part: of its two streams)

  // x of this wave's chunks, for each of the MT rows of x: float4
  // NE4 * (LW*w + L*j) + lane covers chunks LW*w + L*j .. +LW-1.  The loads go
  // out before the first weights; rows past m_rows are zero.
  {
    const bool x_vec = (reinterpret_cast<uintptr_t>(ax) & 15u) == 0;
    const int n4 = ak >> 2;
    f32x4 xv[MT][J * XS];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < J * XS; ++j) {
        const int f = NE4 * (LW * wv + L * (j / XS)) + kWave * (j % XS) + lane;
        const float* xr = ax + (size_t)m * ak;
        xv[m][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if ((MT == 1 || m < p.m_rows) && f < n4) {
          if (x_vec) xv[m][j] = *reinterpret_cast<const f32x4*>(xr + 4 * f);
          else xv[m][j] = f32x4{xr[4 * f], xr[4 * f + 1], xr[4 * f + 2], xr[4 * f + 3]};
        }
      }
    fetch_all(cv);
    // The grid size lives in the hidden kernel arguments, a scalar-cache line
    // of its own: read it while the first loads are in flight instead of after
    // the arithmetic, where its latency would add to every launch.
    grid = (int)gridDim.x;
    asm volatile("" ::"s"(grid));
    // The output pointers are not among the preloaded arguments: read them
    // here too, in the same wait, rather than before the store, where the
    // load would add its latency to the end of every launch.
    if constexpr (!MULTI) {
      ys[0] = static_cast<float*>(const_cast<void*>(a3));
      if constexpr (NW == 2 || PAIR) {
        ys[1] = p.part0.y[1];
        asm volatile("" ::"s"(ys[1]));
      }
    } else if constexpr (MPRE) {
      ys[0] = p.out.y[0];
      ys[1] = p.out.y[1];
      ys[2] = p.out.y[2];
      asm volatile("" ::"s"(ys[0]), "s"(ys[1]), "s"(ys[2]));
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < J * XS; ++j) {
        const int f = NE4 * (LW * wv + L * (j / XS)) + kWave * (j % XS) + lane;
        const int li = kWave * (j % XS) + lane;  // float4 within the slice
        const int e4 = li % NE4;
        const int u = LW * (j / XS) + li / NE4;
        if (f < n4) xs[(m * NE4 + e4) * XP + u] = xv[m][j];
        if constexpr (SUMS) {
          // sum of each 32-element half: 8 consecutive float4s on 8 consecutive lanes
          const float sm = group_sum(((xv[m][j].x + xv[m][j].y) + xv[m][j].z) + xv[m][j].w, 8);
          if (f < n4 && (e4 & 7) == 0) xsum[(m * U + u) * 2 + (e4 >> 3)] = sm;
        }
      }
    // LDS operations of one wave complete in order; this only keeps the
    // compiler from moving the reads above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // One row group: multiply the loaded chunks, issue the next group's loads,
  // then finish the butterfly across waves and store.
  auto group = [&](int it) {
    float acc[NW][R][MT];
#pragma unroll
    for (int s = 0; s < NW; ++s)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[s][r][m] = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int tg = vl + L * j;
      if (tg < n_chunks) compute_chunk<FMT, MT, NW, R>(ch[j], xs, xsum, XP, U, LW * j + c, tg, acc);
    }
    float* rb = red + (it & 1) * (NW * WV * ROWS * MT);
#pragma unroll
    for (int s = 0; s < NW; ++s)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float v = acc[s][r][m];
          v += dpp_mov<0xB1>(v);                      // quad_perm [1,0,3,2]
          v += dpp_mov<0x4E>(v);                      // quad_perm [2,3,0,1]
          if constexpr (LW == 8) v += dpp_mov<0x141>(v);  // row_half_mirror
          if (c == 0) rb[((s * WV + wv) * ROWS + rset + RS * r) * MT + m] = v;
        }
    const int g_done = g;
    // where group g_done's outputs go (stream 0; a dual part's stream 1 is
    // picked per thread below), worked out here where it is uniform
    PartStore ps;
    if constexpr (MULTI && MPRE) {
      const bool past0 = g_done >= ag1, past1 = g_done >= ag2;
      ps.y = sel(past1, ys[2], sel(past0, ys[1], ys[0]));
      ps.n = sel(past1, an2, sel(past0, an1, an0));
      ps.group0 = sel(past1, ag2, sel(past0, ag1, 0));
      ps.ldy = MT == 1 ? 0 : p.out.ldy[__builtin_amdgcn_readfirstlane((past0 ? 1 : 0) + (past1 ? 1 : 0))];
    } else if constexpr (MULTI) {
      ps = part_store(p, part_of_group(p, g_done));
    } else {
      ps = PartStore{ys[0], MT == 1 ? 0 : p.part0.ldy, an0, 0};
      if constexpr (PAIR) {
        // groups of the second stream are numbered after the first's
        const bool second = g_done >= pair_groups;
        ps.y = sel(second, ys[1], ys[0]);
        ps.group0 = second ? pair_groups : 0;
      }
    }
    g += grid;
    if (g < an_groups) {
      view_of(g, cv);
      fetch_all(cv);
    }
    __syncthreads();
    if (threadIdx.x < NW * ROWS * MT) {
      const int s = threadIdx.x / (ROWS * MT);
      const int r = threadIdx.x / MT % ROWS;
      const int m = threadIdx.x % MT;
      constexpr int WS = ROWS * MT;  // stride between waves
      const float* a = rb + (s * WV * ROWS + r) * MT + m;
      const float b0 = a[0 * WS] + a[1 * WS];
      const float b1 = a[2 * WS] + a[3 * WS];
      float t;
      if constexpr (WV == 16) {
        const float b2 = a[4 * WS] + a[5 * WS];
        const float b3 = a[6 * WS] + a[7 * WS];
        const float b4 = a[8 * WS] + a[9 * WS];
        const float b5 = a[10 * WS] + a[11 * WS];
        const float b6 = a[12 * WS] + a[13 * WS];
        const float b7 = a[14 * WS] + a[15 * WS];
        t = ((b0 + b1) + (b2 + b3)) + ((b4 + b5) + (b6 + b7));
      } else if constexpr (WV == 8) {
        const float b2 = a[4 * WS] + a[5 * WS];
        const float b3 = a[6 * WS] + a[7 * WS];
        t = (b0 + b1) + (b2 + b3);
      } else {
        t = b0 + b1;
      }
      float* yo = ps.y;
      if constexpr (NW == 2) yo = sel(s == 0, ps.y, ys[1]);
      const int rr = (g_done - ps.group0) * ROWS + r;
      if (rr < ps.n && (MT == 1 || m < p.m_rows)) yo[(size_t)m * ps.ldy + rr] = t;
    }
  };
  // The first group is peeled off the loop, so that its loads, issued in
  // straight-line code, are waited for one chunk at a time.
  group(0);
  for (int it = 1; g < an_groups; ++it) group(it);
}

// The leading scalar arguments repeat what the first loads need from p: the
// hardware preloads leading scalar kernel arguments into scalar registers
// before the wave starts (the build asks for it; a struct argument is not
// preloaded), so those loads leave without waiting for a kernel-argument
// load.  The number of preloaded dwords costs time too: 14 instead of 13
// measured 0.04 us more per launch of the 4096 x 4096 Q4_K product, so a
// single-part launch passes 12 and only a multi-part launch with its parts
// in the arguments passes 14.
//
// Single part, or a multi-part launch that reads its part table from p:
// x, part 0's weights (both streams of a dual or pair launch), its first
// output, K, its rows, the row stride and the group count.
template <int FMT, int MT, int NW, int L, int R, int J, int WV, bool MULTI, bool PAIR = false>
__global__ void __launch_bounds__(64 * WV) gemv_ks_kernel(const float* ax, const uint8_t* aw0, const uint8_t* aw1,
                                                          float* ay0, int ak, int an0, int arow_bytes, int an_groups,
                                                          GemvParams p) {
  gemv_ks_body<FMT, MT, NW, L, R, J, WV, MULTI, PAIR, false>(ax, aw0, aw1, ay0, ak, an0, arow_bytes, an_groups, 0, 0,
                                                              p);
}

// Up to three Q4_K parts with their parts in the arguments: x, the parts'
// weights, K, their rows, and the first groups of parts 1 and 2.
template <int FMT, int MT, int NW, int L, int R, int J, int WV>
__global__ void __launch_bounds__(64 * WV) gemv_ks_mp_kernel(const float* ax, const uint8_t* aw0, const uint8_t* aw1,
                                                             const uint8_t* aw2, int ak, int an0, int an1, int an2,
                                                             int ag1, int ag2, GemvParams p) {
  gemv_ks_body<FMT, MT, NW, L, R, J, WV, true, false, true>(ax, aw0, aw1, aw2, ak, an0, an1, an2, ag1, ag2, p);
}

// ---------------------------------------------------------------------------
// Plain kernel for shapes and alignments the chunked kernel does not take
// (K not a multiple of 64 for Q4_0, misaligned Q4_K rows, affine K % 32 != 0,
// group_size < 32 or misaligned codes): one thread per output.  Launched once
// per part.  The sum over K is split so that no serial f32 chain is longer
// than 64 terms: a sequential chain over each 32-element piece of K, the piece
// sums added 64 at a time into the next level, and so on, in a fixed order.
struct PlainParams {
  const uint8_t* w[2];
  const float* scales;
  const float* biases;
  const float* x;
  float* y[2];
  long long ldy;
  long long row_bytes;
  int n, k, gs;
};

// Weight k of a row of the plain kernel's format, decoded to f32 (Q4_0: exactly
// d (q - 8); Q4_K: one rounding of d sc q - dmin m; affine: one rounding of s q + b).
template <int FMT>
__device__ __forceinline__ float plain_weight(const PlainParams& p, const uint8_t* row, int n, int k) {
  if constexpr (FMT == FMT_Q40) {
    const uint8_t* blk = row + 18 * (k / 32);
    const uint32_t d = blk[0] | ((uint32_t)blk[1] << 8);
    const int j = k % 32;
    const uint32_t byte = blk[2 + (j & 15)];
    const int nib = j < 16 ? (int)(byte & 15u) : (int)(byte >> 4);
    return f16_bits_to_f32(d) * (float)(nib - 8);
  } else if constexpr (FMT == FMT_Q4K) {
    const uint8_t* sb = row + 144 * (k / 256);
    const int e = k % 256;
    const int j = e / 32;
    const float d = f16_bits_to_f32(sb[0] | ((uint32_t)sb[1] << 8));
    const float dmin = f16_bits_to_f32(sb[2] | ((uint32_t)sb[3] << 8));
    int sc, mn;
    q4k_sc_m(sb + 4, j, sc, mn);
    const uint32_t byte = sb[16 + 32 * (e / 64) + (e % 32)];
    const int q = (e % 64) < 32 ? (int)(byte & 15u) : (int)(byte >> 4);
    return __builtin_fmaf(d * (float)sc, (float)q, -(dmin * (float)mn));
  } else {
    const int groups = p.k / p.gs;
    const size_t gi = (size_t)n * groups + k / p.gs;
    uint32_t code;
    if constexpr (FMT == FMT_AFF) code = row[k];
    else code = (row[k >> 1] >> (4 * (k & 1))) & 15u;
    return __builtin_fmaf(p.scales[gi], (float)code, p.biases[gi]);
  }
}

template <int FMT, int NW>
__global__ void __launch_bounds__(256) gemv_plain_kernel(PlainParams p, int m_count) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= p.n || m >= m_count) return;
  const float* xr = p.x + (size_t)m * p.k;
#pragma unroll
  for (int s = 0; s < NW; ++s) {
    const uint8_t* row = p.w[s] + (size_t)n * (size_t)p.row_bytes;
    // s1 adds up to 64 piece sums, s2 up to 64 values of s1, ... (K < 2^31
    // needs five levels)
    float s1 = 0.0f, s2 = 0.0f, s3 = 0.0f, s4 = 0.0f, s5 = 0.0f;
    int c1 = 0, c2 = 0, c3 = 0, c4 = 0;
    for (int k0 = 0; k0 < p.k; k0 += 32) {
      const int k1 = p.k - k0 < 32 ? p.k : k0 + 32;
      float a = 0.0f;
      for (int k = k0; k < k1; ++k) a = __builtin_fmaf(xr[k], plain_weight<FMT>(p, row, n, k), a);
      s1 += a;
      if (++c1 == 64) {
        s2 += s1, s1 = 0.0f, c1 = 0;
        if (++c2 == 64) {
          s3 += s2, s2 = 0.0f, c2 = 0;
          if (++c3 == 64) {
            s4 += s3, s3 = 0.0f, c3 = 0;
            if (++c4 == 64) s5 += s4, s4 = 0.0f, c4 = 0;
          }
        }
      }
    }
    p.y[s][(size_t)m * p.ldy + n] = (((s5 + s4) + s3) + s2) + s1;
  }
}

}  // namespace qg
