// Shared device helpers for the gfx950 kernels of libqgemv_q4.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

constexpr int kWave = 64;

// Weight formats: GGML block_q4_0, GGML block_q4_K, MLX-style affine groups
// with u8 codes, and the same with codes packed eight per u32.
enum { FMT_Q40 = 0, FMT_Q4K = 1, FMT_AFF = 2, FMT_AFF4 = 3 };

// Most weight tensors (parts) one product may have.
constexpr int kMaxParts = 8;

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4a4 __attribute__((ext_vector_type(4), aligned(4)));  // dword-aligned: one global_load_dwordx4
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Hide a value from the optimiser so that a following byte extract maps to
// v_cvt_f32_ubyteN instead of being re-folded into one bfe per nibble.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}

// Byte i (0..3) of v as a float: v_cvt_f32_ubyte{i}.
template <int I>
__device__ __forceinline__ float ubyte_f32(uint32_t v) {
  if constexpr (I == 3) return (float)(v >> 24);
  else return (float)((v >> (8 * I)) & 0xFFu);
}

// Four signed codes, one int8 per byte, as floats (v_cvt_f32_i32 with a
// sign-extended byte source).
__device__ __forceinline__ void signed_codes_f32(uint32_t v, float& q0, float& q1, float& q2, float& q3) {
  q0 = (float)(int8_t)(v);
  q1 = (float)(int8_t)(v >> 8);
  q2 = (float)(int8_t)(v >> 16);
  q3 = (float)(int8_t)(v >> 24);
}

// Q4_0 nibbles as signed int8 bytes 16 (q - 8), exact: flipping the top bit
// of a 4-bit code q gives q - 8 in 4-bit two's complement, and placed in the
// top half of a byte that reads as the int8 16 (q - 8).  The factor 16 is
// taken out of the block scale (d / 16 is exact), so a block of codes 8
// contributes exactly 0 and the sum is d * sum x (q - 8) as the format
// defines it.
__device__ __forceinline__ uint32_t q40_hi16(uint32_t q) { return (q ^ 0x88888888u) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t q40_lo16(uint32_t q) { return ((q ^ 0x88888888u) << 4) & 0xF0F0F0F0u; }

// DPP lane moves (gfx9 encodings): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of `width` lanes (width = 4, 8, 16, 32 or 64);
// every lane of a group gets the group's sum.  Within a row of 16 lanes the
// partial sums move by DPP (no LDS traffic): xor 1, xor 2, then the half-row
// and row mirrors, which pair each quad (then each half-row) with its partner.
// The last one or two steps cross rows with a lane shuffle.  The order of the
// additions is fixed (the same as an xor butterfly), so results are
// reproducible bit for bit.
__device__ __forceinline__ float group_sum(float v, int width) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  if (width >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror
  if (width >= 16) v += dpp_mov<0x140>(v);  // row_mirror
  if (width >= 32) v += __shfl_xor(v, 16, kWave);
  if (width >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Scale and min of sub-block j (0..7) of a block_q4_K from its 12 packed
// scale bytes s12: 6 bits each; for j >= 4 the top two bits live in bits 6..7
// of bytes j-4 (scale) and j (min).
__device__ __forceinline__ void q4k_sc_m(const uint8_t* s12, int j, int& sc, int& mn) {
  if (j < 4) {
    sc = s12[j] & 63;
    mn = s12[j + 4] & 63;
  } else {
    sc = (s12[j + 4] & 0x0F) | ((s12[j - 4] >> 6) << 4);
    mn = (s12[j + 4] >> 4) | ((s12[j] >> 6) << 4);
  }
}

// Sum over the 64 lanes of a wave (xor butterfly; fixed order).
__device__ __forceinline__ float wave_sum_xor(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace qg
