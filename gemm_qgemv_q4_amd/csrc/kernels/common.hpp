// Shared device helpers for the gfx950 kernels of libqgemv_q4.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

constexpr int kWave = 64;

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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

// Sum over the 64 lanes of a wave (xor butterfly; fixed order, so the
// result is the same on every call with the same inputs).
__device__ __forceinline__ float wave_sum_xor(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace qg
