// Fused-QKV split: qkv[t, :] = [Q (q_sp) | K (k_sp) | V (v_sp)] -> contiguous
// q [seq, q_sp], k [seq, k_sp], v [seq, v_sp]; every input element is written
// to exactly one output, bit for bit (mlx-native qkv_split.rs, module doc).
//
// gfx950 design: a pure HBM copy.  When the three spans are multiples of 4
// floats and all four pointers are 16-byte aligned, each lane moves one
// float4 (global_load_dwordx4 / global_store_dwordx4, coalesced along the
// row); blockIdx.y walks tokens so no 64-bit division is needed per element.
// Loads are non-temporal: the fused input is read exactly once.
#pragma once
#include "common.hpp"

namespace qg {

template <typename T>
__global__ void __launch_bounds__(256) qkv_split_kernel(const T* __restrict__ qkv, T* __restrict__ q,
                                                        T* __restrict__ k, T* __restrict__ v,
                                                        long long seq, int qs, int ks, int vs) {
  const int ch = qs + ks + vs;
  const int qk = qs + ks;
  for (long long t = blockIdx.y; t < seq; t += gridDim.y) {
    const T* src = qkv + (size_t)t * ch;
    T* qd = q + (size_t)t * qs;
    T* kd = k + (size_t)t * ks;
    T* vd = v + (size_t)t * vs;
    for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < ch; c += gridDim.x * blockDim.x) {
      const T val = __builtin_nontemporal_load(src + c);
      if (c < qs) qd[c] = val;
      else if (c < qk) kd[c - qs] = val;
      else vd[c - qk] = val;
    }
  }
}

}  // namespace qg
