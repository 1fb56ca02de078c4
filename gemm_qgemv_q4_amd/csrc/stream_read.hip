// Streaming-read probe for the benchmark's ceilings (not part of the product
// ABI; built into its own library, libqg_read.so, which only bench.py loads).
//
// qg_stream_read reads `bytes` bytes at `src` (16-byte aligned, a multiple of
// 16) once, in ordinary 16-byte loads like the GEMV kernels', and writes
// nothing (the XOR of the data is compared with a flag of 0, which never
// matches): the plain read of a buffer the size of a kernel's operands, timed
// like the kernels.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte loads in flight per thread and step

__global__ void __launch_bounds__(kThreads) stream_read_kernel(const uint4* __restrict__ src, long long n16,
                                                               unsigned* out, unsigned flag) {
  const long long stride = (long long)gridDim.x * kThreads * kUnroll;
  unsigned acc = 0;
  for (long long base = (long long)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16; base += stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long i = base + (long long)u * kThreads;
      v[u] = i < n16 ? src[i] : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (flag != 0 && acc == flag) out[blockIdx.x] = acc;
}

}  // namespace

extern "C" int qg_stream_read(const void* src, long long bytes, unsigned* out, int blocks, void* stream) {
  if (src == nullptr || bytes <= 0 || (bytes & 15) != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0 ||
      blocks < 1)
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), bytes / 16, out, 0u);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
