// stream_ceiling.hip -- measurement probe, not part of libar.so.
//
// Plain streaming kernels that move a known number of bytes through HBM with
// the same access style as the ring kernel's user-buffer traffic (16-byte
// vectors per lane, non-temporal loads and stores).  Their rate on the box is
// the practical ceiling for an HBM-bound kernel, reported beside the 8 TB/s
// datasheet peak:
//   kind 0  copy:               b = a            (1 read, 1 write)
//   kind 1  two reads, a write: b = a + c (u32)  (the reduce-scatter step's mix)
//   kind 2  read only:          sum of a         (result kept only if impossible)
//   kind 3  write only:         b = constant
// Buffers hold `bytes` bytes each (a multiple of 16); grid-stride loops, four
// vectors in flight per lane.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kBlock = 256, kUnroll = 4;

template <int KIND>
__global__ void __launch_bounds__(kBlock) streamKernel(const v4u* __restrict__ a, const v4u* __restrict__ c,
                                                       v4u* __restrict__ b, size_t n) {
  const size_t stride = (size_t)gridDim.x * kBlock * kUnroll;
  v4u acc = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * kBlock * kUnroll + threadIdx.x; i < n; i += stride) {
    v4u x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + (size_t)u * kBlock;
      if (j >= n) continue;
      if (KIND == 3) x[u] = v4u{1u, 2u, 3u, 4u};
      else x[u] = __builtin_nontemporal_load(a + j);
      if (KIND == 1) x[u] += __builtin_nontemporal_load(c + j);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + (size_t)u * kBlock;
      if (j >= n) continue;
      if (KIND == 2) acc += x[u];
      else __builtin_nontemporal_store(x[u], b + j);
    }
  }
  if (KIND == 2 && acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) b[0] = acc;   // keeps the loads alive
}
}  // namespace

// Launch one pass of `kind` over `bytes` bytes on `stream` (a hipStream_t);
// 0 on success, -1 on a bad argument, else the hipError_t of the launch.
extern "C" int streamCeilingLaunch(int kind, const void* a, const void* c, void* b, size_t bytes, int grid,
                                   void* stream) {
  if (bytes % 16 != 0 || grid < 1 || kind < 0 || kind > 3) return -1;
  if ((kind != 3 && a == nullptr) || (kind == 1 && c == nullptr) || b == nullptr) return -1;
  const size_t n = bytes / 16;
  const hipStream_t s = (hipStream_t)stream;
  const v4u* va = (const v4u*)a;
  const v4u* vc = (const v4u*)c;
  v4u* vb = (v4u*)b;
  switch (kind) {
    case 0: hipLaunchKernelGGL(streamKernel<0>, dim3(grid), dim3(kBlock), 0, s, va, vc, vb, n); break;
    case 1: hipLaunchKernelGGL(streamKernel<1>, dim3(grid), dim3(kBlock), 0, s, va, vc, vb, n); break;
    case 2: hipLaunchKernelGGL(streamKernel<2>, dim3(grid), dim3(kBlock), 0, s, va, vc, vb, n); break;
    case 3: hipLaunchKernelGGL(streamKernel<3>, dim3(grid), dim3(kBlock), 0, s, va, vc, vb, n); break;
  }
  return (int)hipGetLastError();
}
