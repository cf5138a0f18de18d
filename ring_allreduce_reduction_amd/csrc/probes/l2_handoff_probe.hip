// l2_handoff_probe.hip -- measurement probe (not part of libar.so).
// Does a line written by one wavefront stay readable in L2 for a reader
// wavefront of the same workgroup?  One workgroup of 2 waves; wave 0 writes
// NB bytes, releases a flag (workgroup scope); wave 1 acquires and reads them
// back.  Run under rocprofv3 --pmc FETCH_SIZE / TCC_HIT_sum TCC_MISS_sum.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdint.h>
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int NB = 256 * 1024;            // bytes written then read
constexpr int NV = NB / 16;               // 16-byte vectors

template <int MODE>   // 0 plain store, 1 nontemporal store
__global__ void __launch_bounds__(128) write_then_read(v4u* buf, uint64_t* flag, v4u* out) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (wave == 0) {
    for (int i = lane; i < NV; i += 64) {
      v4u v = {(uint32_t)i, 1u, 2u, 3u};
      if (MODE == 0) buf[i] = v; else __builtin_nontemporal_store(v, &buf[i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_store(flag, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    uint64_t spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0 && spins < (1ull << 24)) {
      __builtin_amdgcn_s_sleep(1); ++spins;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    v4u acc = {0, 0, 0, 0};
    for (int i = lane; i < NV; i += 64) acc += buf[i];
    out[lane] = acc;
  }
}

__global__ void __launch_bounds__(64) read_cold(const v4u* buf, v4u* out) {
  v4u acc = {0, 0, 0, 0};
  for (int i = threadIdx.x; i < NV; i += 64) acc += buf[i];
  out[threadIdx.x] = acc;
}

int main() {
  v4u *buf, *buf2, *out; uint64_t* flag;
  if (hipMalloc(&buf, NB) || hipMalloc(&buf2, NB) || hipMalloc(&out, 64 * 16) || hipMalloc(&flag, 8)) return 1;
  hipMemset(buf2, 0, NB);
  for (int rep = 0; rep < 3; ++rep) {
    hipMemset(flag, 0, 8);
    hipLaunchKernelGGL(write_then_read<0>, dim3(1), dim3(128), 0, 0, buf, flag, out);
    hipMemset(flag, 0, 8);
    hipLaunchKernelGGL(write_then_read<1>, dim3(1), dim3(128), 0, 0, buf, flag, out);
    hipLaunchKernelGGL(read_cold, dim3(1), dim3(64), 0, 0, buf2, out);
  }
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  printf("probe done (256 KiB written+read per write_then_read dispatch)\n");
  return 0;
}
