// l2_handoff_probe.hip -- measurement probe (not part of libar.so).
// Does a line written by one wavefront stay readable in L2 for a reader
// wavefront of the same workgroup, and does the writer's store policy
// matter?  One workgroup of 2 waves; wave 0 writes NB bytes, waits for its
// stores and releases a flag (workgroup scope); wave 1 acquires it and reads
// the bytes back.  Run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE /
// TCC_HIT_sum TCC_MISS_sum; each store policy is its own kernel:
//   write_then_read<0>  plain 16-byte stores
//   write_then_read<1>  non-temporal stores
//   write_then_read<2>  relaxed workgroup-scope 8-byte atomic stores (sc0)
//   write_then_read<3>  relaxed agent-scope atomic stores (sc1)
//   write_then_read<4>  relaxed system-scope atomic stores (sc0 sc1)
//   write_then_read<5>  plain stores to lines wave 0 read first (already valid in L2)
//   read_cold           reads NB bytes that no kernel wrote
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdint.h>
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint64_t u64;
constexpr int NB = 256 * 1024;            // bytes written then read
constexpr int NV = NB / 16;               // 16-byte vectors

template <int MODE>
__global__ void __launch_bounds__(128) write_then_read(v4u* buf, u64* flag, v4u* out) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (wave == 0) {
    if (MODE == 5) {
      v4u acc = {0u, 0u, 0u, 0u};
      for (int i = lane; i < NV; i += 64) acc += buf[i];
      if (acc.x == 0x9e3779b9u) out[64 + lane] = acc;   // keeps the loads alive
    }
    for (int i = lane; i < NV; i += 64) {
      const v4u v = {(uint32_t)i, 1u, 2u, 3u};
      u64* p = (u64*)&buf[i];
      const u64 lo = ((u64)v.y << 32) | v.x, hi = ((u64)v.w << 32) | v.z;
      if (MODE == 0 || MODE == 5) {
        buf[i] = v;
      } else if (MODE == 1) {
        __builtin_nontemporal_store(v, &buf[i]);
      } else if (MODE == 2) {
        __hip_atomic_store(p, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_store(p + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else if (MODE == 3) {
        __hip_atomic_store(p, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        __hip_atomic_store(p, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(p + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every store has completed
    if (lane == 0) __hip_atomic_store(flag, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    uint64_t spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0 && spins < (1ull << 24)) {
      __builtin_amdgcn_s_sleep(1);
      ++spins;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    v4u acc = {0u, 0u, 0u, 0u};
    for (int i = lane; i < NV; i += 64) acc += buf[i];
    out[lane] = acc;
  }
}

__global__ void __launch_bounds__(64) read_cold(const v4u* buf, v4u* out) {
  v4u acc = {0u, 0u, 0u, 0u};
  for (int i = threadIdx.x; i < NV; i += 64) acc += buf[i];
  out[threadIdx.x] = acc;
}

int main() {
  v4u *buf, *buf2, *out;
  u64* flag;
  if (hipMalloc(&buf, NB) || hipMalloc(&buf2, NB) || hipMalloc(&out, 128 * 16) || hipMalloc(&flag, 8)) return 1;
  (void)hipMemset(buf, 0, NB);
  (void)hipMemset(buf2, 0, NB);
  for (int rep = 0; rep < 3; ++rep) {
#define AR_PROBE_RUN(M)                                                                         \
  (void)hipMemset(flag, 0, 8);                                                                  \
  hipLaunchKernelGGL(write_then_read<M>, dim3(1), dim3(128), 0, 0, buf, flag, out);
    AR_PROBE_RUN(0) AR_PROBE_RUN(1) AR_PROBE_RUN(2) AR_PROBE_RUN(3) AR_PROBE_RUN(4) AR_PROBE_RUN(5)
#undef AR_PROBE_RUN
    hipLaunchKernelGGL(read_cold, dim3(1), dim3(64), 0, 0, buf2, out);
  }
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  printf("probe done (256 KiB written+read per write_then_read dispatch)\n");
  return 0;
}
