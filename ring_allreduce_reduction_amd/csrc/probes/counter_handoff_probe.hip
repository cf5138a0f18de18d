// counter_handoff_probe.hip -- measurement probe (not part of libar.so).
// How long does one FIFO handoff between two wavefronts take, by where the
// counter lives, and does a payload published through an LDS counter ever
// read stale?  Each workgroup holds two wavefronts that hand a counter back
// and forth ITERS times; every hop writes 16 bytes per lane of payload in
// global memory, publishes the counter, and the other side reads the payload
// back and checks it.  Variants:
//   0: counters in global memory, workgroup-scope relaxed atomics
//   1: counters in LDS, workgroup scope; payload still in global memory
//   2: counters and payload device-coherent (agent-scope relaxed atomics,
//      payload stores drained with s_waitcnt vmcnt(0) before the counter)
// Every wait is bounded (SPIN_MAX polls); a timeout is counted and ends the
// loop.  Payload values carry a per-launch salt, so a stale read cannot match.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef unsigned int u32;
typedef unsigned long long u64;
constexpr int ITERS = 2000;
constexpr long SPIN_MAX = 2000000;

template <int V>
__device__ __forceinline__ u32 ldc(u32* g, u32* l) {
  if (V == 0) return __hip_atomic_load(g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (V == 1) return __hip_atomic_load(l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __hip_atomic_load(g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <int V>
__device__ __forceinline__ void stc(u32* g, u32* l, u32 v) {
  if (V == 0) __hip_atomic_store(g, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else if (V == 1) __hip_atomic_store(l, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else __hip_atomic_store(g, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int V>
__device__ __forceinline__ void rel() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if constexpr (V == 2) __builtin_amdgcn_s_waitcnt(0x0F70);
}
__device__ __forceinline__ void acq() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup"); }
template <int V>
__device__ __forceinline__ void stData(uint4* p, uint4 v) {
  if constexpr (V == 2) {
    __hip_atomic_store((u64*)p, ((u64)v.y << 32) | v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store((u64*)p + 1, ((u64)v.w << 32) | v.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *p = v;
  }
}
template <int V>
__device__ __forceinline__ uint4 ldData(const uint4* p) {
  if constexpr (V == 2) {
    const u64 a = __hip_atomic_load((const u64*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const u64 b = __hip_atomic_load((const u64*)p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return uint4{(u32)a, (u32)(a >> 32), (u32)b, (u32)(b >> 32)};
  } else {
    return *p;
  }
}

template <int V>
__global__ __launch_bounds__(128) void pingpong(uint4* data, u32* ctr, u64* cycles, u64* wall, int* err, u32 salt) {
  __shared__ u32 lctr[2];
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  uint4* mine = data + (size_t)blockIdx.x * 256 + w * 128;        // 2 x 64 x 16 B per wave
  uint4* theirs = data + (size_t)blockIdx.x * 256 + (1 - w) * 128;
  u32* gc = ctr + blockIdx.x * 64;                                  // 256 B apart per block
  if (threadIdx.x < 2) lctr[threadIdx.x] = 0;
  __syncthreads();
  u64 t0 = clock64();
  u64 w0 = wall_clock64();
  uint4 acc = {0, 0, 0, 0};
  bool ok = true;
  int bad = 0;
  for (int i = 1; i <= ITERS && ok; ++i) {
    // wave 0 sends on odd half-steps, wave 1 answers
    if (w == 0) {
      stData<V>(&mine[(i & 1) * 64 + lane], uint4{(u32)i ^ (salt << 16), acc.x, 0, 0});
      rel<V>();
      if (lane == 0) stc<V>(gc + 0, lctr + 0, (u32)i);
      long spins = 0;
      while (ldc<V>(gc + 32, lctr + 1) < (u32)i) if (++spins > SPIN_MAX) { ok = false; break; }
      acq();
      uint4 x = ldData<V>(&theirs[(i & 1) * 64 + lane]);
      acc.x += x.x;
      if (x.x != ((u32)i ^ (salt << 16))) ++bad;
    } else {
      long spins = 0;
      while (ldc<V>(gc + 0, lctr + 0) < (u32)i) if (++spins > SPIN_MAX) { ok = false; break; }
      acq();
      uint4 x = ldData<V>(&theirs[(i & 1) * 64 + lane]);
      acc.x += x.x;
      if (x.x != ((u32)i ^ (salt << 16))) ++bad;
      stData<V>(&mine[(i & 1) * 64 + lane], uint4{(u32)i ^ (salt << 16), acc.x, 0, 0});
      rel<V>();
      if (lane == 0) stc<V>(gc + 32, lctr + 1, (u32)i);
    }
    ok = __all(ok);
  }
  u64 t1 = clock64();
  u64 w1 = wall_clock64();
  if (!ok && lane == 0) atomicAdd(err, 1);
  if (bad) atomicAdd(err + 1, bad);
  if (threadIdx.x == 0) { cycles[blockIdx.x] = t1 - t0; wall[blockIdx.x] = w1 - w0; }
  if (acc.x == 0xFFFFFFFFu && acc.y == 7) data[0] = acc;   // keep acc live
}

// background load: streaming copy over a large buffer by other workgroups
__global__ __launch_bounds__(256) void stream(const uint4* a, uint4* b, size_t n, int reps) {
  for (int r = 0; r < reps; ++r)
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
      b[i] = a[i];
}

#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1); } } while (0)

static u32 g_salt = 0;

template <int V>
void run(int blocks, bool loaded, uint4* data, u32* ctr, u64* cyc, u64* wall, int* err, const uint4* sa, uint4* sb, size_t sn) {
  CK(hipMemset(ctr, 0, (size_t)blocks * 256));
  CK(hipMemset(err, 0, 2 * sizeof(int)));
  hipStream_t s1, s2;
  CK(hipStreamCreate(&s1));
  CK(hipStreamCreate(&s2));
  if (loaded) hipLaunchKernelGGL(stream, dim3(512), dim3(256), 0, s2, sa, sb, sn, 4);
  hipLaunchKernelGGL(pingpong<V>, dim3(blocks), dim3(128), 0, s1, data, ctr, cyc, wall, err, ++g_salt);
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  std::vector<u64> h(blocks), hw(blocks);
  int herr[2] = {0, 0};
  CK(hipMemcpy(h.data(), cyc, blocks * sizeof(u64), hipMemcpyDeviceToHost));
  CK(hipMemcpy(hw.data(), wall, blocks * sizeof(u64), hipMemcpyDeviceToHost));
  int rate = 0;
  CK(hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, 0));   // kHz
  double wmean = 0;
  for (auto c : hw) wmean += (double)c;
  wmean /= blocks;
  CK(hipMemcpy(herr, err, 2 * sizeof(int), hipMemcpyDeviceToHost));
  double mean = 0;
  for (auto c : h) mean += (double)c;
  mean /= blocks;
  // clock64 runs at the shader clock; report cycles per round trip
  printf("variant %d blocks %4d loaded %d: %.0f cycles, %.0f ns per round trip (2 hops), timeouts %d, stale reads %d\n", V,
         blocks, (int)loaded, mean / ITERS, wmean / ITERS / (rate * 1e-6), herr[0], herr[1]);
  CK(hipStreamDestroy(s1));
  CK(hipStreamDestroy(s2));
}

int main() {
  const int maxBlocks = 1024;
  uint4* data; u32* ctr; u64* cyc; u64* wall; int* err;
  CK(hipMalloc(&data, (size_t)maxBlocks * 256 * sizeof(uint4)));
  CK(hipMalloc(&ctr, (size_t)maxBlocks * 256));
  CK(hipMalloc(&cyc, maxBlocks * sizeof(u64)));
  CK(hipMalloc(&wall, maxBlocks * sizeof(u64)));
  CK(hipMalloc(&err, 2 * sizeof(int)));
  const size_t sn = (size_t)1 << 26;   // 1 GiB of uint4
  uint4 *sa, *sb;
  CK(hipMalloc(&sa, sn * sizeof(uint4)));
  CK(hipMalloc(&sb, sn * sizeof(uint4)));
  CK(hipMemset(sa, 1, sn * sizeof(uint4)));
  for (int blocks : {1, 256, 1024}) {
    run<0>(blocks, false, data, ctr, cyc, wall, err, sa, sb, sn);
    run<1>(blocks, false, data, ctr, cyc, wall, err, sa, sb, sn);
    run<2>(blocks, false, data, ctr, cyc, wall, err, sa, sb, sn);
  }
  for (int blocks : {1, 256}) {
    run<0>(blocks, true, data, ctr, cyc, wall, err, sa, sb, sn);
    run<1>(blocks, true, data, ctr, cyc, wall, err, sa, sb, sn);
    run<2>(blocks, true, data, ctr, cyc, wall, err, sa, sb, sn);
  }
  printf("done\n");
  return 0;
}
