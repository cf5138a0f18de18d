// ar_noalloc.hip -- arAllReduceNoAlloc, the AllReduce for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// Its FIFOs live in `scratch`, a fixed array in the library's device code:
// the loader gives every GPU the library runs on its own copy, held until
// the process ends.  Host code never passes the array's name to a kernel or
// copy (on the host it names a stand-in, not device memory): on a device's
// first call the device address is looked up once with hipGetSymbolAddress
// and kept per device, and every later use goes through that address.
#include <mutex>

#include "ar_internal.h"

namespace {
constexpr size_t kScratchBytes = 64u << 20;   // the most FIFO memory the entry point may use, per GPU
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex gScratchMu;
char* gScratchDev[kMaxDevices];   // device address of `scratch` on each device, once looked up

// Zero the scratch header (control block and failed word): the abort word a
// waiting member polls must read zero.  A kernel rather than a memset, so a
// first call made under graph capture records nothing but kernels.
__global__ void clearScratchHeader(uint32_t* words, int n) {
  for (int i = (int)threadIdx.x; i < n; i += (int)blockDim.x) words[i] = 0u;
}

// This device's scratch address: looked up on the device's first call (the
// device current), its header cleared on the caller's stream.
arResult_t scratchOf(int dev, hipStream_t stream, char** out) {
  std::lock_guard<std::mutex> lock(gScratchMu);
  if (gScratchDev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return arHipError;
    hipLaunchKernelGGL(clearScratchHeader, dim3(1), dim3(256), 0, stream, (uint32_t*)p,
                       (int)(ar::kScratchHeaderBytes / sizeof(uint32_t)));
    if (hipGetLastError() != hipSuccess) return arHipError;
    gScratchDev[dev] = (char*)p;
  }
  *out = gScratchDev[dev];
  return arSuccess;
}

}  // namespace

extern "C" arResult_t arAllReduceNoAlloc(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                         int nChannels, size_t count, arDataType_t dtype, arRedOp_t op,
                                         void* stream) {
  if (nranks < 1 || nranks > ar::kMaxMembersPerGroup) return arInvalidArgument;
  if (nChannels < 1 || nChannels > AR_MAX_CHANNELS) return arInvalidArgument;
  bool aligned16 = true, aligned128 = true;   // bad arguments enqueue nothing, the first call's set-up included
  const arResult_t chk = ar::checkCollArgs(nranks, ar::kCollAllReduce, sendbufs, recvbufs, count, dtype, op,
                                           &aligned16, &aligned128);
  if (chk != arSuccess || count == 0) return chk;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return arHipError;
  if (dev < 0 || dev >= kMaxDevices) return arInvalidUsage;
  char* s = nullptr;
  const arResult_t r = scratchOf(dev, (hipStream_t)stream, &s);
  if (r != arSuccess) return r;
  return ar::allReduceInScratch(s, kScratchBytes, sendbufs, recvbufs, nranks, nChannels, count, dtype, op,
                                (hipStream_t)stream);
}
