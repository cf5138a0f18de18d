// ar_kernels.hip -- picks and launches the kernel of a plan.  The kernels
// themselves (device code in ar_device.h) are compiled in the translation
// units ar_kernels_*.hip, one per family.
#include <map>
#include <mutex>
#include <tuple>

#include "ar_internal.h"

namespace ar {
namespace {

// Batched launches (several AllReduces from a task table) exist for
// AllReduce only.
KernelFn pickKernel(const Plan& plan, int coll, int dtype, int op, bool batch) {
  if (plan.algo == arAlgoTree) {
    if (coll != kCollAllReduce) return nullptr;
    return batch ? pickTreeAllReduceBatch(plan, dtype, op) : pickTreeAllReduce(plan, dtype, op);
  }
  if (coll == kCollAllReduce) {
    if (batch) return pickRingAllReduceBatch(plan, dtype, op);
    return plan.proto == kSimple ? pickRingAllReduceSimple(plan, dtype, op) : pickRingAllReduceLL(plan, dtype, op);
  }
  if (batch) return nullptr;
  if (coll == kCollReduceScatter) return pickRingReduceScatter(plan, dtype, op);
  if (coll == kCollAllGather) return pickRingAllGather(plan, dtype, op);
  return nullptr;
}

}  // namespace

hipError_t launchRing(const Plan& plan, int dtype, int op, const KernelArgs& args, hipStream_t stream) {
  KernelFn fn = pickKernel(plan, args.coll, dtype, op, args.nTasks > 0);
  if (fn == nullptr) return hipErrorInvalidValue;
  if (plan.nGroups > 1 && plan.proto == kSimple && plan.unroll > kGroupedSimpleUnrollMax)
    return hipErrorInvalidValue;   // that kernel has no cross-workgroup edges
  if (plan.launchCoop) {
    void* params[] = {(void*)&args};
    return hipLaunchCooperativeKernel((const void*)fn, dim3(plan.grid), dim3(plan.block), params,
                                      (unsigned)plan.ldsBytes, stream);
  }
  hipLaunchKernelGGL(fn, dim3(plan.grid), dim3(plan.block), (unsigned)plan.ldsBytes, stream, args);
  return hipGetLastError();
}

// Resident workgroups per CU of a kernel at a block size, per device.  The
// planner asks for many (kernel, block) pairs on every call of a grouped
// ring or tree; the answers never change, so they are kept.
hipError_t ringKernelOccupancy(const Plan& plan, int coll, int dtype, int op, bool batch, int* blocksPerCU) {
  KernelFn fn = pickKernel(plan, coll, dtype, op, batch);
  if (fn == nullptr) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, int, int>, int> known;
  const auto key = std::make_tuple((const void*)fn, plan.block, plan.ldsBytes, dev);
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = known.find(key);
    if (it != known.end()) {
      *blocksPerCU = it->second;
      return hipSuccess;
    }
  }
  int n = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)fn, plan.block, (size_t)plan.ldsBytes);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(mu);
  known[key] = n;
  *blocksPerCU = n;
  return hipSuccess;
}

}  // namespace ar
