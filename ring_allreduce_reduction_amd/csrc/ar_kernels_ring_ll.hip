// ar_kernels_ring_ll.hip -- the single-call ring AllReduce kernels, LL protocol (device code in ar_device.h).
#include "ar_device.h"

namespace ar {

KernelFn pickRingAllReduceLL(const Plan& plan, int dtype, int op) {
  if (plan.proto == kLL128) return pickRingAllReduceLL128(plan, dtype, op);
  return plan.proto == kLL ? pickRingLLOnly<kCollAllReduce, false>(plan, dtype, op) : nullptr;
}

}  // namespace ar
