// ar_kernels_ring_simple.hip -- the single-call ring AllReduce kernels, Simple protocol (device code in ar_device.h).
#include "ar_device.h"

namespace ar {

KernelFn pickRingAllReduceSimple(const Plan& plan, int dtype, int op) {
  return plan.proto == kSimple ? pickRingSimple<kCollAllReduce, false>(plan, dtype, op) : nullptr;
}

}  // namespace ar
