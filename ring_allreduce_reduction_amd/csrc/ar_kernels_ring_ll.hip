// ar_kernels_ring_ll.hip -- the single-call ring AllReduce kernels, LL and LL128 protocols (device code in ar_device.h).
#include "ar_device.h"

namespace ar {

KernelFn pickRingAllReduceLL(const Plan& plan, int dtype, int op) {
  return plan.proto != kSimple ? pickRingLL<kCollAllReduce, false>(plan, dtype, op) : nullptr;
}

}  // namespace ar
