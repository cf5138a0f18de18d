// ar_kernels_ring_ll128.hip -- the single-call ring AllReduce kernels, LL128 protocol (device code in ar_device.h).
#include "ar_device.h"

namespace ar {

KernelFn pickRingAllReduceLL128(const Plan& plan, int dtype, int op) {
  return plan.proto == kLL128 ? pickRingLL128Only<kCollAllReduce, false>(plan, dtype, op) : nullptr;
}

}  // namespace ar
