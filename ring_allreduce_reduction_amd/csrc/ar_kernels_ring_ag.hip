// ar_kernels_ring_ag.hip -- the ring AllGather kernels (device code in ar_device.h).
#include "ar_device.h"

namespace ar {

KernelFn pickRingAllGather(const Plan& plan, int dtype, int op) {
  return pickRingProto<kCollAllGather, false>(plan, dtype, op);
}

}  // namespace ar
