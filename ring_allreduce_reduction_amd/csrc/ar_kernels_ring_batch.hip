// ar_kernels_ring_batch.hip -- the batched ring AllReduce kernels (several AllReduces per launch) (device code in ar_device.h).
#include "ar_device.h"

namespace ar {

KernelFn pickRingAllReduceBatch(const Plan& plan, int dtype, int op) {
  return pickRingProto<kCollAllReduce, true>(plan, dtype, op);
}

}  // namespace ar
