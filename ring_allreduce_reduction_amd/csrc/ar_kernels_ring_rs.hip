// ar_kernels_ring_rs.hip -- the ring ReduceScatter kernels (device code in ar_device.h).
#include "ar_device.h"

namespace ar {

KernelFn pickRingReduceScatter(const Plan& plan, int dtype, int op) {
  return pickRingProto<kCollReduceScatter, false>(plan, dtype, op);
}

}  // namespace ar
