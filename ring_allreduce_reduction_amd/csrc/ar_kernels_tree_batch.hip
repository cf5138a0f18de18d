// ar_kernels_tree_batch.hip -- the batched double-binary-tree AllReduce kernels (device code in ar_device.h).
#include "ar_device.h"

namespace ar {

KernelFn pickTreeAllReduceBatch(const Plan& plan, int dtype, int op) { return pickTreeProto<true>(plan, dtype, op); }

}  // namespace ar
