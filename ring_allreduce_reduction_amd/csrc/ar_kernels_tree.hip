// ar_kernels_tree.hip -- the single-call double-binary-tree AllReduce kernels (device code in ar_device.h).
#include "ar_device.h"

namespace ar {

KernelFn pickTreeAllReduce(const Plan& plan, int dtype, int op) { return pickTreeProto<false>(plan, dtype, op); }

}  // namespace ar
