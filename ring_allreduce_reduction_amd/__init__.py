"""Ring AllReduce (reduce-scatter + all-gather over Simple / LL / LL128 FIFOs),
N virtual ranks emulated on one MI355X.  The compute path is the C-ABI library
libar.so (hand-written HIP for gfx950); `ring_allreduce_reduction_amd.binding`
marshals arguments to it.  Importing this package loads nothing; the binding
loads the library on first use (`import ring_allreduce_reduction_amd.binding`)."""
