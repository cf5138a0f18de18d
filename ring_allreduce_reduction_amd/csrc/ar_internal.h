// ar_internal.h -- layouts shared by the host side of libar.so and its HIP
// kernels.  Nothing here is visible through the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ar.h"

namespace ar {

constexpr int kWave = 64;                 // CDNA wavefront width
constexpr int kMaxMembersPerGroup = 16;   // ring members (one wavefront each) per workgroup
constexpr int kMaxWorkers = 32768;        // (rank, lane) wavefronts a comm provisions FIFOs for
// FIFO depth in slots per protocol (LL, LL128, Simple).  The pages' ring
// FIFO has 8 steps; on MI355X a 2-slot Simple FIFO of 8 KiB slots measured
// fastest (the smaller live footprint outweighs the lost slack).
constexpr int kDefaultSlots[3] = {8, 8, 2};
constexpr int kMaxSlots = 8;              // FIFO depth provisioned per worker
constexpr int kLdsFifoSlots = 3;          // depth of FIFOs kept in LDS
constexpr int kGroupedSlotsMax = 4;       // rings cut into workgroups: FIFO depth at most, where it
                                          // fits LDS (at most kMaxSlots)

// One ring member is one wavefront.  Per FIFO slot ("step") a wavefront moves
// `unroll` pieces per lane:
//   Simple: 16-byte pieces, slot = unroll KiB, all payload.
//   LL:     16-byte lines {data0, flag, data1, flag}: 8 payload bytes per lane.
//   LL128:  each wavefront instruction fills 8 lines of 128 bytes; a line is
//           seven 16-byte payload pieces, 8 payload bytes and an 8-byte flag.
constexpr int kSimpleUnrollMax = 8;       // Simple slot = unroll KiB (1, 2, 4 or 8)
constexpr int kSimpleUnrollDefault = 8;
constexpr int kBatchSimpleUnrollMax = 8;  // batched ring launches: any Simple slot (8 KiB fits in
                                          // 120 VGPRs with the task loop)
constexpr int kGroupedSimpleUnrollMax = 4;  // rings cut into several workgroups: Simple slot at most
                                           // 4 KiB (the 8 KiB kernel holds no cross-workgroup edge
                                           // code, which would make it spill)
constexpr int kGroupedWavesPerCU = 24;     // single-call rings and trees cut into workgroups:
                                          // their wavefronts per CU at most
constexpr int kTreeSimpleUnrollMax = 4;   // the tree's Simple slot is at most 4 KiB (three slot
                                          // arrays live per lane: 8 KiB would spill)
constexpr int kTreeEdges = 3;             // a tree node's FIFOs: from d0, from d1, from its parent
constexpr int kLLUnroll = 2;
constexpr int kLL128Unroll = 2;           // LL128 slot in 1 KiB units (8 lines of 128 bytes)
constexpr int kLL128UnrollLarge = 4;      // single-call rings may use 4-unit LL128 slots

constexpr int kSimpleSlotBytesMax = kSimpleUnrollMax * kWave * 16;   // 8192
constexpr int kLLSlotBytes = kLLUnroll * kWave * 16;           // 2048 wire
constexpr int kLLSlotPayload = kLLUnroll * kWave * 8;          // 1024 payload
constexpr int kLL128LinePayload = 120;
constexpr int kLL128LineBytes = 128;                           // 120 payload + the 8-byte flag
constexpr int kLL128UnitBytes = kWave * 16;                    // 1024 = 8 lines
constexpr int kLL128UnitPayload = 8 * kLL128LinePayload;       // 960
constexpr int kLL128SlotBytesMax = kLL128UnrollLarge * kLL128UnitBytes;

// Nominal chunk sizes (bytes).  Simple: two slices of AR_SLICE_BYTES (one
// chunk = 2 slices).  LL and LL128: builder choices, multiples of 16 bytes.
constexpr size_t kDefaultSliceBytes = 512 * 1024;
constexpr size_t kLLChunkBytes = 64 * 1024;
constexpr size_t kLL128ChunkBytes = 240 * 1024;

// Receive-side counters of one FIFO (one per protocol and worker).  The
// sender bumps `tail` after filling a slot, the receiver bumps `head` after
// draining one; each counter has a 128-byte line of its own.  Both are
// monotonic for the life of the comm, so no reset is ever needed between
// calls; at every call boundary tail == head.
struct Conn {
  uint64_t tail;
  uint64_t pad0[15];
  uint64_t head;
  uint64_t pad1[15];
};
static_assert(sizeof(Conn) == 256, "Conn layout");

// Host-pinned, device-visible control block.
struct Control {
  uint32_t abortFlag;   // set by arCommAbort
  uint32_t pad0[31];
  uint32_t status;      // 0 ok; kStatusTimeout / kStatusAbort from the kernel
  uint32_t pad1[31];
};
constexpr uint32_t kStatusTimeout = 1;
constexpr uint32_t kStatusAbort = 2;

enum Proto : int { kLL = 0, kLL128 = 1, kSimple = 2 };
// Collectives run by the ring kernel (values of arFunc_t).
enum Coll : int { kCollAllReduce = 0, kCollReduceScatter = 1, kCollAllGather = 2 };

struct KernelArgs {
  const void* send[AR_MAX_RANKS];
  void* recv[AR_MAX_RANKS];
  char* fifo;                 // this protocol's FIFOs, fifoWorkerBytes per worker
  Conn* conn;                 // this protocol's counters, one per worker
  Control* ctrl;              // host-pinned control block (device address)
  uint32_t* failed;           // device word: nonzero once a member of this comm gave up
  uint64_t count;             // elements per rank (per rank block for ReduceScatter / AllGather)
  uint64_t chunkElems;        // nominal chunk (elements)
  uint64_t fifoWorkerBytes;   // nSlots * slot bytes
  uint64_t timeoutTicks;      // wall-clock ticks a wait may take
  int nranks;
  int nChannels;
  int lanes;                  // wavefronts per (rank, channel)
  int groupSize;              // ring members per workgroup
  int nGroups;                // workgroups per (channel, lane)
  int nSlots;
  int aligned16;              // every send/recv base is 16-byte aligned
  int direct;                 // Simple: all-gather writes the successor's output directly
  int coll;                   // kCollAllReduce / kCollReduceScatter / kCollAllGather (selects the kernel)
  int deadRank;               // debug: this rank's members return at once
  // Batched launch (several AllReduces of one aggregate): nTasks rows of
  // 1 + 2 * nranks words {count, send[nranks], recv[nranks]}; 0 = one call
  // described by count / send / recv above.
  const uint64_t* tasks;
  int nTasks;
  int taskSlots;              // tasks in flight at once (each on nChannels x lanes wavefront sets)
  int laneSets;               // single call: workgroup FIFO sets (<= nChannels x lanes); set L runs
                              // (channel, lane) pairs L, L + laneSets, ...
  int groupSpread;            // debug: groups of one lane on consecutive workgroup ids (other XCDs)
  // 1: every member starts at step 0 and publishes nothing when it ends (the
  // comm-less AllReduce, whose rings keep every edge's counters in LDS): no
  // state carries from one call to the next, so no counter need persist
  int freshSteps;
};

// Everything arAllReduce decides for one call.
struct Plan {
  int algo = 0;               // arAlgoRing or arAlgoTree
  int proto = 0;
  int nChannels = 0;
  uint64_t chunkElems = 0;
  int lanes = 0;
  int groupSize = 0;
  int nGroups = 1;            // the kernel picked for the plan depends on it (one group or several)
  int grid = 0;
  int block = 0;
  int slotBytes = 0;
  int slotPayload = 0;
  int nSlots = 0;
  int unroll = 0;             // pieces per lane per slot
  int taskSlots = 0;          // batched launches: collectives running at once
  int laneSets = 0;           // single-group single call: FIFO sets the grid runs (see KernelArgs)
  bool direct = false;
  bool cooperative = false;   // the whole grid must be co-resident (rings / trees cut into workgroups)
  bool launchCoop = false;    // launched with the cooperative launch call (else a plain launch)
  bool perKind = false;       // single-workgroup LL128 rings: steps compiled per kind (small grids)
  bool ldsFifo = false;       // single-workgroup Simple rings, single calls: FIFO slots in LDS
  int ldsBytes = 0;           // dynamic LDS per workgroup (N x nSlots x slot bytes with ldsFifo)
  float predictedUs = 0.0f;
};

// Provided by ar_kernels.hip (the picker functions below by ar_kernels_*.hip).
hipError_t launchRing(const Plan& plan, int dtype, int op, const KernelArgs& args, hipStream_t stream);
hipError_t ringKernelOccupancy(const Plan& plan, int coll, int dtype, int op, bool batch, int* blocksPerCU);

// The kernel for a plan, element type and op, or nullptr; each family is
// compiled in a translation unit of its own (ar_kernels_*.hip) so the build
// runs them in parallel.
typedef void (*KernelFn)(const KernelArgs);
KernelFn pickRingAllReduceSimple(const Plan& plan, int dtype, int op);   // single call, Simple
KernelFn pickRingAllReduceLL(const Plan& plan, int dtype, int op);       // single call, LL / LL128
KernelFn pickRingAllReduceLL128(const Plan& plan, int dtype, int op);    // single call, LL128
KernelFn pickRingAllReduceBatch(const Plan& plan, int dtype, int op);    // batched launch
KernelFn pickRingReduceScatter(const Plan& plan, int dtype, int op);
KernelFn pickRingAllGather(const Plan& plan, int dtype, int op);
KernelFn pickTreeAllReduce(const Plan& plan, int dtype, int op);        // single call
KernelFn pickTreeAllReduceBatch(const Plan& plan, int dtype, int op);   // batched launch

// Argument checks of one collective (shared by the comm calls and the
// comm-less AllReduce); also reports 16- and 128-byte alignment.
arResult_t checkCollArgs(int N, int func, const void* const* sendbufs, void* const* recvbufs, size_t count,
                         int dtype, int op, bool* aligned16, bool* aligned128);

// The comm-less AllReduce: ring, Simple, rings of at most 16 ranks, its FIFOs
// in `scratch` (scratchBytes of device memory on the current device, owned by
// the caller of this function).  Allocates nothing.
constexpr size_t kScratchHeaderBytes = 4096;   // control block and failed word
arResult_t allReduceInScratch(char* scratch, size_t scratchBytes, const void* const* sendbufs, void* const* recvbufs,
                              int nranks, int nChannels, size_t count, int dtype, int op, hipStream_t stream);

inline int elemSize(int dtype) {
  switch (dtype) {
    case arInt32: case arFloat32: return 4;
    case arFloat16: case arBfloat16: return 2;
    case arUint64: return 8;
    default: return 0;
  }
}

}  // namespace ar
