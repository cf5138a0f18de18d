// ar_comm.cpp -- communicator lifecycle, per-call planning and the C ABI.
//
// Init follows the reference's shape ["NCCL 原始碼解讀：一個 AllReduce 的 GPU
// 旅程", ch.3 §3.1-§3.6]: validate, allocate the comm with magic sentinels,
// read the environment once, provision per-protocol FIFOs and counters, and
// make device state visible once.  There is no bootstrap: one process owns
// every virtual rank.  An AllReduce follows ch.6 §一-§六: argument checks,
// count == 0 and one-rank short cuts, tuning, channel split, kernel arguments,
// one launch on the caller's stream.
#include <ctype.h>
#include <float.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "ar_internal.h"
#include "ar_tune_table.h"

// A ROCTx range around an API call, as the pages mark each API entry with an
// NVTX range ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.3 §3.1, ch.6, the
// ncclAllReduce call chain]: rocprofv3 --marker-trace records one per call
// (host time of the call: argument checks, planning and the enqueue).
struct ApiRange {
  explicit ApiRange(const char* name) { roctxRangePushA(name); }
  ~ApiRange() { roctxRangePop(); }
  ApiRange(const ApiRange&) = delete;
  ApiRange& operator=(const ApiRange&) = delete;
};

using namespace ar;

namespace {

constexpr uint64_t kCommMagic = 0x4152434f4d4d3031ull;   // "ARCOMM01"

// ----------------------------------------------------------- environment
// Read once per process and cached, like the reference's parameter cache
// [ch.3 §3.5]; AR_PROTO uses the reference's list syntax with '^' to exclude.
struct Env {
  int protoMask = 7;      // allowed protocols for tuning
  int forcedProto = -2;   // -2: none
  int forcedAlgo = -2;    // -2: none; else arAlgoRing / arAlgoTree (AR_ALGO)
  int nChannels = 0;      // 0: not set
  size_t sliceBytes = kDefaultSliceBytes;
  int nSteps = 0;         // 0: per-protocol defaults
  int64_t timeoutUs = 5000000;
  int debug = 0;          // 0 warn, 1 info, 2 trace
};

int protoFromName(const char* s, size_t n) {
  char buf[16] = {0};
  if (n >= sizeof(buf)) return -1;
  for (size_t i = 0; i < n; ++i) buf[i] = (char)toupper((unsigned char)s[i]);
  if (!strcmp(buf, "LL")) return arProtoLL;
  if (!strcmp(buf, "LL128")) return arProtoLL128;
  if (!strcmp(buf, "SIMPLE")) return arProtoSimple;
  return -1;
}

const Env& env() {
  static Env e;
  static std::once_flag once;
  std::call_once(once, [] {
    if (const char* p = getenv("AR_PROTO")) {
      bool negate = p[0] == '^';
      const char* s = negate ? p + 1 : p;
      int mask = 0;
      while (*s) {
        const char* t = strchr(s, ',');
        size_t n = t ? (size_t)(t - s) : strlen(s);
        int pr = protoFromName(s, n);
        if (pr >= 0) mask |= 1 << pr;
        else fprintf(stderr, "[ar] WARN ignoring unknown protocol in AR_PROTO=%s\n", p);
        s += n;
        if (*s == ',') ++s;
      }
      if (negate) mask = 7 & ~mask;
      if (mask != 0) {
        e.protoMask = mask;
        if (mask == 1 || mask == 2 || mask == 4) e.forcedProto = mask == 1 ? 0 : mask == 2 ? 1 : 2;
      }
    }
    if (const char* p = getenv("AR_ALGO")) {
      if (!strcasecmp(p, "RING")) e.forcedAlgo = arAlgoRing;
      else if (!strcasecmp(p, "TREE")) e.forcedAlgo = arAlgoTree;
      else fprintf(stderr, "[ar] WARN ignoring AR_ALGO=%s (RING or TREE)\n", p);
    }
    if (const char* p = getenv("AR_NCHANNELS")) e.nChannels = atoi(p);
    if (const char* p = getenv("AR_SLICE_BYTES")) {
      long long v = atoll(p);
      if (v >= 16 && v % 16 == 0) e.sliceBytes = (size_t)v;
      else fprintf(stderr, "[ar] WARN ignoring AR_SLICE_BYTES=%s (need a multiple of 16)\n", p);
    }
    if (const char* p = getenv("AR_STEPS")) {
      int v = atoi(p);
      if (v >= 2 && v <= kMaxSlots) e.nSteps = v;
      else fprintf(stderr, "[ar] WARN ignoring AR_STEPS=%s (2..%d)\n", p, kMaxSlots);
    }
    if (const char* p = getenv("AR_TIMEOUT_MS")) {
      long long v = atoll(p);
      if (v > 0) e.timeoutUs = v * 1000;
    }
    if (const char* p = getenv("AR_DEBUG")) {
      if (!strcasecmp(p, "INFO")) e.debug = 1;
      else if (!strcasecmp(p, "TRACE")) e.debug = 2;
    }
  });
  return e;
}

// The cost model's constants are the fit in ar_tune_table.txt (or AR_TUNE_FILE's
// "model" lines), read through ar::tuneTableModels.

constexpr int kStagingBuffers = 4;

// One collective queued inside arGroupStart / arGroupEnd.
struct GroupTask {
  int func;
  size_t count;
  int dtype;
  int op;
  hipStream_t stream;
  bool aligned16;
  bool aligned128;
  std::vector<const void*> send;
  std::vector<void*> recv;
};

}  // namespace

struct arComm {
  uint64_t startMagic;
  int nranks;
  int maxChannels;
  int proto;            // default protocol or arProtoAuto
  int algo;             // AllReduce algorithm or arAlgoAuto
  int nChannels;        // default channel count
  int device;
  int numCUs;
  int wallClockKHz;
  int nSlots[3];        // FIFO depth per protocol
  size_t sliceBytes;
  size_t llChunkBytes;     // nominal LL / LL128 chunks (0: the defaults)
  size_t ll128ChunkBytes;
  int lanesMax;         // lanes (channel x lane) per rank provisioned
  char* fifo[3];
  Conn* conn[3];
  size_t fifoWorkerBytes[3];
  int fifoDepth[3];     // slots per worker the protocol's FIFOs are provisioned for (0: none yet)
  Control* ctrlHost;
  Control* ctrlDev;
  uint32_t* failedDev;  // device word the kernels set when a member gives up
  arTuneModel_t models[3];       // ring
  arTuneModel_t treeModels[3];
  int64_t timeoutUs;
  int deadRank;
  int forcedLanes;      // 0: automatic
  int laneSetsMax;      // 0: one workgroup per (channel, lane); else at most this many FIFO sets
  int groupSpread;      // debug: a lane's groups on consecutive workgroup ids
  int groupSizeMax;     // members per workgroup at most (debug; kMaxMembersPerGroup by default)
  bool ldsFifo;         // Simple rings inside one workgroup may keep their FIFO slots in LDS
  int ldsSlots;         // depth of such LDS FIFOs
  bool slotsForced;     // a depth set by AR_STEPS or arDebugSlots (else rings cut into
                        // workgroups may take deeper FIFOs where they fit LDS)
  int ldsPerBlock;      // LDS bytes a workgroup may use
  int simpleUnroll;     // Simple slot size in KiB (1, 2, 4)
  int ll128Unroll;      // LL128 slot in 1 KiB units (2 or 4); 0: chosen per call
  bool direct;          // Simple all-gather writes outputs directly
  bool plainLaunch;     // grouped plans launched without the cooperative launch call
  hipStream_t lastStream;
  bool launched;
  bool aborted;
  uint64_t opCount;
  // group calls [ch.7 §一]: collectives queued until the outermost arGroupEnd
  std::vector<GroupTask> pending;
  bool inGroup;
  std::vector<arPlan_t> groupPlans;   // the last launched group's plans, call order
  uint64_t* taskTable;                // device rows {count, send[N], recv[N]}
  // pinned host copy sources, used in turn so that the host need not wait
  // for the previous group's copy before writing the next table
  uint64_t* taskStaging[kStagingBuffers];
  hipEvent_t stagingDone[kStagingBuffers];   // the last copy out of each
  bool stagingBusy[kStagingBuffers];
  int stagingNext;
  size_t taskTableWords;
  uint64_t endMagic;
};

namespace {

bool commOk(const arComm* c) {
  return c != nullptr && c->startMagic == kCommMagic && c->endMagic == kCommMagic;
}

// Slot geometry: Simple slots are `unroll` KiB; the FIFO is provisioned for
// the largest Simple slot.
int slotBytesOf(int proto, int unroll) {
  return proto == kSimple ? unroll * kWave * 16 : proto == kLL ? kLLSlotBytes : unroll * kLL128UnitBytes;
}
int slotPayloadOf(int proto, int unroll) {
  return proto == kSimple ? unroll * kWave * 16 : proto == kLL ? kLLSlotPayload : unroll * kLL128UnitPayload;
}

// FIFOs and counters of one protocol [ch.2 §2.1 buffSizes per protocol;
// ch.3 §3.6 devCommSetup]: every worker (N ranks x lanesMax (channel, lane)
// pairs) gets `depth` slots of the protocol's largest slot, zeroed with its
// counters.  A protocol's lines are never read as another's (LL flags live
// inside the data), so each has its own region.  Re-provisioning (a deeper
// FIFO) first waits for the comm's last stream, then starts the new region
// from zero: its counters restart at 0 along with every slot, so both ends
// of each FIFO still agree.
arResult_t provisionFifo(arComm* c, int p, int depth) {
  if (c->nranks < 2) return arSuccess;
  if (c->fifo[p] != nullptr && c->fifoDepth[p] >= depth) return arSuccess;
  if (c->fifo[p] != nullptr) {
    if (c->launched && hipStreamSynchronize(c->lastStream) != hipSuccess) return arHipError;
    (void)hipFree(c->fifo[p]);
    (void)hipFree(c->conn[p]);
    c->fifo[p] = nullptr;
    c->conn[p] = nullptr;
    c->fifoDepth[p] = 0;
  }
  const size_t workers = (size_t)c->nranks * (size_t)c->lanesMax;
  const size_t workerBytes = (size_t)depth * (size_t)slotBytesOf(p, p == kLL128 ? kLL128UnrollLarge : kSimpleUnrollMax);
  const size_t fb = workers * workerBytes, cb = workers * sizeof(Conn);
  if (hipMalloc((void**)&c->fifo[p], fb) != hipSuccess || hipMalloc((void**)&c->conn[p], cb) != hipSuccess ||
      hipMemset(c->fifo[p], 0, fb) != hipSuccess || hipMemset(c->conn[p], 0, cb) != hipSuccess) {
    if (c->fifo[p]) (void)hipFree(c->fifo[p]);
    if (c->conn[p]) (void)hipFree(c->conn[p]);
    c->fifo[p] = nullptr;
    c->conn[p] = nullptr;
    return arHipError;
  }
  // hipMemset is ordered on the null stream only: a kernel launched next on a
  // stream created non-blocking (as torch's are) could run while the FIFOs
  // and counters are still being cleared, and start from counters that the
  // clear then resets under it.  Wait for the clear before any launch.
  c->fifoWorkerBytes[p] = workerBytes;
  c->fifoDepth[p] = depth;
  return hipDeviceSynchronize() == hipSuccess ? arSuccess : arHipError;
}

// Device bytes a comm holds: FIFOs and counters of the protocols provisioned,
// the failed word, and the task table of grouped launches.
size_t deviceFootprint(const arComm* c) {
  size_t b = 256;   // the failed word's line
  const size_t workers = (size_t)c->nranks * (size_t)c->lanesMax;
  for (int p = 0; p < 3; ++p)
    if (c->fifo[p] != nullptr) b += workers * (c->fifoWorkerBytes[p] + sizeof(Conn));
  return b + c->taskTableWords * sizeof(uint64_t);
}

size_t chunkBytesOf(const arComm* c, int proto) {
  if (proto == kSimple) return 2 * c->sliceBytes;   // one chunk = 2 slices
  if (proto == kLL) return c->llChunkBytes > 0 ? c->llChunkBytes : kLLChunkBytes;
  return c->ll128ChunkBytes > 0 ? c->ll128ChunkBytes : kLL128ChunkBytes;
}

uint64_t divUpU(uint64_t x, uint64_t y) { return (x + y - 1) / y; }
uint64_t alignUpU(uint64_t x, uint64_t a) { return divUpU(x, a) * a; }

void freeComm(arComm* c) {
  for (int p = 0; p < 3; ++p) {
    if (c->fifo[p]) (void)hipFree(c->fifo[p]);
    if (c->conn[p]) (void)hipFree(c->conn[p]);
  }
  if (c->ctrlHost) (void)hipHostFree(c->ctrlHost);
  if (c->failedDev) (void)hipFree(c->failedDev);
  if (c->taskTable) (void)hipFree(c->taskTable);
  for (int i = 0; i < kStagingBuffers; ++i) {
    if (c->taskStaging[i]) (void)hipHostFree(c->taskStaging[i]);
    if (c->stagingDone[i]) (void)hipEventDestroy(c->stagingDone[i]);
  }
  c->startMagic = c->endMagic = 0;
  delete c;
}

// Parent of rank r in tree t of the double binary tree over n ranks (-1 for
// the root), as the kernel builds it: tree 0 is the in-order binary tree
// whose node r has parent (r with its lowest set bit cleared and the next bit
// up set, or only cleared when that is out of range); tree 1 relabels rank x
// as n-1-x (even n) or x-1 (odd n) and maps the parent back.  Used to count
// the tree edges that cross workgroups in a plan's device bytes.
int treeParent(int n, int r, int t) {
  const bool mirror = (n & 1) == 0;
  const int x = t == 0 ? r : mirror ? n - 1 - r : (r == 0 ? n - 1 : r - 1);
  if (x == 0) return -1;
  const int bit = x & -x;
  int up = (x & ~bit) | (bit << 1);
  if (up >= n) up = x & ~bit;
  if (t == 0) return up;
  return mirror ? n - 1 - up : (up + 1 == n ? 0 : up + 1);
}

// The public view of a plan (p == nullptr: the one-rank / empty short cut).
void exportPlan(const arComm* c, int func, size_t count, int dtype, const Plan* p, arPlan_t* out) {
  memset(out, 0, sizeof(*out));
  const double S = (double)count * elemSize(dtype);
  const double N = (double)c->nranks;
  out->modelBytes = func == arFuncAllReduce ? 5.0 * (N - 1.0) * S
                    : func == arFuncReduceScatter ? 3.0 * N * (N - 1.0) * S : 2.0 * N * (N - 1.0) * S;
  out->groupLaunch = -1;
  out->tasksInLaunch = 1;
  out->deviceBytes = out->modelBytes;
  if (p == nullptr) {
    out->proto = arProtoSimple;
    out->algo = arAlgoRing;
    return;
  }
  out->algo = p->algo;
  if (p->algo == arAlgoTree) out->modelBytes = (2.0 * N + 4.0 * (N - 1.0)) * S;
  out->proto = p->proto;
  out->nChannels = p->nChannels;
  out->chunkElems = p->chunkElems;
  out->lanesPerChannel = p->lanes;
  out->ranksPerGroup = p->groupSize;
  out->workgroups = p->grid;
  out->threadsPerGroup = p->block;
  out->stepBytes = p->slotBytes;
  out->stepPayload = p->slotPayload;
  out->nSlots = p->nSlots;
  out->predictedUs = p->predictedUs;
  out->deviceBytes = out->modelBytes;
  if (p->ldsFifo && p->algo == arAlgoTree) {
    // inputs read and outputs written once; each tree edge between
    // workgroups carries its share of the data up and back down, each slot
    // written and read once
    out->ldsFifoBytes = p->ldsBytes;
    double cross = 0.0;
    const int trees = p->nChannels > 1 ? 2 : 1;
    for (int t = 0; t < trees; ++t)
      for (int r = 0; r < N; ++r) {
        const int up = treeParent(N, r, t);
        if (up >= 0 && up / p->groupSize != r / p->groupSize) cross += 1.0 / trees;
      }
    out->deviceBytes = 2.0 * N * S + 4.0 * cross * S;
  } else if (p->ldsFifo) {
    // inputs read and outputs written once; a ring cut into G workgroups
    // also writes and reads a slot on each of its G edges between them at
    // every send (2N-2 sends of S/N per AllReduce member, N-1 of a block for
    // the two halves)
    out->ldsFifoBytes = p->ldsBytes;
    const double G = p->nGroups > 1 ? (double)p->nGroups : 0.0;
    out->deviceBytes = func == arFuncAllReduce ? 2.0 * N * S + 4.0 * (N - 1.0) * G * S / N
                                               : (N + 1.0) * N * S + 2.0 * (N - 1.0) * G * S;
  }
}

// The cost model a comm evaluates.  The pages' model prices one GPU per rank;
// here the N virtual ranks share one GPU's HBM, so a bandwidth-bound call
// slows with N at a fixed per-rank size.  The constants' caps (the
// bandwidth-bound regime) are fitted at kCalibRanks ranks; each algorithm's
// cap is scaled by its HBM bytes per model byte there over that at N:
//   ring (all three collectives): HBM bytes grow as N times the model's
//     (AllReduce 5(N-1)S against 2(N-1)S/N), so cap x kCalibRanks / N;
//   tree: (2N + 4(N-1))S against the model's S, so cap x (6*8-4) / (6N-4).
// Latency and per-channel terms are per ring member and stay as fitted.
constexpr int kCalibRanks = 8;

void sharedHbmModels(const arComm* c, arTuneModel_t ring[3], arTuneModel_t tree[3]) {
  const float n = (float)c->nranks;
  const float ringScale = (float)kCalibRanks / n;
  const float treeScale = (6.0f * (float)kCalibRanks - 4.0f) / (6.0f * n - 4.0f);
  for (int p = 0; p < 3; ++p) {
    ring[p] = c->models[p];
    ring[p].maxBwGBs *= ringScale;
    tree[p] = c->treeModels[p];
    tree[p].maxBwGBs *= treeScale;
  }
}

// The channel count of the 32 KiB-per-channel rule for nBytes (at most 64):
// the count the tuner's table was measured at.
int ruleChannels(uint64_t nBytes) {
  int c = 1;
  while (c * 2 <= AR_MAX_CHANNELS && nBytes / (uint64_t)(c * 2) >= 32768) c *= 2;
  return c;
}

// Algorithm, protocol and channels for a call of nBytes (per rank for
// AllReduce).  First the pages' cost model [ch.5 §一]; then, for an
// AllReduce whose candidates the tuner's table covers at the channel count it
// was measured at, the table's times override the model's, as the pages let a
// tuner plugin override the cost table before the argmin (step 3): the
// candidate with the shortest time wins (ring Simple, LL128, LL, then tree
// Simple, LL128, LL on ties), at the channel count the model gives it.
arResult_t tuneCall(const arComm* c, int func, uint64_t nBytes, int maxCh, unsigned algoMask, unsigned protoMask,
                    arAlgo_t* algoOut, arProto_t* protoOut, int* nchOut, float* predOut) {
  arTuneModel_t ringM[3], treeM[3];
  sharedHbmModels(c, ringM, treeM);
  arAlgo_t al = arAlgoRing;
  arProto_t pr = arProtoSimple;
  int ch = 1;
  float pred = 0.0f;
  arResult_t r = arTuneEvalAlgo((arFunc_t)func, c->nranks, maxCh, nBytes, ringM, treeM, algoMask, protoMask, &al,
                                &pr, &ch, &pred);
  if (r != arSuccess) return r;
  if (func == kCollAllReduce && c->nranks > 1 && nBytes > 0 && maxCh >= ruleChannels(nBytes)) {
    static const int order[6][2] = {{arAlgoRing, arProtoSimple}, {arAlgoRing, arProtoLL128}, {arAlgoRing, arProtoLL},
                                    {arAlgoTree, arProtoSimple}, {arAlgoTree, arProtoLL128}, {arAlgoTree, arProtoLL}};
    float best = FLT_MAX;
    int bi = -1;
    for (int i = 0; i < 6 && tuneTableCovers(c->nranks); ++i) {
      const int a = order[i][0], p = order[i][1];
      if (!(algoMask & (1u << a)) || !(protoMask & (1u << p))) continue;
      float t = 0.0f;
      if (!tuneTableTime(c->nranks, nBytes, a, p, &t)) continue;   // it cannot run there
      if (t < best) {
        best = t;
        bi = i;
      }
    }
    if (bi >= 0) {
      al = (arAlgo_t)order[bi][0];
      pr = (arProto_t)order[bi][1];
      r = arTuneEvalAlgo((arFunc_t)func, c->nranks, maxCh, nBytes, ringM, treeM, 1u << al, 1u << pr, nullptr, nullptr,
                         &ch, nullptr);
      if (r != arSuccess) return r;
      pred = best;
    }
  }
  if (algoOut) *algoOut = al;
  if (protoOut) *protoOut = pr;
  if (nchOut) *nchOut = ch;
  if (predOut) *predOut = pred;
  return arSuccess;
}

// Protocol, channels, chunk, lanes and grid for one call, or for a batched
// launch (`batch`) of `nTasks` collectives whose largest has `count` elements
// and whose bytes together are `tuneBytes` (0: a single call).
arResult_t makePlan(arComm* c, int func, uint64_t count, int dtype, int op, bool aligned128, Plan* plan,
                    bool batch = false, int nTasks = 1, uint64_t tuneBytes = 0) {
  const Env& e = env();
  const int esz = elemSize(dtype);
  // the tuner's message: per rank for AllReduce, the whole nranks x count
  // traffic for ReduceScatter / AllGather [ch.6 §三]; an aggregate's
  // collectives share one launch and run side by side, so it is tuned on
  // their bytes together [ch.6 §四: aggregate, then select]
  const uint64_t nBytes = tuneBytes > 0 ? tuneBytes
                                        : count * (uint64_t)esz * (func == kCollAllReduce ? 1u : (uint64_t)c->nranks);
  int proto = e.forcedProto != -2 ? e.forcedProto : c->proto;
  int nch = e.nChannels > 0 ? e.nChannels : c->nChannels;
  if (nch > c->maxChannels) nch = c->maxChannels;
  // the algorithm: the tree serves AllReduce only [ch.5 §四]
  int algo = e.forcedAlgo != -2 ? e.forcedAlgo : c->algo;
  if (func != kCollAllReduce) algo = arAlgoRing;
  const unsigned algoMask = algo == arAlgoAuto ? 3u : 1u << algo;
  float predicted = 0.0f;
  arAlgo_t al = algo == arAlgoAuto ? arAlgoRing : (arAlgo_t)algo;
  if (proto == arProtoAuto) {
    unsigned mask = (unsigned)e.protoMask;
    if (!aligned128) mask &= ~(1u << arProtoLL128);
    if (mask == 0) mask = 1u << arProtoSimple;
    arProto_t p;
    int ch;
    arResult_t r = tuneCall(c, func, nBytes, c->maxChannels, algoMask, mask, &al, &p, &ch, &predicted);
    if (r != arSuccess) return r;
    proto = p;
    nch = ch < 1 ? 1 : ch;
  } else {
    if (proto == arProtoLL128 && !aligned128) return arInvalidUsage;   // LL128 needs 128-byte buffers
    // a fixed protocol and channel count; with arAlgoAuto the tuner picks the algorithm
    (void)tuneCall(c, func, nBytes, nch, algoMask, 1u << proto, &al, nullptr, nullptr, &predicted);
  }
  const bool tree = al == arAlgoTree;
  const int N = c->nranks;
  // A batched launch of rings cut into workgroups runs its tasks side by
  // side only while all their grids are resident together, so it takes at
  // most the channels (a power of two) for which every task's grid of one
  // lane per channel fits two workgroups per CU in the largest groups; with
  // more, the tasks run in rounds, each round a whole ring's chain of steps
  // (16 AllReduces of 256 KiB per rank, fp32: 24 ranks on 64 channels
  // 31.0 us per AllReduce, on 16 9.2 us; 72 ranks on 16 channels 119 us, on
  // 4 44 us).
  if (batch && nTasks > 1 && !tree && N > kMaxMembersPerGroup) {
    const int64_t groups = (N + kMaxMembersPerGroup - 1) / kMaxMembersPerGroup;
    const int64_t fit = (int64_t)c->numCUs * 2 / (groups * nTasks);
    int ch = 1;
    while ((int64_t)ch * 2 <= fit) ch *= 2;
    if (nch > ch) nch = ch;
  }
  const uint64_t A = 16 / (uint64_t)esz;
  // FIFOs per (rank, lane): one for the ring, one per incoming edge for the tree
  const int edges = tree ? kTreeEdges : 1;
  plan->algo = al;
  plan->proto = proto;
  plan->nChannels = nch;
  plan->chunkElems = chunkBytesOf(c, proto) / (uint64_t)esz;
  plan->unroll = proto == kSimple ? c->simpleUnroll : proto == kLL ? kLLUnroll
                                                    : c->ll128Unroll > 0 ? c->ll128Unroll : kLL128Unroll;
  // large LL128 slots serve single-call rings only
  if (proto == kLL128 && (tree || batch)) plan->unroll = kLL128Unroll;
  if (tree && proto == kSimple && plan->unroll > kTreeSimpleUnrollMax) plan->unroll = kTreeSimpleUnrollMax;
  if (batch && proto == kSimple && plan->unroll > kBatchSimpleUnrollMax) plan->unroll = kBatchSimpleUnrollMax;
  plan->direct = !tree && proto == kSimple && c->direct;
  plan->slotBytes = slotBytesOf(proto, plan->unroll);
  plan->slotPayload = slotPayloadOf(proto, plan->unroll);
  plan->nSlots = c->nSlots[proto];
  plan->predictedUs = predicted;

  // Members per workgroup: the whole ring when it fits (N <= 16).  Longer
  // rings are cut into balanced groups joined by device-coherent edges; the
  // launch is then cooperative, so the largest group size whose grid (one
  // lane per channel at least) is co-resident is taken, with Simple slots of
  // at most 4 KiB.
  auto layout = [&](int gs, int* nGroupsOut, int* gsOut) {
    int ng = (N + gs - 1) / gs;
    *nGroupsOut = ng;
    *gsOut = (N + ng - 1) / ng;
  };
  // elements one stage of one member covers: a chunk of the AllReduce loop,
  // or the loop's range of one rank block for ReduceScatter / AllGather; the
  // tree's lanes split the whole channel share
  const uint64_t loop = (uint64_t)N * plan->chunkElems;
  auto chunkBytesFor = [&](int ch) {
    const uint64_t per = alignUpU(divUpU(count, (uint64_t)ch), A);
    const uint64_t cur = tree ? per
                         : func != kCollAllReduce ? (per < plan->chunkElems ? per : plan->chunkElems)
                         : per < loop ? alignUpU(divUpU(per, (uint64_t)N), A) : plan->chunkElems;
    return cur * (uint64_t)esz;
  };
  uint64_t chunkBytes = chunkBytesFor(nch);

  int nGroups = 1, groupSize = N;
  auto gridFor = [&](int ln) {
    const int lt = nch * ln;
    return nGroups == 1 ? lt : ((lt + 7) / 8) * 8 * nGroups;
  };
  // About 64 wavefronts per CU: measured best on MI355X (workgroups finish
  // unevenly, so a grid of a few resident rounds balances better than one).
  // Rings whose FIFOs will sit in LDS (below) hold one or two workgroups per
  // CU at once, and twice that many lanes measured faster (8 ranks x 256 MiB
  // fp32, 4 KiB slots at depth 3: 32 lanes 0.818 ms, 64 lanes 0.778 ms).
  // A lane's share of a chunk is at least one slot.  When the chunk is too
  // small to give every lane a full Simple slot, smaller slots are used so
  // that more lanes share the work: the time of a short message is the number
  // of sequential steps per lane, not bandwidth.
  const int gsMax = batch ? kMaxMembersPerGroup : c->groupSizeMax;   // members per workgroup at most
  const bool ldsPlan = proto == kSimple && !tree && c->ldsFifo && N <= gsMax && c->ldsPerBlock > 0;
  const uint64_t wavesPerCU = ldsPlan ? 128 : 64;
  // A Simple ring cut into workgroups keeps the slots of the edges inside each
  // group in that group's LDS (the edges between groups keep device FIFOs),
  // at the comm's Simple depth; the co-residency checks below count that LDS.
  const bool ldsGrouped = proto == kSimple && !tree && !batch && c->ldsFifo && N > gsMax && c->ldsPerBlock > 0;
  auto groupLds = [&](int members) {
    const int64_t bytes = (int64_t)members * plan->nSlots * plan->slotBytes;
    plan->ldsFifo = ldsGrouped && bytes + 256 <= (int64_t)c->ldsPerBlock;
    plan->ldsBytes = plan->ldsFifo ? (int)bytes : 0;
  };
  // A single call of a ring or tree cut into workgroups puts at most 24 of
  // its wavefronts on one CU (the grid spread evenly over the CUs).  Its hops
  // are bound by instruction issue (the members of a workgroup step in
  // lockstep), and past 24 the time per hop doubles.  Rings, 2 MiB per rank
  // over 64 channels in 8 groups: 96 ranks (two 12-member workgroups per CU)
  // 345 us, 100 and 104 ranks (two of 13) 637 and 659 us, 120 ranks on 32
  // channels (one of 15) 401 us; 8 MiB per rank, 48 ranks (two of 12) 254 us,
  // 52 (two of 13) 419 us, 60 (one of 15) 335 us.  Trees, 128 KiB per rank
  // over 4 channels: 38-42 ranks (two of 13-14 on a CU) 41-43 us, 44 and 48
  // (one of 15-16) 28 and 22 us, 50-56 (two of 13-14) 42-46 us, 60 and 64
  // (one of 15-16) 27 and 24 us.  Batched launches keep their own rules, and
  // forced lanes are taken as given.
  auto wavesOverCap = [&](int64_t grid, int members) {
    const int64_t perCUUsed = grid <= c->numCUs ? 1 : (grid + c->numCUs - 1) / c->numCUs;
    return perCUUsed * members > kGroupedWavesPerCU;
  };
  auto ringWavesCapped = [&](int64_t grid, int members) { return !tree && !batch && wavesOverCap(grid, members); };
  auto targetFor = [&]() { return (int)((uint64_t)c->numCUs * wavesPerCU / ((uint64_t)N * (uint64_t)nch)); };
  auto lanesFor = [&](int slotPayload) {
    int ln = targetFor();
    // round up: a 120-byte-line LL128 slot never divides a power-of-two chunk
    const int byChunk = (int)((chunkBytes + (uint64_t)slotPayload - 1) / (uint64_t)slotPayload);
    if (ln > byChunk) ln = byChunk;
    if (ln > c->lanesMax / (edges * nch)) ln = c->lanesMax / (edges * nch);
    return ln < 1 ? 1 : ln;
  };
  auto setSlot = [&](int u) {
    plan->unroll = u;
    plan->slotBytes = slotBytesOf(proto, u);
    plan->slotPayload = slotPayloadOf(proto, u);
  };
  const int unroll0 = plan->unroll;
  const int uMax0 = proto == kSimple && unroll0 > kGroupedSimpleUnrollMax ? kGroupedSimpleUnrollMax : unroll0;

  // A grouped tree: its channels and lanes both cut the data into
  // independent column streams, each a chain of batches up and down the
  // tree, and the call takes about as long as the columns those streams keep
  // in flight allow (72 ranks x 4 MiB: 64 channels x 1 lane of 2 KiB slots in
  // 9-member groups, 1.16 ms; 16 channels x 3 lanes of 4 KiB in 15-member
  // groups, 0.60 ms).  So the channel count (at most the one asked for), the
  // slot and the group size are chosen, in a co-resident grid, for the
  // largest groups first: every tree edge between workgroups is a
  // device-coherent hop two to three times slower than one inside a
  // workgroup (72 ranks x 4 MiB: 64 channels x 1 lane of 4 KiB in 9-member
  // groups, 256 KiB in flight, 0.76 ms; 16 x 3 lanes of 4 KiB in 15-member
  // groups, 192 KiB, 0.59 ms).  Then for the most bytes in flight (channels x
  // the smaller of lanes x slot payload and a channel's share).  Ties keep the
  // smaller slot, as more lanes of it take a share that is in flight at once
  // through the tree a little faster (24 ranks x 4 KiB: 4 lanes of 1 KiB
  // 38.3 us, 2 of 2 KiB 39.1, 1 of 4 KiB 42.9), then more channels.
  // A Simple tree cut into workgroups (single calls) keeps the FIFOs of the
  // edges inside each workgroup in its LDS, two per node (up and down) at the
  // comm's Simple depth beside 512 bytes of counters, wherever they fit at
  // the slot and group size the search below picks (which counts their LDS
  // in its co-residency checks); the edges between workgroups keep device
  // FIFOs.  The search keeps its own order: preferring plans whose FIFOs fit
  // took smaller slots than the bytes in flight want (72 ranks x 1 MiB in
  // 2 KiB slots 780 us, in 4 KiB slots with device FIFOs 562 us), while at
  // the same geometry the LDS FIFOs win (72 x 4 KiB 27.5 -> 27.0 us, 32 x
  // 4 KiB 18.1 -> 15.2 us, 128 x 4 KiB 26.3 -> 23.5 us).
  const bool treeLdsOk = tree && proto == kSimple && !batch && c->ldsFifo && c->ldsPerBlock > 0;
  auto treeLds = [&](int members) {
    const int64_t bytes = (int64_t)2 * members * plan->nSlots * plan->slotBytes;
    plan->ldsFifo = treeLdsOk && bytes + 512 <= (int64_t)c->ldsPerBlock;
    plan->ldsBytes = plan->ldsFifo ? (int)bytes : 0;
  };
  bool placed = false;
  if (tree && !batch && N > gsMax && c->forcedLanes == 0) {
    const int nchAsked = nch;
    uint64_t bestBytes = 0;
    int bestU = 0, bestGs = 0, bestCh = 0, bestSize = 0;
    for (int u = uMax0; u >= 1; u /= 2) {
      setSlot(u);
      for (int ch = nchAsked; ch >= 1; ch /= 2) {
        nch = ch;
        chunkBytes = chunkBytesFor(ch);
        for (int gs = gsMax; gs >= 1; --gs) {
          layout(gs, &nGroups, &groupSize);
          plan->nGroups = nGroups;
          plan->block = groupSize * kWave;
          treeLds(groupSize);
          int pc = 0;
          if (ringKernelOccupancy(*plan, func, dtype, op, batch, &pc) != hipSuccess) return arHipError;
          const int cap = pc * c->numCUs;
          if (cap < gridFor(1) || wavesOverCap(gridFor(1), groupSize)) continue;
          int ln = lanesFor(plan->slotPayload);
          while (ln > 1 && (gridFor(ln) > cap || wavesOverCap(gridFor(ln), groupSize))) --ln;
          const uint64_t lanesBytes = (uint64_t)ln * (uint64_t)plan->slotPayload;
          const uint64_t bytes = (uint64_t)ch * (lanesBytes < chunkBytes ? lanesBytes : chunkBytes);
          if (groupSize > bestSize ||
              (groupSize == bestSize &&
               (bytes > bestBytes || (bytes == bestBytes && (u < bestU || (u == bestU && ch > bestCh)))))) {
            bestSize = groupSize;
            bestBytes = bytes;
            bestU = u;
            bestGs = gs;
            bestCh = ch;
          }
          break;   // the largest group that fits at this (slot, channels)
        }
      }
      if (proto != kSimple) break;
    }
    if (bestBytes > 0) {
      setSlot(bestU);
      nch = bestCh;
      plan->nChannels = nch;
      chunkBytes = chunkBytesFor(nch);
      layout(bestGs, &nGroups, &groupSize);
      treeLds(groupSize);
      placed = true;
    } else {
      plan->ldsFifo = false;
      plan->ldsBytes = 0;
      setSlot(unroll0);
      nch = nchAsked;
      chunkBytes = chunkBytesFor(nch);
    }
  }
  // Other grouped plans (the ring; a batched or forced-lane tree).  A Simple
  // slot smaller than the default keeps more wavefronts resident (fewer
  // registers) when the whole grid must be co-resident.  First
  // choice: the smallest slot of at least half a chunk, with enough lanes
  // that each lane's share is one slot, if such a grid can be co-resident
  // (72 ranks x 4 MiB: 912-byte chunks in 1 KiB slots and 12-member groups
  // run in 520 us, in 4 KiB slots, whose kernel fits only 9 members a group,
  // in 853 us).  Otherwise the largest slot (at most 4 KiB) whose one-lane
  // grid is co-resident.  If no grid of one lane per channel can be
  // co-resident, the channels are halved until one can (the plan reports
  // the count that runs).
  while (!placed && N > gsMax) {
    setSlot(unroll0);
    // the group size for a grid of `ln` lanes per channel with slot u whose
    // grid is co-resident (0: none; -1: HIP error): the largest one whose
    // grid is also balanced over the CUs (a multiple of their count, or at
    // most one workgroup per CU) down to half the largest co-resident size,
    // else that largest size.  Measured on MI355X (Simple, 1 KiB slots, 64
    // channels): 72 ranks x 4 MiB in groups of 12 (384 workgroups on 256 CUs)
    // 417 us, of 9 (512) 393 us; 72 x 1 MiB 386 -> 361 us; 128 ranks x 1 MiB
    // in 16 (256 workgroups) 594 us against 690 in 12 (352); 24 and 48 ranks
    // already balanced in 12.
    auto fit = [&](int u, int ln) -> int {
      if (proto == kSimple) setSlot(u);
      int first = 0;
      for (int gs = gsMax; gs >= 1; --gs) {
        layout(gs, &nGroups, &groupSize);
        if (first > 0 && 2 * groupSize < first) break;
        plan->nGroups = nGroups;
        plan->block = groupSize * kWave;
        groupLds(groupSize);
        int perCU = 0;
        if (ringKernelOccupancy(*plan, func, dtype, op, batch, &perCU) != hipSuccess) return -1;
        const int64_t grid = (int64_t)((nch * ln + 7) / 8) * 8 * nGroups;
        if ((int64_t)perCU * c->numCUs < grid) continue;
        if (ringWavesCapped(grid, groupSize)) continue;
        if (grid <= c->numCUs || grid % c->numCUs == 0) return 1;
        if (first == 0) first = groupSize;
      }
      if (first == 0) return 0;
      layout(first, &nGroups, &groupSize);
      plan->nGroups = nGroups;
      plan->block = groupSize * kWave;
      groupLds(groupSize);
      return 1;
    };
    const int uMax = uMax0;
    int found = 0;
    if (proto == kSimple) {
      int u = uMax;
      while (u > 1 && 2 * (uint64_t)slotPayloadOf(proto, u / 2) >= chunkBytes) u /= 2;
      const uint64_t need = (chunkBytes + (uint64_t)slotPayloadOf(proto, u) - 1) / (uint64_t)slotPayloadOf(proto, u);
      if (u < uMax && need >= 1 && need <= 2) found = fit(u, (int)need);
    }
    // One lane per channel: every Simple slot is tried.  The plan whose edges
    // inside a workgroup keep their FIFOs in LDS is taken first, then the
    // largest groups, then the smallest slot that holds a whole chunk (else
    // the largest slot).  Taking the largest slot that fits at all put 76
    // ranks x 8 MiB (1.8 KiB chunks) in one-member groups of 4 KiB slots,
    // every hop between workgroups (1390 us; in 10-member groups of 2 KiB
    // slots 365 us), and 72 ranks x 8 MiB in 9-member groups of 4 KiB slots
    // (654 us), a step of the 4 KiB kernel moving the same 1.8 KiB as one of
    // the 2 KiB kernel.
    if (found == 0) {
      int bestU = 0, bestSize = 0;
      bool bestLds = false;
      auto covers = [&](int u) { return (uint64_t)slotPayloadOf(proto, u) >= chunkBytes; };
      for (int u = uMax; u >= 1; u /= 2) {
        const int f = fit(u, 1);
        if (f < 0) return arHipError;
        const bool lds = plan->ldsFifo && groupSize > 1;
        const bool better = bestU == 0 || (lds && !bestLds) ||
                            (lds == bestLds && (groupSize > bestSize ||
                                                (groupSize == bestSize && covers(u) && covers(bestU))));
        if (f > 0 && better) {
          bestU = u;
          bestSize = groupSize;
          bestLds = lds;
        }
        if (proto != kSimple) break;
      }
      if (bestU > 0) found = fit(bestU, 1);
    }
    if (found < 0) return arHipError;
    if (found > 0) break;
    if (nch == 1) return arInvalidUsage;
    nch /= 2;
    plan->nChannels = nch;
    chunkBytes = chunkBytesFor(nch);
  }
  plan->groupSize = groupSize;
  plan->nGroups = nGroups;
  plan->block = groupSize * kWave;
  plan->cooperative = nGroups > 1;   // the whole grid must be co-resident
  plan->launchCoop = plan->cooperative && !c->plainLaunch;

  // Lanes per (rank, channel): one resident round of workgroups (the grid is
  // sized to what the chip holds at once, so no tail round), but never a
  // lane share below two FIFO slots of the largest chunk.
  int perCU = 0;
  if (ringKernelOccupancy(*plan, func, dtype, op, batch, &perCU) != hipSuccess) return arHipError;
  if (perCU < 1) perCU = 1;
  const int capacity = perCU * c->numCUs;   // resident workgroups
  const int target = targetFor();
  int lanes = lanesFor(plan->slotPayload);
  // LL128, automatic slot: the large slot when every lane still gets a full
  // batch of large slots (nSlots/2 columns): that halves the batches, each of
  // which fills and drains the ring (16 ranks x 512 MiB bf16: 13.3 -> 10.5 ms).
  // With fewer columns the batch only gets shallower (8 ranks x 128 MiB fp32:
  // 1.49 -> 1.65 ms), so short shares keep the small slot.
  if (proto == kLL128 && c->ll128Unroll == 0 && !tree && !batch && !plan->cooperative && c->forcedLanes == 0) {
    const int pay = slotPayloadOf(proto, kLL128UnrollLarge);
    const int ln = lanesFor(pay);
    if (chunkBytes / (uint64_t)ln >= (uint64_t)(plan->nSlots / 2) * (uint64_t)pay) {
      plan->unroll = kLL128UnrollLarge;
      plan->slotBytes = slotBytesOf(proto, kLL128UnrollLarge);
      plan->slotPayload = pay;
      lanes = ln;
    }
  }
  if (proto == kSimple && !plan->cooperative && c->forcedLanes == 0) {
    // Smaller slots spread a short chunk over more lanes, but only while the
    // grid stays within one workgroup per CU, or 8 wavefronts per CU where a
    // workgroup holds fewer than 8 members: past that, each lane is a
    // chain of 2N-1 one-column steps and more of such chains side by side
    // cost more than bigger slots (8 ranks, 16 MiB per rank: 4 lanes of
    // 8 KiB take 112 us, 8 of 4 KiB 130 us, 32 lanes of 1 KiB in four rounds
    // 165 us; 16 ranks, 4 MiB: 4 lanes of 1 KiB take 88 us, 2 of 2 KiB
    // 102 us).  Below 8 members one workgroup per CU leaves the CUs nearly
    // idle (2 ranks x 4 MiB: 4 lanes of 8 KiB take 12.0 us, 16 of 2 KiB
    // 8.0 us; 4 ranks x 8 MiB: 34.1 -> 25.7 us).  A halving that keeps the
    // lane count is taken too while the lane share still fits one slot of the
    // smaller size, whose kernel is faster on it (a 4 KiB share: 1 lane at
    // 8, 4 and 2 KiB slots, 2 at 1 KiB); not where the FIFOs cap the lanes
    // and the share spans several slots (8 ranks x 8 MiB tree: 21 lanes of
    // 2 KiB slots 104 us, of 4 KiB 69 us).
    const int members = nGroups == 1 ? N : groupSize;
    const int maxGrid = c->numCUs * (members < 8 ? 8 / members : 1);
    while (lanes < target && plan->unroll > 1 && (uint64_t)lanes * plan->slotPayload >= chunkBytes / 2) {
      const int u = plan->unroll / 2;
      const int ln = lanesFor(slotPayloadOf(proto, u));
      if (ln < lanes || (ln > lanes && gridFor(ln) > maxGrid)) break;
      if (ln == lanes && (uint64_t)ln * slotPayloadOf(proto, u) < chunkBytes) break;
      plan->unroll = u;
      plan->slotBytes = slotBytesOf(proto, u);
      plan->slotPayload = slotPayloadOf(proto, u);
      lanes = ln;
    }
  }
  if (c->forcedLanes > 0) {
    const int cap = c->lanesMax / (edges * nch);
    lanes = c->forcedLanes <= cap ? c->forcedLanes : cap;
  }
  if (plan->cooperative) {
    while (lanes > 1 && (gridFor(lanes) > capacity ||
                         (!batch && c->forcedLanes == 0 && wavesOverCap(gridFor(lanes), groupSize))))
      --lanes;
    if (gridFor(lanes) > capacity) return arInvalidUsage;
  }
  // a batched launch runs up to nTasks collectives at once, each on its own
  // nch x lanes wavefront sets: as many as the FIFOs (and, cooperative, the
  // resident grid) allow
  int slots = 1;
  if (batch) {
    slots = nTasks;
    const int byFifo = c->lanesMax / (edges * nch * lanes);
    if (slots > byFifo) slots = byFifo;
    if (plan->cooperative)
      while (slots > 1 && gridFor(lanes * slots) > capacity) --slots;
    if (slots < 1) slots = 1;
  }
  plan->taskSlots = slots;
  plan->lanes = lanes;
  plan->grid = gridFor(lanes * slots);
  plan->laneSets = nch * lanes;
  if (!batch && nGroups == 1 && c->laneSetsMax > 0 && c->laneSetsMax < plan->laneSets) {
    plan->laneSets = c->laneSetsMax;
    plan->grid = plan->laneSets;
  }
  // Single-workgroup LL128 rings compile each step for its kind only when the
  // grid is one workgroup per CU at most: there the steps' chain is the
  // time; the per-kind kernel's extra registers cost a grid of several
  // resident rounds more than they save.
  plan->perKind = proto == kLL128 && nGroups == 1 && !batch && plan->grid <= c->numCUs;
  // A Simple ring inside one workgroup (single calls and batched launches,
  // whose tasks then continue on the workgroup's LDS FIFOs) keeps its slots in
  // LDS: every handoff is then LDS to LDS, and the kernel reads each input
  // and writes each output once, nothing more.  The counters of such edges
  // are in LDS already; the static ones take 256 bytes.  The FIFOs get the
  // comm's LDS depth (3) at the largest slot, at most the planned one and
  // 4 KiB, whose N x depth slots fit a workgroup's LDS (8 ranks: 4 KiB, 96
  // KiB of LDS; 16 ranks: 2 KiB): measured on MI355X, depth 3 at 4 KiB beats
  // depth 2 at 8 KiB by 3% at 8 ranks x 256 MiB fp32 and ties at 16 ranks x
  // 512 MiB bf16, and 8 KiB gains nothing where it fits (4 ranks x 8 MiB);
  // the lane count stays, so a lane's share spans more, smaller slots.
  if (treeLdsOk && placed && nGroups > 1) {
    treeLds(groupSize);   // as the co-residency checks above counted it
    // Deeper FIFOs, as for the ring below, where the FIFOs stay where they
    // are (in LDS if they fit there at depth 2, else in device memory) and
    // the grid stays co-resident: the tree moves a batch of nSlots columns
    // up and down at a time, so a deeper FIFO keeps more bytes in flight
    // (72 ranks x 4 MiB, 16 channels x 3 lanes of 4 KiB in 15-member groups:
    // depth 2 562 us, 4 448 us; 68 x 2 MiB 0.76x; 24 x 4 KiB 0.94x; 32 x
    // 256 KiB at depth 4 would leave LDS for device FIFOs, 1.28x, so keeps
    // depth 2).
    if (!c->slotsForced) {
      const int d0 = plan->nSlots;
      const bool lds0 = plan->ldsFifo;
      for (int d = kGroupedSlotsMax; d > d0; --d) {
        plan->nSlots = d;
        treeLds(groupSize);
        if (plan->ldsFifo == lds0) {
          int pc = 0;
          if (ringKernelOccupancy(*plan, func, dtype, op, batch, &pc) != hipSuccess) return arHipError;
          if ((int64_t)pc * c->numCUs >= (int64_t)plan->grid) break;
        }
        plan->nSlots = d0;
        treeLds(groupSize);
      }
    }
    return arSuccess;
  }
  if (ldsGrouped && nGroups > 1) {
    groupLds(groupSize);   // as the co-residency check above counted it
    if (plan->ldsFifo) plan->direct = false;
    // Deeper FIFOs at the chosen slot and grid, where they still fit the
    // workgroup's LDS and keep the grid co-resident: the members of a ring
    // cut into workgroups step in lockstep, and a deeper FIFO lets each run
    // further ahead of its successor, which absorbs the jitter of the hops
    // (72 ranks x 4 MiB in 9-member groups of 1 KiB slots: depth 2 281 us,
    // 3 258 us, 4 252 us; 48 x 4 MiB at depth 3 0.93x, 24 x 4 MiB 0.94x).
    // The edges between workgroups get the same depth; their device FIFOs
    // are provisioned for it on the first such call.
    if (plan->ldsFifo && !c->slotsForced) {
      const int d0 = plan->nSlots;
      for (int d = kGroupedSlotsMax; d > d0; --d) {
        plan->nSlots = d;
        groupLds(groupSize);
        int pc = 0;
        if (ringKernelOccupancy(*plan, func, dtype, op, batch, &pc) != hipSuccess) return arHipError;
        if (plan->ldsFifo && (int64_t)pc * c->numCUs >= (int64_t)plan->grid) break;
        plan->nSlots = d0;
        groupLds(groupSize);
      }
    }
    return arSuccess;
  }
  plan->ldsFifo = false;
  plan->ldsBytes = 0;
  if (ldsPlan && nGroups == 1) {
    const int d = c->ldsSlots;
    int u = plan->unroll < kGroupedSimpleUnrollMax ? plan->unroll : kGroupedSimpleUnrollMax;
    while (u > 1 && (int64_t)N * d * slotBytesOf(kSimple, u) + 256 > (int64_t)c->ldsPerBlock) u /= 2;
    const int64_t bytes = (int64_t)N * d * slotBytesOf(kSimple, u);
    if (bytes + 256 <= (int64_t)c->ldsPerBlock) {
      setSlot(u);
      plan->ldsFifo = true;
      plan->ldsBytes = (int)bytes;
      plan->nSlots = d;
      plan->direct = false;
    }
  }
  // A Simple tree inside one workgroup keeps its FIFOs in LDS too: one up and
  // one down per node (2N), at the comm's depth, with the largest slot (at
  // most the planned one) that fits beside the tree's 512 bytes of counters.
  if (tree && proto == kSimple && nGroups == 1 && c->ldsFifo && c->ldsPerBlock > 0 && N <= gsMax) {
    const int d = plan->nSlots;
    int u = plan->unroll;
    while (u > 1 && (int64_t)2 * N * d * slotBytesOf(kSimple, u) + 512 > (int64_t)c->ldsPerBlock) u /= 2;
    const int64_t bytes = (int64_t)2 * N * d * slotBytesOf(kSimple, u);
    if (bytes + 512 <= (int64_t)c->ldsPerBlock) {
      setSlot(u);
      plan->ldsFifo = true;
      plan->ldsBytes = (int)bytes;
    }
  }
  return arSuccess;
}

}  // namespace

extern "C" {

const char* arGetErrorString(arResult_t r) {
  switch (r) {
    case arSuccess: return "no error";
    case arHipError: return "HIP runtime error (or no usable GPU)";
    case arSystemError: return "system error (host allocation or OS call failed)";
    case arInternalError: return "internal error";
    case arInvalidArgument: return "invalid argument";
    case arInvalidUsage: return "invalid usage";
    case arRemoteError: return "remote error: a ring member timed out or the comm was aborted";
    case arInProgress: return "operation in progress";
    default: return "unknown result code";
  }
}

arResult_t arInit(arComm_t* out, int nranks, int nChannels, arProto_t proto, arAlgo_t algo) {
  ApiRange range("arInit");
  if (out == nullptr) return arInvalidArgument;
  *out = nullptr;
  if (nranks < 1 || nranks > AR_MAX_RANKS) return arInvalidArgument;
  if (nChannels < 1 || nChannels > AR_MAX_CHANNELS) return arInvalidArgument;
  if (proto != arProtoAuto && proto != arProtoLL && proto != arProtoLL128 && proto != arProtoSimple)
    return arInvalidArgument;
  if (algo != arAlgoRing && algo != arAlgoTree && algo != arAlgoAuto) return arInvalidArgument;
  const Env& e = env();

  int dev = 0, ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return arHipError;
  if (hipGetDevice(&dev) != hipSuccess) return arHipError;
  int cus = 0, clk = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return arHipError;
  if (hipDeviceGetAttribute(&clk, hipDeviceAttributeWallClockRate, dev) != hipSuccess || clk <= 0) clk = 100000;

  arComm* c = new (std::nothrow) arComm();
  if (c == nullptr) return arSystemError;
  c->startMagic = c->endMagic = kCommMagic;
  c->nranks = nranks;
  c->maxChannels = nChannels;
  c->proto = proto;
  c->algo = algo;
  c->nChannels = nChannels;
  c->device = dev;
  c->numCUs = cus;
  c->wallClockKHz = clk;
  for (int p = 0; p < 3; ++p) c->nSlots[p] = e.nSteps > 0 ? e.nSteps : kDefaultSlots[p];
  c->sliceBytes = e.sliceBytes;
  c->timeoutUs = e.timeoutUs;
  c->deadRank = -1;
  c->simpleUnroll = kSimpleUnrollDefault;
  c->ll128Unroll = 0;   // automatic
  c->direct = true;
  c->groupSizeMax = kMaxMembersPerGroup;
  c->ldsFifo = true;
  c->ldsSlots = e.nSteps > 0 ? e.nSteps : kLdsFifoSlots;
  c->slotsForced = e.nSteps > 0;
  if (hipDeviceGetAttribute(&c->ldsPerBlock, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    c->ldsPerBlock = 0;
  // Grouped plans are launched plainly: the planner sizes their grid to what
  // the GPU holds at once, and the cooperative launch call cost 15-20 us per
  // launch, 60-70 us more on some streams (the runtime routes it through a
  // queue of its own), for the same residency on an otherwise idle GPU.
  c->plainLaunch = true;
  tuneTableModels(c->models, c->treeModels);

  // FIFOs and counters: every protocol the comm may run (all three when it
  // tunes per call), each at the depth it runs with; a protocol switched to
  // later is provisioned by arSetConfig or its first call.
  c->lanesMax = kMaxWorkers / nranks > nChannels ? kMaxWorkers / nranks : nChannels;
  for (int p = 0; p < 3; ++p) {
    const bool used = proto == arProtoAuto || proto == p || e.forcedProto == p;
    if (used && provisionFifo(c, p, c->nSlots[p]) != arSuccess) {
      freeComm(c);
      return arHipError;
    }
  }
  if (hipHostMalloc((void**)&c->ctrlHost, sizeof(Control), hipHostMallocCoherent | hipHostMallocMapped) !=
      hipSuccess) {
    freeComm(c);
    return arHipError;
  }
  memset(c->ctrlHost, 0, sizeof(Control));
  if (hipHostGetDevicePointer((void**)&c->ctrlDev, c->ctrlHost, 0) != hipSuccess ||
      hipMalloc((void**)&c->failedDev, 256) != hipSuccess || hipMemset(c->failedDev, 0, 256) != hipSuccess ||
      hipEventCreateWithFlags(&c->stagingDone[0], hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->stagingDone[1], hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->stagingDone[2], hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->stagingDone[3], hipEventDisableTiming) != hipSuccess) {
    freeComm(c);
    return arHipError;
  }
  if (hipDeviceSynchronize() != hipSuccess) {
    freeComm(c);
    return arHipError;
  }
  if (e.debug >= 1)
    fprintf(stderr, "[ar] INFO init nranks=%d maxChannels=%d proto=%d CUs=%d slots=%d slice=%zu\n", nranks,
            nChannels, (int)proto, cus, c->nSlots[kSimple], c->sliceBytes);
  *out = c;
  return arSuccess;
}

arResult_t arSetConfig(arComm_t c, arProto_t proto, int nChannels) {
  if (!commOk(c)) return arInvalidArgument;
  if (proto != arProtoAuto && proto != arProtoLL && proto != arProtoLL128 && proto != arProtoSimple)
    return arInvalidArgument;
  if (nChannels < 1 || nChannels > c->maxChannels) return arInvalidArgument;
  if (c->inGroup) return arInvalidUsage;   // queued calls may still plan with the old setting
  c->proto = proto;
  c->nChannels = nChannels;
  for (int p = 0; p < 3; ++p)   // the FIFOs of every protocol it may now run
    if ((proto == arProtoAuto || proto == p) && provisionFifo(c, p, c->nSlots[p]) != arSuccess) return arHipError;
  return arSuccess;
}

arResult_t arSetDebug(arComm_t c, arDebugKnob_t knob, int64_t value) {
  if (!commOk(c)) return arInvalidArgument;
  if (knob == arDebugTimeoutUs) {
    if (value <= 0) return arInvalidArgument;
    c->timeoutUs = value;
    return arSuccess;
  }
  if (knob == arDebugDeadRank) {
    if (value < -1 || value >= c->nranks) return arInvalidArgument;
    c->deadRank = (int)value;
    return arSuccess;
  }
  if (knob == arDebugLanes) {
    if (value < 0 || value > c->lanesMax) return arInvalidArgument;
    c->forcedLanes = (int)value;
    return arSuccess;
  }
  if (knob == arDebugSimpleSlotKiB) {
    if (value != 1 && value != 2 && value != 4 && value != 8) return arInvalidArgument;
    c->simpleUnroll = (int)value;
    return arSuccess;
  }
  if (knob == arDebugGroupSpread) {
    if (value != 0 && value != 1) return arInvalidArgument;
    c->groupSpread = (int)value;
    return arSuccess;
  }
  if (knob == arDebugLL128SlotKiB) {
    if (value != 0 && value != kLL128Unroll && value != kLL128UnrollLarge) return arInvalidArgument;
    c->ll128Unroll = (int)value;
    return arSuccess;
  }
  if (knob == arDebugSlots) {
    if (value < 2 || value > kMaxSlots) return arInvalidArgument;
    if (c->inGroup) return arInvalidUsage;
    for (int p = 0; p < 3; ++p) {
      c->nSlots[p] = (int)value;
      if (c->fifo[p] != nullptr && provisionFifo(c, p, c->nSlots[p]) != arSuccess) return arHipError;
    }
    c->ldsSlots = (int)value;
    c->slotsForced = true;
    return arSuccess;
  }
  if (knob == arDebugLaneSets) {
    if (value < 0 || value > c->lanesMax) return arInvalidArgument;
    c->laneSetsMax = (int)value;
    return arSuccess;
  }
  if (knob == arDebugLLChunkBytes || knob == arDebugLL128ChunkBytes) {
    if (value < 0 || value > ((int64_t)64 << 20) || value % 16 != 0) return arInvalidArgument;
    (knob == arDebugLLChunkBytes ? c->llChunkBytes : c->ll128ChunkBytes) = (size_t)value;
    return arSuccess;
  }
  if (knob == arDebugCooperative) {
    if (value != 0 && value != 1) return arInvalidArgument;
    c->plainLaunch = value == 0;
    return arSuccess;
  }
  if (knob == arDebugLdsFifo) {
    if (value != 0 && value != 1) return arInvalidArgument;
    c->ldsFifo = value != 0;
    return arSuccess;
  }
  if (knob == arDebugGroupSize) {
    if (value < 0 || value > kMaxMembersPerGroup) return arInvalidArgument;
    c->groupSizeMax = value == 0 ? kMaxMembersPerGroup : (int)value;
    return arSuccess;
  }
  if (knob == arDebugDirect) {
    if (value != 0 && value != 1) return arInvalidArgument;
    c->direct = value != 0;
    return arSuccess;
  }
  return arInvalidArgument;
}

arResult_t arTuneGetAlgoModel(arComm_t c, arAlgo_t algo, arProto_t proto, arTuneModel_t* model) {
  if (!commOk(c) || model == nullptr || proto < arProtoLL || proto > arProtoSimple) return arInvalidArgument;
  if (algo != arAlgoRing && algo != arAlgoTree) return arInvalidArgument;
  *model = algo == arAlgoRing ? c->models[proto] : c->treeModels[proto];
  return arSuccess;
}

arResult_t arTuneSetAlgoModel(arComm_t c, arAlgo_t algo, arProto_t proto, const arTuneModel_t* model) {
  if (!commOk(c) || model == nullptr || proto < arProtoLL || proto > arProtoSimple) return arInvalidArgument;
  if (algo != arAlgoRing && algo != arAlgoTree) return arInvalidArgument;
  if (!(model->bwPerChGBs > 0.0f) || !(model->maxBwGBs > 0.0f) || model->baseLatUs < 0.0f ||
      model->stepLatUs < 0.0f)
    return arInvalidArgument;
  (algo == arAlgoRing ? c->models : c->treeModels)[proto] = *model;
  return arSuccess;
}

arResult_t arTuneGetModel(arComm_t c, arProto_t proto, arTuneModel_t* model) {
  return arTuneGetAlgoModel(c, arAlgoRing, proto, model);
}

arResult_t arTuneSetModel(arComm_t c, arProto_t proto, const arTuneModel_t* model) {
  return arTuneSetAlgoModel(c, arAlgoRing, proto, model);
}

arResult_t arTuneAlgo(arComm_t c, size_t nBytes, arAlgo_t* algo, arProto_t* proto, int* nChannels,
                      float* predictedUs) {
  if (!commOk(c)) return arInvalidArgument;
  const int a = env().forcedAlgo != -2 ? env().forcedAlgo : c->algo;
  const unsigned algoMask = a == arAlgoAuto ? 3u : 1u << a;
  return tuneCall(c, arFuncAllReduce, nBytes, c->maxChannels, algoMask, (unsigned)env().protoMask, algo, proto,
                  nChannels, predictedUs);
}

arResult_t arTune(arComm_t c, size_t nBytes, arProto_t* proto, int* nChannels, float* predictedUs) {
  return arTuneAlgo(c, nBytes, nullptr, proto, nChannels, predictedUs);
}

arResult_t arSetAlgo(arComm_t c, arAlgo_t algo) {
  if (!commOk(c)) return arInvalidArgument;
  if (algo != arAlgoRing && algo != arAlgoTree && algo != arAlgoAuto) return arInvalidArgument;
  c->algo = algo;
  return arSuccess;
}

arResult_t arGetPlanColl(arComm_t c, arFunc_t func, size_t count, arDataType_t dtype, int aligned128,
                         arPlan_t* out) {
  if (!commOk(c) || out == nullptr || elemSize(dtype) == 0) return arInvalidArgument;
  if (func != arFuncAllReduce && func != arFuncReduceScatter && func != arFuncAllGather) return arInvalidArgument;
  const int op = dtype == arUint64 ? arProbe : arSum;
  if (c->nranks == 1 || count == 0) {
    exportPlan(c, func, count, dtype, nullptr, out);
    return arSuccess;
  }
  Plan p;
  arResult_t r = makePlan(c, func, count, dtype, op, aligned128 != 0, &p);
  if (r != arSuccess) return r;
  exportPlan(c, func, count, dtype, &p, out);
  return arSuccess;
}

arResult_t arGetPlan(arComm_t c, size_t count, arDataType_t dtype, int aligned128, arPlan_t* out) {
  return arGetPlanColl(c, arFuncAllReduce, count, dtype, aligned128, out);
}

}  // extern "C"

namespace {

// Group state of the calling thread [ch.7 §一: the group depth, the first
// error and the communicators with queued work are thread-local].
thread_local int tGroupDepth = 0;
thread_local arResult_t tGroupError = arSuccess;
thread_local std::vector<arComm*> tGroupComms;

// A member of an earlier call timed out or saw the abort word: its edges were
// left mid-call, so the comm accepts no more work (the kernels of calls
// already queued check the device copy of this word and do nothing).
bool memberGaveUp(arComm* c) {
  if (__atomic_load_n(&c->ctrlHost->status, __ATOMIC_ACQUIRE) == 0) return false;
  c->aborted = true;
  return true;
}

// Every (channel, lane, rank, edge) FIFO the kernel indexes must exist.
bool fifosCover(const arComm* c, const Plan& plan) {
  const int edges = plan.algo == arAlgoTree ? kTreeEdges : 1;
  return (size_t)plan.nChannels * (size_t)plan.lanes * (size_t)edges * (size_t)plan.taskSlots <=
         (size_t)c->lanesMax;
}

// Kernel arguments of one call (batched launches add the task table).
void buildArgs(const arComm* c, const Plan& plan, int func, size_t count, const void* const* sendbufs,
               void* const* recvbufs, bool aligned16, KernelArgs* a) {
  const int N = c->nranks;
  memset(a, 0, sizeof(*a));
  for (int i = 0; i < N; ++i) {
    a->send[i] = sendbufs[i];
    a->recv[i] = recvbufs[i];
  }
  a->fifo = c->fifo[plan.proto];
  a->conn = c->conn[plan.proto];
  a->ctrl = c->ctrlDev;
  a->failed = c->failedDev;
  a->count = count;
  a->chunkElems = plan.chunkElems;
  a->fifoWorkerBytes = c->fifoWorkerBytes[plan.proto];
  a->timeoutTicks = (uint64_t)c->timeoutUs * (uint64_t)c->wallClockKHz / 1000u;
  a->nranks = N;
  a->nChannels = plan.nChannels;
  a->lanes = plan.lanes;
  a->groupSize = plan.groupSize;
  a->nGroups = plan.nGroups;
  a->nSlots = plan.nSlots;
  a->aligned16 = aligned16 ? 1 : 0;
  a->direct = plan.direct ? 1 : 0;
  a->coll = func;
  a->deadRank = c->deadRank;
  a->taskSlots = 1;
  a->laneSets = plan.laneSets;
  a->groupSpread = c->groupSpread;
}

}  // namespace

// Argument checks of one collective call [ch.6 §二, ArgsCheck]: element type
// and op, buffer pointers (set, element-aligned), and no output overlapping
// another rank's buffers or its own input except exactly in place.  `count`
// is per rank for AllReduce and per rank block for the other two; count == 0
// passes with nothing checked (the empty call does no work).  Also reports
// whether every buffer (and rank block) is 16- and 128-byte aligned.
arResult_t ar::checkCollArgs(int N, int func, const void* const* sendbufs, void* const* recvbufs, size_t count,
                             int dtype, int op, bool* aligned16Out, bool* aligned128Out) {
  const int esz = elemSize(dtype);
  if (esz == 0) return arInvalidArgument;
  if (op != arSum && op != arMax && op != arMin && op != arProbe) return arInvalidArgument;
  if ((op == arProbe) != (dtype == arUint64) && func != kCollAllGather) return arInvalidArgument;
  if (count == 0) return arSuccess;   // empty collective: no work [ch.6 §三]
  if (sendbufs == nullptr || recvbufs == nullptr) return arInvalidArgument;
  if (count > (uint64_t)1 << 40) return arInvalidArgument;
  const size_t block = count * (size_t)esz;
  const size_t sendBytes = func == kCollReduceScatter ? block * (size_t)N : block;
  const size_t recvBytes = func == kCollAllGather ? block * (size_t)N : block;
  bool aligned16 = true, aligned128 = true;
  for (int r = 0; r < N; ++r) {
    const uintptr_t s = (uintptr_t)sendbufs[r], d = (uintptr_t)recvbufs[r];
    if (s == 0 || d == 0) return arInvalidArgument;
    if (s % (uintptr_t)esz != 0 || d % (uintptr_t)esz != 0) return arInvalidArgument;
    aligned16 = aligned16 && s % 16 == 0 && d % 16 == 0;
    aligned128 = aligned128 && s % 128 == 0 && d % 128 == 0;
  }
  if (func != kCollAllReduce) {   // rank blocks start inside the buffers
    aligned16 = aligned16 && block % 16 == 0;
    aligned128 = aligned128 && block % 128 == 0;
  }
  // Outputs must not overlap each other or another rank's input.  Against its
  // own input an output is either disjoint or exactly in place: the same
  // buffer (AllReduce), block r of the input (ReduceScatter), or the input as
  // block r of the output (AllGather).
  for (int i = 0; i < N; ++i) {
    const uintptr_t di = (uintptr_t)recvbufs[i], si = (uintptr_t)sendbufs[i];
    const bool inPlace = func == kCollAllReduce ? di == si
                         : func == kCollReduceScatter ? di == si + (uintptr_t)i * block
                                                      : si == di + (uintptr_t)i * block;
    if (!inPlace && di < si + sendBytes && si < di + recvBytes) return arInvalidArgument;
    for (int j = 0; j < N; ++j) {
      if (j == i) continue;
      const uintptr_t dj = (uintptr_t)recvbufs[j], sj = (uintptr_t)sendbufs[j];
      if (di < dj + recvBytes && dj < di + recvBytes) return arInvalidArgument;
      if (di < sj + sendBytes && sj < di + recvBytes) return arInvalidArgument;
    }
  }
  *aligned16Out = aligned16;
  *aligned128Out = aligned128;
  return arSuccess;
}

namespace {

// One collective call: argument checks (nothing is enqueued on failure), the
// empty and one-rank short cuts, planning, kernel arguments, one launch.
// `count` is per rank for AllReduce and per rank block for the other two.
arResult_t runColl(arComm* c, int func, const void* const* sendbufs, void* const* recvbufs, size_t count,
                   arDataType_t dtype, arRedOp_t op, void* stream) {
  if (!commOk(c)) return arInvalidArgument;
  if (c->aborted) return arInvalidUsage;
  if (memberGaveUp(c)) return arRemoteError;
  const int N = c->nranks;
  bool aligned16 = true, aligned128 = true;
  const arResult_t chk = checkCollArgs(N, func, sendbufs, recvbufs, count, dtype, op, &aligned16, &aligned128);
  if (chk != arSuccess) return chk;
  if (count == 0) return arSuccess;   // empty collective: no work [ch.6 §三]
  const size_t block = count * (size_t)elemSize(dtype);
  hipStream_t st = (hipStream_t)stream;
  if (tGroupDepth > 0) {   // queued until the outermost arGroupEnd [ch.7 §一]
    if (!c->pending.empty() && c->pending[0].stream != st) return arInvalidUsage;
    GroupTask t;
    t.func = func;
    t.count = count;
    t.dtype = dtype;
    t.op = op;
    t.stream = st;
    t.aligned16 = aligned16;
    t.aligned128 = aligned128;
    t.send.assign(sendbufs, sendbufs + N);
    t.recv.assign(recvbufs, recvbufs + N);
    c->pending.push_back(std::move(t));
    if (!c->inGroup) {
      c->inGroup = true;
      tGroupComms.push_back(c);
    }
    return arSuccess;
  }
  c->opCount++;

  if (N == 1) {   // one rank: the result is the input [ch.6 §三, one-rank path]
    c->lastStream = st;
    c->launched = true;
    if (recvbufs[0] == sendbufs[0]) return arSuccess;
    return hipMemcpyAsync(recvbufs[0], sendbufs[0], block, hipMemcpyDeviceToDevice, st) == hipSuccess
               ? arSuccess
               : arHipError;
  }

  Plan plan;
  const int kop = func == kCollAllGather ? (dtype == arUint64 ? arProbe : arSum) : op;
  arResult_t r = makePlan(c, func, count, dtype, kop, aligned128, &plan);
  if (r != arSuccess) return r;
  if (!fifosCover(c, plan)) return arInternalError;
  // FIFOs in LDS need no device memory, but the edges between the
  // workgroups of a ring or tree cut into groups keep theirs in it
  if (!plan.ldsFifo || plan.nGroups > 1) {
    r = provisionFifo(c, plan.proto, plan.nSlots);   // a protocol this comm has not run yet
    if (r != arSuccess) return r;
  }

  KernelArgs a;
  buildArgs(c, plan, func, count, sendbufs, recvbufs, aligned16, &a);

  if (env().debug >= 1)
    fprintf(stderr,
            "[ar] INFO op %llu func=%d count=%zu dtype=%d op=%d algo=%d proto=%d nch=%d chunk=%llu lanes=%d "
            "groups=%dx%d grid=%d block=%d coop=%d unroll=%d direct=%d pred=%.1fus\n",
            (unsigned long long)c->opCount, func, count, (int)dtype, (int)op, plan.algo, plan.proto, plan.nChannels,
            (unsigned long long)plan.chunkElems, plan.lanes, plan.nGroups, plan.groupSize, plan.grid, plan.block,
            (int)plan.cooperative, plan.unroll, (int)plan.direct, plan.predictedUs);
  hipError_t he = launchRing(plan, dtype, kop, a, st);
  if (he != hipSuccess) {
    fprintf(stderr, "[ar] WARN kernel launch failed: %s\n", hipGetErrorString(he));
    return arHipError;
  }
  c->lastStream = st;
  c->launched = true;
  return arSuccess;
}


// Compute units, wall-clock rate and LDS per workgroup of a device, read
// once per device.
void deviceInfo(int dev, int* cus, int* clkKHz, int* ldsPerBlock) {
  static std::mutex mu;
  static int known[64][3];
  static bool have[64];
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < 64 && have[dev]) {
    *cus = known[dev][0];
    *clkKHz = known[dev][1];
    *ldsPerBlock = known[dev][2];
    return;
  }
  int c = 0, k = 0, l = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 0;
  if (hipDeviceGetAttribute(&k, hipDeviceAttributeWallClockRate, dev) != hipSuccess || k <= 0) k = 100000;
  if (hipDeviceGetAttribute(&l, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) l = 0;
  if (dev >= 0 && dev < 64 && c > 0) {
    known[dev][0] = c;
    known[dev][1] = k;
    known[dev][2] = l;
    have[dev] = true;
  }
  *cus = c;
  *clkKHz = k;
  *ldsPerBlock = l;
}

}  // namespace

arResult_t ar::allReduceInScratch(char* scratch, size_t scratchBytes, const void* const* sendbufs,
                                  void* const* recvbufs, int nranks, int nChannels, size_t count, int dtype, int op,
                                  hipStream_t stream) {
  if (nranks < 1 || nranks > kMaxMembersPerGroup) return arInvalidArgument;   // one workgroup per ring
  if (nChannels < 1 || nChannels > AR_MAX_CHANNELS) return arInvalidArgument;
  bool aligned16 = true, aligned128 = true;
  const arResult_t chk =
      checkCollArgs(nranks, kCollAllReduce, sendbufs, recvbufs, count, dtype, op, &aligned16, &aligned128);
  if (chk != arSuccess || count == 0) return chk;
  if (nranks == 1) {   // the result is the input [ch.6 §三, one-rank path]
    if (recvbufs[0] == sendbufs[0]) return arSuccess;
    return hipMemcpyAsync(recvbufs[0], sendbufs[0], count * (size_t)elemSize(dtype), hipMemcpyDeviceToDevice,
                          stream) == hipSuccess
               ? arSuccess
               : arHipError;
  }
  const Env& e = env();
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return arHipError;
  // A comm description on the stack, for the planner: the same defaults as
  // arInit with a Simple ring of nChannels, and as many lanes as the scratch
  // FIFOs hold at the largest slot (the lane count never changes a result).
  arComm c = arComm();   // value-initialised: every field not set below is zero
  c.startMagic = c.endMagic = kCommMagic;
  c.nranks = nranks;
  c.maxChannels = c.nChannels = nChannels;
  c.proto = arProtoSimple;
  c.algo = arAlgoRing;
  c.device = dev;
  deviceInfo(dev, &c.numCUs, &c.wallClockKHz, &c.ldsPerBlock);
  if (c.numCUs <= 0) return arHipError;
  c.groupSizeMax = kMaxMembersPerGroup;
  c.ldsFifo = true;   // where the slots fit LDS, the scratch FIFOs go unused
  c.ldsSlots = e.nSteps > 0 ? e.nSteps : kLdsFifoSlots;
  for (int p = 0; p < 3; ++p) c.nSlots[p] = e.nSteps > 0 ? e.nSteps : kDefaultSlots[p];
  c.sliceBytes = e.sliceBytes;
  c.timeoutUs = e.timeoutUs;
  c.deadRank = -1;
  c.simpleUnroll = kSimpleUnrollDefault;
  c.ll128Unroll = 0;
  c.direct = true;
  tuneTableModels(c.models, c.treeModels);
  const size_t workerBytesMax = (size_t)c.nSlots[kSimple] * (size_t)kSimpleSlotBytesMax + sizeof(Conn);
  if (scratchBytes <= kScratchHeaderBytes) return arInvalidUsage;
  const size_t workersFit = (scratchBytes - kScratchHeaderBytes) / workerBytesMax;
  const size_t lanesFit = workersFit / (size_t)nranks;
  const int lanesDefault = kMaxWorkers / nranks > nChannels ? kMaxWorkers / nranks : nChannels;
  c.lanesMax = lanesDefault;

  // The plan arAllReduce makes; if its FIFOs are not in LDS, they go into the
  // scratch array, with as many lanes as it holds.
  Plan plan;
  arResult_t r = makePlan(&c, kCollAllReduce, count, dtype, op, aligned128, &plan);
  if (r != arSuccess) return r;
  if (!plan.ldsFifo) {
    if (lanesFit < (size_t)nChannels) return arInvalidUsage;   // not even one lane per channel fits
    c.lanesMax = (size_t)lanesDefault < lanesFit ? lanesDefault : (int)lanesFit;
    r = makePlan(&c, kCollAllReduce, count, dtype, op, aligned128, &plan);
    if (r != arSuccess) return r;
  }
  // the environment can force another protocol or algorithm (AR_PROTO, AR_ALGO)
  if (plan.proto != kSimple || plan.algo != arAlgoRing || plan.nGroups != 1) return arInvalidUsage;
  if (!fifosCover(&c, plan)) return arInternalError;
  // layout: header (control block, failed word), FIFOs, counters
  const size_t workers = (size_t)nranks * (size_t)c.lanesMax;
  c.fifoWorkerBytes[kSimple] = (size_t)plan.nSlots * (size_t)plan.slotBytes;
  c.ctrlDev = (Control*)scratch;
  c.failedDev = (uint32_t*)(scratch + 256);
  c.fifo[kSimple] = scratch + kScratchHeaderBytes;
  c.conn[kSimple] = (Conn*)(scratch + kScratchHeaderBytes + workers * c.fifoWorkerBytes[kSimple]);
  if (!plan.ldsFifo && kScratchHeaderBytes + workers * (c.fifoWorkerBytes[kSimple] + sizeof(Conn)) > scratchBytes)
    return arInternalError;   // (FIFOs in LDS leave the scratch FIFOs unused)

  KernelArgs a;
  buildArgs(&c, plan, kCollAllReduce, count, sendbufs, recvbufs, aligned16, &a);
  a.freshSteps = 1;
  if (e.debug >= 1)
    fprintf(stderr, "[ar] INFO no-alloc allreduce n=%d count=%zu dtype=%d op=%d nch=%d lanes=%d grid=%d unroll=%d\n",
            nranks, count, dtype, op, plan.nChannels, plan.lanes, plan.grid, plan.unroll);
  const hipError_t he = launchRing(plan, dtype, op, a, stream);
  c.startMagic = c.endMagic = 0;
  if (he != hipSuccess) {
    fprintf(stderr, "[ar] WARN kernel launch failed: %s\n", hipGetErrorString(he));
    return arHipError;
  }
  return arSuccess;
}

namespace {

// Device room for `words` task-table words (and the pinned staging copies).
arResult_t ensureTaskTable(arComm* c, size_t words) {
  if (words <= c->taskTableWords) return arSuccess;
  // earlier launches may still read the old table, earlier copies the old staging
  if (c->launched && hipStreamSynchronize(c->lastStream) != hipSuccess) return arHipError;
  for (int i = 0; i < kStagingBuffers; ++i) {
    if (c->stagingBusy[i] && hipEventSynchronize(c->stagingDone[i]) != hipSuccess) return arHipError;
    c->stagingBusy[i] = false;
    if (c->taskStaging[i]) (void)hipHostFree(c->taskStaging[i]);
    c->taskStaging[i] = nullptr;
  }
  if (c->taskTable) (void)hipFree(c->taskTable);
  c->taskTable = nullptr;
  c->taskTableWords = 0;
  const size_t cap = words < 4096 ? 4096 : words * 2;
  if (hipMalloc((void**)&c->taskTable, cap * sizeof(uint64_t)) != hipSuccess) return arHipError;
  for (int i = 0; i < kStagingBuffers; ++i)
    if (hipHostMalloc((void**)&c->taskStaging[i], cap * sizeof(uint64_t), hipHostMallocDefault) != hipSuccess)
      return arHipError;
  c->taskTableWords = cap;
  return arSuccess;
}

// Launch a comm's queued collectives [ch.6 §四, ch.7 §一]: one-rank calls are
// copies; the rest are aggregated by arGroupAggregate (AllReduces of one
// (op, type) within 4x of a run's largest share one launch; the halves run
// alone), each launch planned on its largest collective, and batched
// launches read their collectives from one task table copied to the device
// first.
arResult_t launchGroup(arComm* c) {
  std::vector<GroupTask>& T = c->pending;
  const int N = c->nranks;
  const int n = (int)T.size();
  const hipStream_t st = T[0].stream;
  if (c->aborted) return arInvalidUsage;
  if (memberGaveUp(c)) return arRemoteError;
  c->groupPlans.assign((size_t)n, arPlan_t());
  c->opCount += (uint64_t)n;
  if (N == 1) {   // the result is the input [ch.6 §三, one-rank path]
    for (int i = 0; i < n; ++i) {
      exportPlan(c, T[i].func, T[i].count, T[i].dtype, nullptr, &c->groupPlans[(size_t)i]);
      if (T[i].recv[0] != T[i].send[0] &&
          hipMemcpyAsync(T[i].recv[0], T[i].send[0], T[i].count * (size_t)elemSize(T[i].dtype),
                         hipMemcpyDeviceToDevice, st) != hipSuccess)
        return arHipError;
    }
    c->lastStream = st;
    c->launched = true;
    return arSuccess;
  }
  std::vector<int> keys((size_t)n), isolate((size_t)n), order((size_t)n), launchOf((size_t)n);
  std::vector<size_t> bytes((size_t)n);
  for (int i = 0; i < n; ++i) {
    keys[(size_t)i] = (T[i].func * 4 + T[i].op) * 8 + T[i].dtype;
    bytes[(size_t)i] = T[i].count * (size_t)elemSize(T[i].dtype) * (T[i].func == kCollAllReduce ? 1u : (size_t)N);
    isolate[(size_t)i] = T[i].func != kCollAllReduce;   // batched launches are AllReduce only
  }
  int nLaunches = 0;
  arResult_t r = arGroupAggregate(n, keys.data(), bytes.data(), isolate.data(), order.data(), launchOf.data(),
                                  &nLaunches);
  if (r != arSuccess) return r;

  // plan every launch before anything is enqueued
  struct Launch {
    int first, size;   // range of `order`
    Plan plan;
    bool aligned16;
    size_t row;        // first task-table row (batched launches)
  };
  std::vector<Launch> L;
  size_t rows = 0;
  for (int pos = 0; pos < n;) {
    Launch l;
    l.first = pos;
    while (pos < n && launchOf[(size_t)order[(size_t)pos]] == launchOf[(size_t)order[(size_t)l.first]]) ++pos;
    l.size = pos - l.first;
    const GroupTask& lead = T[(size_t)order[(size_t)l.first]];   // the largest
    bool a128 = true;
    l.aligned16 = true;
    for (int q = l.first; q < pos; ++q) {
      const GroupTask& t = T[(size_t)order[(size_t)q]];
      a128 = a128 && t.aligned128;
      l.aligned16 = l.aligned16 && t.aligned16;
    }
    const int kop = lead.func == kCollAllGather ? (lead.dtype == arUint64 ? arProbe : arSum) : lead.op;
    uint64_t aggBytes = 0;   // the aggregate's bytes together (its tasks run side by side)
    for (int q = l.first; q < pos; ++q) aggBytes += bytes[(size_t)order[(size_t)q]];
    r = l.size == 1 ? makePlan(c, lead.func, lead.count, lead.dtype, kop, a128, &l.plan)
                    : makePlan(c, lead.func, lead.count, lead.dtype, kop, a128, &l.plan, true, l.size, aggBytes);
    if (r != arSuccess) return r;
    if (!fifosCover(c, l.plan)) return arInternalError;
    r = l.plan.ldsFifo && l.plan.nGroups == 1 ? arSuccess : provisionFifo(c, l.plan.proto, l.plan.nSlots);
    if (r != arSuccess) return r;
    l.row = rows;
    if (l.size > 1) rows += (size_t)l.size;
    L.push_back(l);
  }

  // one copy of every batched launch's task rows, stream-ordered before them
  const size_t rowWords = 1 + 2 * (size_t)N;
  if (rows > 0) {
    r = ensureTaskTable(c, rows * rowWords);
    if (r != arSuccess) return r;
    const int sb = c->stagingNext;
    c->stagingNext = (sb + 1) % kStagingBuffers;
    if (c->stagingBusy[sb] && hipEventSynchronize(c->stagingDone[sb]) != hipSuccess) return arHipError;
    uint64_t* staging = c->taskStaging[sb];
    for (const Launch& l : L) {
      if (l.size == 1) continue;
      for (int q = 0; q < l.size; ++q) {
        const GroupTask& t = T[(size_t)order[(size_t)(l.first + q)]];
        uint64_t* w = staging + (l.row + (size_t)q) * rowWords;
        w[0] = t.count;
        for (int k = 0; k < N; ++k) {
          w[1 + k] = (uint64_t)(uintptr_t)t.send[(size_t)k];
          w[1 + N + k] = (uint64_t)(uintptr_t)t.recv[(size_t)k];
        }
      }
    }
    // the device table is rewritten only after the previous group's kernels
    // (same stream) have finished reading it
    if (hipMemcpyAsync(c->taskTable, staging, rows * rowWords * sizeof(uint64_t), hipMemcpyHostToDevice, st) !=
            hipSuccess ||
        hipEventRecord(c->stagingDone[sb], st) != hipSuccess)
      return arHipError;
    c->stagingBusy[sb] = true;
  }

  for (int li = 0; li < (int)L.size(); ++li) {
    const Launch& l = L[(size_t)li];
    const GroupTask& lead = T[(size_t)order[(size_t)l.first]];
    KernelArgs a;
    buildArgs(c, l.plan, lead.func, lead.count, lead.send.data(), lead.recv.data(), l.aligned16, &a);
    if (l.size > 1) {
      a.tasks = c->taskTable + l.row * rowWords;
      a.nTasks = l.size;
      a.taskSlots = l.plan.taskSlots;
    }
    const int kop = lead.func == kCollAllGather ? (lead.dtype == arUint64 ? arProbe : arSum) : lead.op;
    if (env().debug >= 1)
      fprintf(stderr, "[ar] INFO group launch %d: %d x func=%d dtype=%d op=%d algo=%d proto=%d nch=%d lanes=%d\n", li,
              l.size, lead.func, lead.dtype, lead.op, l.plan.algo, l.plan.proto, l.plan.nChannels, l.plan.lanes);
    const hipError_t he = launchRing(l.plan, lead.dtype, kop, a, st);
    if (he != hipSuccess) {
      fprintf(stderr, "[ar] WARN kernel launch failed: %s\n", hipGetErrorString(he));
      return arHipError;
    }
    c->lastStream = st;
    c->launched = true;
    for (int q = 0; q < l.size; ++q) {
      const int ti = order[(size_t)(l.first + q)];
      arPlan_t& pp = c->groupPlans[(size_t)ti];
      exportPlan(c, T[(size_t)ti].func, T[(size_t)ti].count, T[(size_t)ti].dtype, &l.plan, &pp);
      pp.groupLaunch = li;
      pp.tasksInLaunch = l.size;
    }
  }
  return arSuccess;
}
}  // namespace

extern "C" {

static arResult_t noteGroupError(arResult_t r) {
  if (r != arSuccess && tGroupDepth > 0 && tGroupError == arSuccess) tGroupError = r;
  return r;
}

arResult_t arAllReduce(arComm_t c, const void* const* sendbufs, void* const* recvbufs, size_t count,
                       arDataType_t dtype, arRedOp_t op, void* stream) {
  ApiRange range("arAllReduce");
  return noteGroupError(runColl(c, kCollAllReduce, sendbufs, recvbufs, count, dtype, op, stream));
}

arResult_t arReduceScatter(arComm_t c, const void* const* sendbufs, void* const* recvbufs, size_t recvcount,
                           arDataType_t dtype, arRedOp_t op, void* stream) {
  ApiRange range("arReduceScatter");
  return noteGroupError(runColl(c, kCollReduceScatter, sendbufs, recvbufs, recvcount, dtype, op, stream));
}

arResult_t arAllGather(arComm_t c, const void* const* sendbufs, void* const* recvbufs, size_t sendcount,
                       arDataType_t dtype, void* stream) {
  ApiRange range("arAllGather");
  return noteGroupError(runColl(c, kCollAllGather, sendbufs, recvbufs, sendcount, dtype, arSum, stream));
}

arResult_t arGroupStart(void) {
  ++tGroupDepth;
  return arSuccess;
}

arResult_t arGroupEnd(void) {
  ApiRange range("arGroupEnd");
  if (tGroupDepth == 0) return arInvalidUsage;   // not in a group
  if (--tGroupDepth > 0) return arSuccess;       // an inner group: the outermost end launches
  arResult_t r = tGroupError;
  tGroupError = arSuccess;
  std::vector<arComm*> comms;
  comms.swap(tGroupComms);
  for (arComm* c : comms) {
    if (r == arSuccess) {
      const arResult_t rc = launchGroup(c);
      if (rc != arSuccess) r = rc;
    }
    c->pending.clear();
    c->inGroup = false;
  }
  return r;
}

arResult_t arGetGroupPlan(arComm_t c, int index, arPlan_t* plan) {
  if (!commOk(c) || plan == nullptr || index < 0 || (size_t)index >= c->groupPlans.size())
    return arInvalidArgument;
  *plan = c->groupPlans[(size_t)index];
  return arSuccess;
}

arResult_t arCommGetAsyncError(arComm_t c, arResult_t* err) {
  if (!commOk(c) || err == nullptr) return arInvalidArgument;
  const uint32_t st = __atomic_load_n(&c->ctrlHost->status, __ATOMIC_ACQUIRE);
  if (st != 0) c->aborted = true;
  *err = (st != 0 || c->ctrlHost->abortFlag != 0) ? arRemoteError : arSuccess;
  return arSuccess;
}

arResult_t arCommFootprint(arComm_t c, size_t* deviceBytes) {
  if (!commOk(c) || deviceBytes == nullptr) return arInvalidArgument;
  *deviceBytes = deviceFootprint(c);
  return arSuccess;
}

arResult_t arCommCount(arComm_t c, int* nranks) {
  if (!commOk(c) || nranks == nullptr) return arInvalidArgument;
  *nranks = c->nranks;
  return arSuccess;
}

arResult_t arCommAbort(arComm_t c) {
  if (!commOk(c)) return arInvalidArgument;
  __atomic_store_n(&c->ctrlHost->abortFlag, 1u, __ATOMIC_RELEASE);
  c->aborted = true;
  return arSuccess;
}

arResult_t arDestroy(arComm_t c) {
  if (c == nullptr) return arSuccess;
  if (!commOk(c)) return arInvalidArgument;
  if (c->inGroup) return arInvalidUsage;   // it has collectives queued in an open group
  arResult_t r = arSuccess;
  if (c->launched && hipStreamSynchronize(c->lastStream) != hipSuccess) r = arHipError;
  freeComm(c);
  return r;
}

}  // extern "C"
