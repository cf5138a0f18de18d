/*
 * ar.h -- C ABI of libar.so: ring AllReduce (reduce-scatter then all-gather)
 * over per-channel FIFOs in the Simple, LL and LL128 wire formats, with N
 * virtual ranks emulated on one MI355X (gfx950).
 *
 * Sources of the operations (web pages, cited by title and section):
 *  [B]  "NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程" (AiReadCodeBooks)
 *  [T]  "NCCL 源码解析：从硬件拓扑到集合通信选型的完整链路"
 *  [I]  "NVIDIA GPU 集合通信库 NCCL 初始化流程源码级剖析"
 *
 * Conventions for every call:
 *  - Pointers marked "device" must point into memory of the GPU that was
 *    current when the communicator was created; "host" pointers are ordinary
 *    process memory.  No call takes ownership of caller memory.
 *  - Bad arguments return arInvalidArgument and enqueue nothing [B ch.3 §3.1,
 *    argument validation before any work is started].
 *  - A communicator is not thread-safe: calls on one communicator must come
 *    from one thread at a time, and AllReduce calls on one communicator must
 *    be ordered on one stream (or synchronised between streams), since they
 *    share its FIFOs [B ch.2 §2.1].
 */
#ifndef AR_H_
#define AR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque communicator handle [B ch.2 §2.1, the ncclComm_t handle]. */
typedef struct arComm* arComm_t;

/* Result codes, mirroring the reference's result enumeration [B ch.3 §3.1 and
 * ch.5 §一, the InvalidUsage vs InternalError distinction]. */
typedef enum {
  arSuccess = 0,
  arHipError = 1,         /* a HIP runtime call failed (or no usable GPU) */
  arSystemError = 2,      /* host allocation or OS failure */
  arInternalError = 3,    /* a bug: the library reached a state it should not */
  arInvalidArgument = 4,  /* a bad argument; nothing was enqueued */
  arInvalidUsage = 5,     /* legal arguments that cannot be honoured, e.g. a
                             forced protocol whose requirements are not met */
  arRemoteError = 6,      /* a ring member timed out or the comm was aborted */
  arInProgress = 7,
  arNumResults = 8
} arResult_t;

/* Wire formats, in the reference's protocol order [B ch.2 §2.4; ch.5 §二]. */
typedef enum {
  arProtoAuto = -1,  /* arTune picks protocol and channel count per call */
  arProtoLL = 0,     /* 8-byte lines: 4 bytes payload + 4 bytes flag */
  arProtoLL128 = 1,  /* 128-byte lines: 120 bytes payload + 8 bytes flag */
  arProtoSimple = 2  /* bulk FIFO slots with head/tail counters */
} arProto_t;

/* Algorithms [B ch.4 "Ring 與 Tree：把搜尋結果變成演算法拓撲"; ch.5 §一]. */
typedef enum {
  arAlgoAuto = -1,   /* arTune picks ring or tree per AllReduce */
  arAlgoRing = 0,    /* ring reduce-scatter + all-gather */
  arAlgoTree = 1     /* double binary tree: reduce up, broadcast down
                        (AllReduce only; ReduceScatter / AllGather use the ring) */
} arAlgo_t;

typedef enum {
  arInt32 = 0,
  arFloat32 = 1,
  arFloat16 = 2,
  arBfloat16 = 3,
  arUint64 = 4       /* only with arProbe (debug order probe) */
} arDataType_t;

typedef enum {
  arSum = 0,
  arMax = 1,         /* acc = (x > acc) ? x : acc, acc the incoming partial */
  arMin = 2,         /* acc = (x < acc) ? x : acc */
  arProbe = 3        /* debug: uint64 acc = acc*16 + x, not commutative, so the
                        folded value spells the order ranks were visited in */
} arRedOp_t;

/*
 * arInit -- create a communicator for `nranks` virtual ranks on the current
 * HIP device [B ch.3 §3.1-§3.3 and §3.6: validate, allocate the comm, set up
 * per-channel rings and FIFOs, one batched copy of device state].
 *  comm      (host, out) receives the handle.
 *  nranks    1..AR_MAX_RANKS virtual ranks; ring order is the identity for
 *            every channel [B ch.2 §2.3; ch.4 ring building].
 *  nChannels 1..AR_MAX_CHANNELS.  With a fixed protocol every AllReduce uses
 *            exactly this many channels (the count changes which elements form
 *            a chunk, hence the summation order).  With arProtoAuto it is the
 *            upper bound arTune may choose.
 *  proto     default protocol, or arProtoAuto.
 *  algo      arAlgoRing, arAlgoTree or arAlgoAuto (the default algorithm for
 *            AllReduce; arAlgoAuto lets arTune choose per call).
 * Allocates the FIFOs, counters and flags of the protocols the comm may run
 * on the device (owned by the comm, freed by arDestroy; see arCommFootprint).  Environment overrides, read once
 * per process: AR_PROTO (LL|LL128|SIMPLE), AR_NCHANNELS, AR_SLICE_BYTES
 * (Simple slice, default 512 KiB; chunk = 2 slices), AR_STEPS (FIFO depth
 * in slots, 2..8; default 2 for Simple, 8 for LL and LL128), AR_TIMEOUT_MS.
 * Errors: arInvalidArgument (bad counts or enums), arHipError (no device or a
 * HIP failure), arSystemError (host allocation).
 */
arResult_t arInit(arComm_t* comm, int nranks, int nChannels, arProto_t proto, arAlgo_t algo);

/*
 * arAllReduce -- every rank's recvbuf receives the reduction over all ranks'
 * sendbufs [B ch.1 §1.3, ch.2 §2.3 ring reduce-scatter + all-gather].
 * With the tree algorithm [B ch.4, ncclGetBtree / ncclGetDtree; "NCCL
 * Tree拓扑介绍"] channel ch of nCh runs on the second tree of the double
 * binary tree when nCh > 1 and 2*ch >= nCh, else on the first; each node
 * folds OP(OP(partial of child d0, partial of child d1), own value) and the
 * root's result is broadcast back down.  The ring's result depends on the
 * channel count and chunk size, the tree's on the channel count only.
 *  sendbufs  (host array of nranks device pointers) rank r's input, `count`
 *            contiguous elements.  The array itself is copied at call time.
 *  recvbufs  (host array of nranks device pointers) rank r's output.  In place
 *            (recvbufs[r] == sendbufs[r]) is allowed; otherwise buffers must
 *            not overlap.
 *  count     elements per rank.  count == 0 succeeds with no work [B ch.6 §三].
 *  dtype/op  see the enums; arProbe only with arUint64.
 *  stream    a hipStream_t (passed as void*); NULL is the default stream.
 * The call only enqueues: one kernel launch on `stream`, or a device copy
 * when nranks == 1 [B ch.6 §三, the one-rank path].  The caller synchronises
 * the stream before reading results [B ch.1 §1.3].  Buffers must stay valid
 * until the work completes.  Graph capture: once the comm has made one call
 * of the same plan, a call records that launch and nothing else (no
 * allocation, memset, copy or synchronisation), so calls may be captured on
 * `stream` into a HIP graph and replayed, each replay reducing whatever the
 * captured buffers then hold; rings and trees cut into workgroups carry
 * their edge counters from replay to replay.  Group calls (arGroupEnd) stage
 * their task tables through pinned host memory and are not for capture.  Element pointers need only element alignment;
 * forcing LL128 needs 128-byte aligned buffers, otherwise arInvalidUsage
 * [B ch.2 §2.4, LL128 alignment]; arProtoAuto never picks LL128 then.
 * A Simple ring of at most 16 ranks runs each (channel, lane) in one
 * workgroup and keeps its FIFO slots in that workgroup's LDS (arPlan_t
 * ldsFifoBytes; arDebugLdsFifo): its kernel then moves no FIFO bytes through
 * device memory, only the inputs and outputs.  A Simple tree inside one
 * workgroup does the same; longer rings and trees keep the FIFOs of the
 * edges inside each workgroup in LDS (a tree where they fit its plan's slot)
 * and those of the edges between workgroups in device memory.
 * Residency: a ring or tree of more than 16 ranks is cut into workgroups
 * that wait on one another, so all workgroups of its launch must be resident
 * at once.  The planner sizes that grid to what the GPU holds; a kernel
 * running beside it on another stream only delays the rest of the grid.  Two
 * such launches (of different comms, on streams not ordered with each other)
 * running at the same time could each hold part of the GPU: order them, or
 * set arDebugCooperative to 1, which makes the runtime run them one at a time.
 * A ring member that waits longer than the timeout (or an abort) makes the
 * kernel exit early and is reported by arCommGetAsyncError as arRemoteError;
 * the comm then only accepts arDestroy: a later call returns arRemoteError
 * (arInvalidUsage once arCommGetAsyncError or arCommAbort has been called)
 * and enqueues nothing, and the kernels of calls queued before the failure
 * was seen do nothing (their outputs are left untouched).
 */
arResult_t arAllReduce(arComm_t comm, const void* const* sendbufs, void* const* recvbufs,
                       size_t count, arDataType_t dtype, arRedOp_t op, void* stream);

/*
 * arReduceScatter -- rank r's recvbuf receives the reduction, over all ranks,
 * of block r of their sendbufs: the reduce-scatter half of the ring on its own
 * [B ch.5 §三: nSteps = nRanks-1; ch.6 §三: traffic nRanks x count].
 *  sendbufs  (host array of nranks device pointers) nranks*recvcount elements
 *            each; block q is elements [q*recvcount, (q+1)*recvcount).
 *  recvbufs  (host array of nranks device pointers) recvcount elements each.
 *            In place is recvbufs[r] == sendbufs[r] + r*recvcount elements.
 * Block b is folded in ring order b+1, b+2, ..., b (acc the incoming partial),
 * whatever the channel split.  Same protocols, errors and stream semantics as
 * arAllReduce.
 */
arResult_t arReduceScatter(arComm_t comm, const void* const* sendbufs, void* const* recvbufs,
                           size_t recvcount, arDataType_t dtype, arRedOp_t op, void* stream);

/*
 * arAllGather -- rank r's recvbuf receives every rank's sendbuf in rank order:
 * the all-gather half of the ring on its own [B ch.5 §三; ch.6 §三: it moves
 * data without reduction].
 *  sendbufs  (host array) sendcount elements each.
 *  recvbufs  (host array) nranks*sendcount elements each; rank q's data at
 *            [q*sendcount, (q+1)*sendcount).  In place is sendbufs[r] ==
 *            recvbufs[r] + r*sendcount elements.
 * dtype only sets the element size (arUint64 included).
 */
arResult_t arAllGather(arComm_t comm, const void* const* sendbufs, void* const* recvbufs,
                       size_t sendcount, arDataType_t dtype, void* stream);

/*
 * arTune -- choose protocol and channel count for a per-rank message of
 * nBytes with the pages' cost model [B ch.5 §一 (argmin over candidates),
 * §三 (ring bandwidth and latency); T §五, time = lat*latCount +
 * nBytes/(1000*bw) in microseconds and GB/s].
 *  proto, nChannels, predictedUs (host, out; any may be NULL).
 * nranks == 1 gives Simple with 0 channels [B ch.5 §一, single-rank short cut].
 * Candidates: protocols not disabled (AR_PROTO, LL128 alignment is the
 * caller's concern: arAllReduce re-tunes without LL128 when buffers are not
 * 128-byte aligned) times power-of-two channel counts up to the comm's
 * maximum with at least 32 KiB per channel.  Protocol ties keep Simple before
 * LL128 before LL; channel-count ties keep the larger count.
 * One GPU holds every rank, so a comm evaluates the model with each
 * algorithm's cap (maxBwGBs) scaled for N ranks sharing its HBM: ring x 8/N,
 * tree x 44/(6N-4) (the HBM bytes per model byte at 8 ranks, where the
 * constants are fitted, over that at N).  arTuneEval* take the constants as
 * given; arTuneGetModel returns them unscaled.
 */
arResult_t arTune(arComm_t comm, size_t nBytes, arProto_t* proto, int* nChannels, float* predictedUs);

/*
 * arTuneAlgo -- arTune that also reports the algorithm.  Over the comm's
 * algorithm setting: ring only, tree only, or both for arAlgoAuto (arTune
 * uses the same setting).  algo (host, out; may be NULL).
 */
arResult_t arTuneAlgo(arComm_t comm, size_t nBytes, arAlgo_t* algo, arProto_t* proto, int* nChannels,
                      float* predictedUs);

/* Per-protocol constants of the ring cost model (microseconds, GB/s). */
typedef struct {
  float baseLatUs;    /* per-call latency */
  float stepLatUs;    /* per ring step; a ring AllReduce has 2(N-1) steps */
  float bwPerChGBs;   /* bus bandwidth per channel before protocol discount */
  float maxBwGBs;     /* cap on the discounted bus bandwidth (llMaxBw and
                         the LL128 per-channel cap of the pages, generalised) */
} arTuneModel_t;

/*
 * arTuneEval -- the cost model as a pure function (no device needed).
 *  models     (host) 3 entries indexed by arProtoLL/LL128/Simple.
 *  protoMask  bit p set = protocol p allowed.
 *  busBw = nCh*bwPerCh; LL: min(maxBw, 0.5*busBw); LL128: min(maxBw,
 *  0.92*busBw); Simple: min(maxBw, busBw); algBw = busBw*N/(2(N-1));
 *  lat = baseLat + 2(N-1)*stepLat; t = lat + nBytes/(1000*algBw).
 * Returns arInvalidArgument for bad sizes or an empty mask, arInvalidUsage
 * if no candidate is valid.
 */
arResult_t arTuneEval(int nranks, int maxChannels, size_t nBytes, const arTuneModel_t* models,
                      unsigned protoMask, arProto_t* proto, int* nChannels, float* predictedUs);

/* Collectives, for the tuner and plan queries. */
typedef enum { arFuncAllReduce = 0, arFuncReduceScatter = 1, arFuncAllGather = 2 } arFunc_t;

/*
 * arTuneEvalColl -- arTuneEval for any of the three collectives: nSteps is
 * 2(N-1) for AllReduce and N-1 for ReduceScatter / AllGather, algBw =
 * busBw*N/nSteps [B ch.5 §三].  nBytes is the per-rank message for AllReduce
 * and nranks x count x element size for the other two (their traffic)
 * [B ch.6 §三].
 */
arResult_t arTuneEvalColl(arFunc_t func, int nranks, int maxChannels, size_t nBytes, const arTuneModel_t* models,
                          unsigned protoMask, arProto_t* proto, int* nChannels, float* predictedUs);

/*
 * arTuneEvalAlgo -- the ring and tree cost models as a pure function.
 *  ringModels, treeModels (host) 3 entries each, indexed by protocol; either
 *             may be NULL when its bit is clear in algoMask.
 *  algoMask   bit 0 ring, bit 1 tree.  The tree is only a candidate for
 *             arFuncAllReduce.
 * Tree [B ch.5 §四]: busBw = nCh*bwPerCh*0.92, LL x 1/3.8, LL128 x 120/128,
 * capped at maxBw; times the pages' treeCorrectionFactor[proto][log2i(nBytes
 * >> 6)] when that index is in [0, 23); lat = baseLat + 2*log2i(N)*stepLat;
 * t = lat + nBytes/(1000*busBw).  Candidates: ring (Simple, LL128, LL), then
 * tree (Simple, LL128, LL), each over the same channel counts; ties keep the
 * earlier candidate.  Errors as arTuneEval.
 */
arResult_t arTuneEvalAlgo(arFunc_t func, int nranks, int maxChannels, size_t nBytes,
                          const arTuneModel_t* ringModels, const arTuneModel_t* treeModels, unsigned algoMask,
                          unsigned protoMask, arAlgo_t* algo, arProto_t* proto, int* nChannels,
                          float* predictedUs);

/*
 * arTuneTableTime -- the tuner's measured time of one candidate (pure
 * function, no device).  The pages let a tuner plugin override the cost of
 * any (algorithm, protocol) candidate before the argmin [B ch.5 §一, step 3;
 * T §五, the tuner plugin]; here the override is a table of times measured on
 * MI355X per (ranks, bytes per rank) for the six candidates at the 32 KiB
 * channel rule, compiled in from the library's calibration record or read
 * once per process from the file AR_TUNE_FILE names (lines "ranks bytes
 * t_ringLL t_ringLL128 t_ringSimple t_treeLL t_treeLL128 t_treeSimple" in us,
 * "-" where a candidate cannot run; optional lines "model ring|tree
 * ll|ll128|simple base step bwPerCh cap" replace the cost model's constants;
 * a malformed file is ignored with a warning).  Between lines the time is
 * interpolated log-log in bytes, then log-log between the two nearest rank
 * counts; past a rank count's largest size it grows in proportion to bytes.
 * arTune, arTuneAlgo and arAllReduce (arProtoAuto or arAlgoAuto) pick the
 * fastest covered candidate where the comm may use the table's channel count.
 *  predictedUs (host, out).  arInvalidUsage where the table does not cover
 *  (nranks, nBytes) for that candidate; arInvalidArgument for bad arguments.
 */
arResult_t arTuneTableTime(int nranks, size_t nBytes, arAlgo_t algo, arProto_t proto, float* predictedUs);

/* Read / replace the tuner constants of a comm (calibration): the ring's
 * (arTuneGetModel / arTuneSetModel) or either algorithm's. */
arResult_t arTuneGetModel(arComm_t comm, arProto_t proto, arTuneModel_t* model);
arResult_t arTuneSetModel(arComm_t comm, arProto_t proto, const arTuneModel_t* model);
arResult_t arTuneGetAlgoModel(arComm_t comm, arAlgo_t algo, arProto_t proto, arTuneModel_t* model);
arResult_t arTuneSetAlgoModel(arComm_t comm, arAlgo_t algo, arProto_t proto, const arTuneModel_t* model);

/*
 * arSetConfig -- change the comm's default protocol and channel count, same
 * meaning as in arInit (nChannels must not exceed the value given there).
 * Provisions the FIFOs of a protocol the comm had not run (arHipError if that
 * allocation fails); arInvalidUsage while the comm has calls queued in an
 * open group.
 */
arResult_t arSetConfig(arComm_t comm, arProto_t proto, int nChannels);

/* arSetAlgo -- change the comm's AllReduce algorithm (as arInit's algo). */
arResult_t arSetAlgo(arComm_t comm, arAlgo_t algo);

/* What arAllReduce would run for a message (for tests and benchmarks). */
typedef struct {
  int proto;            /* arProto_t actually used */
  int nChannels;        /* channels (changes the summation order) */
  size_t chunkElems;    /* nominal chunk, elements (changes the summation order) */
  int lanesPerChannel;  /* wavefronts per ring member (pipelining only) */
  int ranksPerGroup;    /* ring members sharing one workgroup */
  int workgroups;       /* grid size of the launch */
  int threadsPerGroup;  /* workgroup size */
  int stepBytes;        /* FIFO slot size per wavefront (wire bytes) */
  int stepPayload;      /* payload bytes per FIFO slot */
  int nSlots;           /* FIFO depth in slots */
  float predictedUs;    /* cost-model time */
  double modelBytes;    /* ring: 5(N-1)*S, the stated HBM traffic model; tree:
                           2N*S + 4(N-1)*S (every input read and output
                           written once, every tree edge written and read
                           once going up and once coming down) */
  int algo;             /* arAlgo_t actually used */
  int groupLaunch;      /* arGetGroupPlan: index of the launch (in launch order)
                           that carried this call; -1 for a copy or a single call */
  int tasksInLaunch;    /* collectives sharing that launch (1 unless batched) */
  int ldsFifoBytes;     /* Simple rings and trees: the FIFO slots of the edges inside a
                           workgroup live in LDS, this many bytes per workgroup (ring:
                           members x nSlots x stepBytes; tree: two FIFOs per member);
                           0: FIFO slots in device memory */
  double deviceBytes;   /* device-memory bytes the plan's kernel must move: modelBytes,
                           except with LDS FIFOs, where only the inputs are read and the
                           outputs written (AllReduce 2N*S; ReduceScatter and AllGather
                           (N+1)*N*S, S the per-rank block), plus, for a ring cut into G
                           workgroups, a slot written and read on each of the G edges
                           between them per send (AllReduce 4(N-1)*G*S/N; the halves
                           2(N-1)*G*S), and for a tree cut into workgroups 4*S for each
                           tree edge between them (its share up and back down) */
} arPlan_t;

/*
 * arGetPlan -- fill `plan` with what arAllReduce(comm, ..., count, dtype, ...)
 * would use for buffers that are 128-byte aligned (aligned128 = 1) or not.
 * The channel count that runs can be below the requested one: a ring or tree
 * of more than 16 ranks needs its whole grid co-resident.  The ring halves its
 * channels until one lane per channel fits; the tree (single calls, automatic
 * lanes) takes the power-of-two fraction of the requested channels, the slot
 * and the group size with the largest groups, then the most bytes in flight
 * (channels x lanes x slot payload).  The result is that of the reported
 * count.
 */
arResult_t arGetPlan(arComm_t comm, size_t count, arDataType_t dtype, int aligned128, arPlan_t* plan);

/* Same for any collective; count as in that collective's call (recvcount /
 * sendcount for ReduceScatter / AllGather).  modelBytes is 5(N-1)*S for
 * AllReduce, 3N(N-1)*B for ReduceScatter and 2N(N-1)*B for AllGather (B =
 * block bytes): each reduce-scatter step reads 2 blocks and writes 1, each
 * all-gather step reads 1 and writes 1. */
arResult_t arGetPlanColl(arComm_t comm, arFunc_t func, size_t count, arDataType_t dtype, int aligned128,
                         arPlan_t* plan);

/*
 * arCommGetAsyncError -- non-blocking: arRemoteError once any ring member of
 * an earlier call timed out or the comm was aborted, else arSuccess
 * [B ch.2 §2.1 asyncResult; ch.7 group error paths].
 */
arResult_t arCommGetAsyncError(arComm_t comm, arResult_t* asyncError);

/*
 * arCommFootprint -- device memory a comm holds [B ch.2 §2.1, the
 * per-protocol FIFO buffers; ch.3 §3.6, device state set up for the comm]:
 * the FIFOs and counters of the protocols provisioned (N ranks x lanesMax
 * workers, each FIFO depth x the protocol's largest slot: 8 KiB Simple,
 * 2 KiB LL, 4 KiB LL128, plus 256 bytes of counters), the failed word and the
 * task table of grouped launches.  arInit provisions the comm's protocol at
 * its depth (all three with arProtoAuto); a protocol switched to later is
 * provisioned by arSetConfig or by its first call (which then allocates),
 * and a deeper FIFO (arDebugSlots) re-provisions after the comm's last
 * stream has finished.
 *  deviceBytes (host, out).
 */
arResult_t arCommFootprint(arComm_t comm, size_t* deviceBytes);

/*
 * arCommCount -- the number of virtual ranks of a comm [B ch.1 §1.2, the
 * query calls that check a new communicator: ncclCommCount].
 *  nranks (host, out).  arInvalidArgument for a bad comm or NULL.
 */
arResult_t arCommCount(arComm_t comm, int* nranks);

/*
 * arCommAbort -- raise the comm's abort word (host memory visible to running
 * kernels): every waiting ring member gives up within a bounded number of
 * polls.  Afterwards only arDestroy is accepted [B ch.1 §1.4].
 */
arResult_t arCommAbort(arComm_t comm);

/* arDestroy -- synchronise the last stream used, free device and host state
 * [B ch.1 §1.4, finalize then destroy]. */
arResult_t arDestroy(arComm_t comm);

/* Debug knobs for failure-handling tests (host-forced conditions; every
 * kernel still exits normally). */
typedef enum {
  arDebugTimeoutUs = 0,  /* a wait longer than this gives up (default 5e6) */
  arDebugDeadRank = 1,   /* rank whose ring members return at once (-1: none) */
  arDebugLanes = 2,      /* wavefronts per (rank, channel); 0 = automatic */
  arDebugSimpleSlotKiB = 3,  /* Simple FIFO slot per wavefront: 1, 2, 4 or 8 KiB */
  arDebugDirect = 4,     /* 1: Simple all-gather writes the successor's output
                            directly (default); 0: through the FIFO */
  arDebugSlots = 5,      /* FIFO depth in slots for every protocol, 2..8 */
  arDebugLaneSets = 6,   /* single-workgroup rings, single calls: at most this many workgroups,
                            each running several (channel, lane) pairs in turn on one FIFO set;
                            0 = one workgroup per pair */
  arDebugLL128SlotKiB = 7,  /* LL128 FIFO slot per wavefront: 2 or 4 KiB of wire (1920 or 3840
                               payload bytes), 0 = chosen per call (default); tree and group
                               (arGroupEnd) launches use 2 */
  arDebugGroupSpread = 8,   /* rings of more than 16 ranks: 1 = place the workgroups of one
                               (channel, lane) on consecutive ids, i.e. on different XCDs under
                               round-robin dispatch (default 0: ids congruent mod 8, one XCD) */
  arDebugLLChunkBytes = 9,     /* nominal chunk of the LL protocol in bytes, a multiple of 16
                                  from 16 to 64 MiB (0: the default); changes the summation
                                  order like the channel count, reported by arGetPlan */
  arDebugLL128ChunkBytes = 10, /* the same for LL128 */
  arDebugCooperative = 11,     /* rings / trees of more than 16 ranks: 1 = cooperative launch (the
                                  runtime checks residency and runs such launches one at a time,
                                  at 15-70 us per launch), 0 = plain launch of the same grid
                                  (default; see arAllReduce on residency) */
  arDebugLdsFifo = 13,         /* 1 (default): Simple rings and trees keep the FIFO slots of
                                  their edges inside a workgroup in LDS (those of at most 16
                                  ranks, single calls and arGroupEnd's batched launches; those
                                  cut into workgroups, single calls); 0: in device memory */
  arDebugGroupSize = 12,       /* at most this many ring or tree members per workgroup, 1..16
                                  (0: 16, the default): a ring or tree longer than this is cut
                                  into groups joined by device-coherent edges, as rings of more
                                  than 16 ranks always are; single calls only */
} arDebugKnob_t;
arResult_t arSetDebug(arComm_t comm, arDebugKnob_t knob, int64_t value);

/*
 * arGroupStart / arGroupEnd -- collectives called between them are queued
 * and launched together at the outermost arGroupEnd [B ch.7 §一, group
 * semantics: a per-thread nesting depth, the first error kept and reported
 * at the end, inner ends launch nothing; ch.6 §四, ncclPrepareTasks].
 * Inside a group each call validates its arguments and returns at once
 * (enqueuing nothing); its buffers must stay untouched until the group's
 * work completes, and collectives of one group must not share buffers.  At
 * the end, per communicator in the order it joined: the calls are
 * aggregated by arGroupAggregate; AllReduces of one (op, dtype) aggregated
 * together run in ONE kernel launch on the algorithm / protocol / channels
 * arTune picks for the largest of them, side by side on separate wavefronts
 * and FIFOs (as many at once as the FIFOs provisioned allow, the rest in
 * turn).  Each call's result is exactly that of a single call with that
 * plan, reported by arGetGroupPlan.  ReduceScatter / AllGather calls run in
 * launches of their own.  All calls on one comm in a group must use the
 * same stream (else arInvalidUsage).  arGroupEnd returns the first error of
 * the group (and launches nothing then), arInvalidUsage without a matching
 * arGroupStart.  arDestroy refuses a comm with queued calls.  The group
 * state is per host thread.
 */
arResult_t arGroupStart(void);
arResult_t arGroupEnd(void);

/*
 * arGroupAggregate -- the aggregation rule as a pure function (no device).
 *  keys      (host, nTasks) bucket of each task, e.g. (func, op, dtype);
 *  bytes     (host, nTasks) traffic of each task;
 *  isolate   (host, nTasks, may be NULL) 1 = never aggregate this task;
 *  order     (host, out, nTasks) task indices in launch order;
 *  launchOf  (host, out, nTasks) launch index of each task;
 *  nLaunches (host, out).
 * Tasks are sorted by bytes, largest first (ties keep call order), bucketed
 * by key (buckets in ascending key order), and inside a bucket a run starts
 * at its first task and takes each following task while 4 * bytes > the
 * first task's bytes [B ch.6 §四: aggregate tasks within 4x; aggIsolate].
 */
arResult_t arGroupAggregate(int nTasks, const int* keys, const size_t* bytes, const int* isolate, int* order,
                            int* launchOf, int* nLaunches);

/* arGetGroupPlan -- the plan the index-th call (call order, count > 0) of
 * the comm's last launched group ran with; arInvalidArgument out of range. */
arResult_t arGetGroupPlan(arComm_t comm, int index, arPlan_t* plan);

/*
 * arAllReduceNoAlloc -- arAllReduce for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It needs no communicator and allocates nothing (no
 * hipMalloc, hipFree or allocating library call, on any call).
 * What it computes: exactly arAllReduce on a comm of `nranks` ranks with
 * arProtoSimple, arAlgoRing and `nChannels` channels (same channel split and
 * chunk, hence the same bits); the same environment overrides apply.
 *  sendbufs, recvbufs, count, dtype, op, stream: as in arAllReduce.
 *  nranks     1..16: every ring fits one workgroup, so every FIFO edge keeps
 *             its counters in LDS and each call starts from step 0.
 *  nChannels  1..AR_MAX_CHANNELS.
 * Its control header (and its FIFOs, if a plan's cannot sit in LDS) live in
 * a fixed 64 MiB device
 * array inside the library, one per GPU it runs on, held until the process
 * ends; the device's first call looks up that array's address and clears its
 * header with a small kernel on `stream`.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (several host threads, or
 * streams not ordered with each other) race and give undefined results;
 * order them on one stream.  FIFOs in the array cap the lanes per channel at
 * what it holds (never a different result).
 * Errors: arInvalidArgument for bad arguments (nothing enqueued);
 * arInvalidUsage when FIFOs must go into the array and even one lane per
 * channel does not fit (the maximum: nranks x nChannels x FIFO depth x 8 KiB
 * plus 256 bytes per lane) or when AR_PROTO / AR_ALGO force another protocol
 * or algorithm; arHipError
 * for HIP failures.  A member that waits longer than the timeout gives up and
 * that call's output is incomplete; with no comm, this path does not report it.
 */
arResult_t arAllReduceNoAlloc(const void* const* sendbufs, void* const* recvbufs, int nranks, int nChannels,
                              size_t count, arDataType_t dtype, arRedOp_t op, void* stream);

const char* arGetErrorString(arResult_t result);

/* Library limits. */
#define AR_MAX_RANKS 128
#define AR_MAX_CHANNELS 64

#ifdef __cplusplus
}
#endif
#endif /* AR_H_ */
