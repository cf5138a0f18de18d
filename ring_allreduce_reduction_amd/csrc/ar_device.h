#pragma once
// ar_device.h -- the ring AllReduce data path for gfx950 (device code).
//
// What runs: one wavefront per ring member (virtual rank r, channel ch, lane
// k).  A member walks the ring schedule of the pages ["NCCL 原始碼解讀：一個
// AllReduce 的 GPU 旅程", ch.2 §2.3, RingARAlgorithm::getNextSendAddr and the
// reduce-scatter / all-gather walkthrough]: at stage s it sends chunk
// (r - 1 - s) mod N, so over 2N-1 stage slots it does
//     send | recv-reduce-send x (N-2) | recv-reduce-copy-send |
//     recv-copy-send x (N-2) | recv
// and every transfer goes through a FIFO in HBM owned by the receiver,
// with credits (head) and readiness (tail counter, or per-line flags for the
// LL / LL128 wire formats) [same book, ch.2 §2.4, the send/recv memory with
// head and tail counters on separate cache lines, and the LL / LL128 /
// Simple protocols].
//
// Where it runs: the N members of one (channel, lane) sit in one workgroup
// (N <= 16), so every producer/consumer pair shares a CU and its vector L1:
// the FIFO handoff needs only workgroup-scope release/acquire, which on gfx950
// is a plain ordered store / load, and there is no cross-workgroup wait at all
// (no co-residency requirement, no deadlock from scheduling).  For N > 16 the
// ring is cut into groups of up to 16 members; an edge between groups moves
// its bytes with device-coherent loads and stores (no L2-wide cache
// maintenance, see releaseEdge) and the launch is cooperative so that every
// group is resident.
//
// Each member reads only its own send buffer, writes only its own receive
// buffer and its successor's FIFO, so in-place use is safe: a member reads
// chunk c of its input before it writes chunk c of its output.
#include "ar_internal.h"

namespace ar {
namespace {

typedef uint32_t u32;
typedef uint64_t u64;
typedef u32 v4u __attribute__((ext_vector_type(4)));
typedef u32 v2u __attribute__((ext_vector_type(2)));

// A step kind is the set of things a member does with one slot: read its
// local operand, receive from its predecessor, send to its successor, write
// its output.  AllReduce uses send / recv-reduce-send / recv-reduce-copy-send /
// recv-copy-send / recv; ReduceScatter ends with recv-reduce-copy; AllGather
// starts with copy-send.
constexpr int kLocalBit = 1, kRecvBit = 2, kSendBit = 4, kOutBit = 8;
enum Kind : int {
  kSend = kLocalBit | kSendBit,
  kRecvReduceSend = kLocalBit | kRecvBit | kSendBit,
  kRecvReduceCopySend = kLocalBit | kRecvBit | kSendBit | kOutBit,
  kRecvCopySend = kRecvBit | kSendBit | kOutBit,
  kRecv = kRecvBit | kOutBit,
  kRecvReduceCopy = kLocalBit | kRecvBit | kOutBit,
  kCopySend = kLocalBit | kSendBit | kOutBit,
};
// A kind as a type, for steps compiled for one kind: their code has no branch
// on what the step does, nor paths for kinds no stage has
// (kKindAtRunTime: the kind is an argument).
constexpr int kKindAtRunTime = -1;
template <int K>
struct KindTag {
  static constexpr int value = K;
};

__device__ __forceinline__ u64 divUp(u64 x, u64 y) { return (x + y - 1) / y; }
__device__ __forceinline__ u64 alignUp(u64 x, u64 a) { return divUp(x, a) * a; }
__device__ __forceinline__ u64 umin(u64 a, u64 b) { return a < b ? a : b; }

// ------------------------------------------------------------- element ops
// Sum / Max / Min with acc the incoming partial and x the local value.
// A 16-bit Sum is the f32 sum of the two exactly widened operands, rounded
// back to nearest-even.  For f16 the packed half add gives those bits
// directly: f32 carries 24 significand bits, at least twice f16's 11 plus two,
// so rounding first to f32 and then to f16 equals rounding once.  bf16 adds in
// f32 and narrows a pair with the packed RNE conversion.  Denormals are kept
// in both (the kernels run with f16 and f32 denormals on).  A NaN sum stays a
// quiet NaN; its payload bits are the hardware's.

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16ToF32(u32 h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16ToF32(u32 h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int DT>
__device__ __forceinline__ u32 sumHalfPair(u32 acc, u32 x) {   // two 16-bit elements
  if (DT == arFloat16) return __builtin_bit_cast(u32, __builtin_bit_cast(h2, acc) + __builtin_bit_cast(h2, x));
  const f2 s = {bf16ToF32(acc & 0xffffu) + bf16ToF32(x & 0xffffu),
                __uint_as_float(acc & 0xffff0000u) + __uint_as_float(x & 0xffff0000u)};
  return __builtin_bit_cast(u32, __builtin_convertvector(s, bf2));
}

template <int DT, int OP>
__device__ __forceinline__ u32 maxMinHalf(u32 acc, u32 x) {   // one 16-bit element
  float a = DT == arBfloat16 ? bf16ToF32(acc) : f16ToF32(acc);
  float b = DT == arBfloat16 ? bf16ToF32(x) : f16ToF32(x);
  if (OP == arMax) return (b > a) ? x : acc;
  return (b < a) ? x : acc;
}

template <int DT, int OP>
__device__ __forceinline__ u32 combineWord(u32 acc, u32 x) {   // one 32-bit word
  if (DT == arFloat32) {
    float a = __uint_as_float(acc), b = __uint_as_float(x);
    if (OP == arSum) return __float_as_uint(a + b);
    if (OP == arMax) return (b > a) ? x : acc;
    return (b < a) ? x : acc;
  } else if (DT == arInt32) {
    if (OP == arSum) return acc + x;   // wraps
    if (OP == arMax) return ((int)x > (int)acc) ? x : acc;
    return ((int)x < (int)acc) ? x : acc;
  } else if (OP == arSum) {
    return sumHalfPair<DT>(acc, x);
  } else {                             // two 16-bit elements
    u32 lo = maxMinHalf<DT, OP>(acc & 0xffffu, x & 0xffffu);
    u32 hi = maxMinHalf<DT, OP>(acc >> 16, x >> 16);
    return lo | (hi << 16);
  }
}

template <int DT, int OP>
__device__ __forceinline__ v4u combine(v4u acc, v4u x) {
  v4u r;
  if (DT == arUint64) {                // probe: acc*16 + x on each 64-bit half
    u64 a0 = ((u64)acc.y << 32) | acc.x, x0 = ((u64)x.y << 32) | x.x;
    u64 a1 = ((u64)acc.w << 32) | acc.z, x1 = ((u64)x.w << 32) | x.z;
    a0 = a0 * 16u + x0;
    a1 = a1 * 16u + x1;
    r.x = (u32)a0; r.y = (u32)(a0 >> 32); r.z = (u32)a1; r.w = (u32)(a1 >> 32);
  } else {
    r.x = combineWord<DT, OP>(acc.x, x.x);
    r.y = combineWord<DT, OP>(acc.y, x.y);
    r.z = combineWord<DT, OP>(acc.z, x.z);
    r.w = combineWord<DT, OP>(acc.w, x.w);
  }
  return r;
}

// ------------------------------------------------------------- memory access
// User buffers stream through once: non-temporal hints keep them from
// evicting the FIFO slots, which are re-used and should stay in cache.

__device__ __forceinline__ v4u ldNt16(const char* p) { return __builtin_nontemporal_load((const v4u*)p); }
__device__ __forceinline__ v2u ldNt8(const char* p) { return __builtin_nontemporal_load((const v2u*)p); }
__device__ __forceinline__ void stNt16(char* p, v4u v) { __builtin_nontemporal_store(v, (v4u*)p); }
__device__ __forceinline__ void stNt8(char* p, v2u v) { __builtin_nontemporal_store(v, (v2u*)p); }

// Load `pieceBytes` (16 or 8) user bytes at p of which `valid` are in range;
// bytes past the range read as zero.  Element-wise when short or unaligned.
template <int ESZ, bool NT>
__device__ __forceinline__ v4u loadUser(const char* p, long valid, int pieceBytes, bool aligned) {
  v4u v = {0u, 0u, 0u, 0u};
  if (valid >= pieceBytes && aligned) {
    if (pieceBytes == 16) {
      v = NT ? ldNt16(p) : *(const v4u*)p;
    } else {
      v2u t = NT ? ldNt8(p) : *(const v2u*)p;
      v.x = t.x; v.y = t.y;
    }
  } else if (valid > 0) {
    u32 w[4] = {0u, 0u, 0u, 0u};
    int nb = valid < pieceBytes ? (int)valid : pieceBytes;
    for (int b = 0; b < nb; b += ESZ) {
      if (ESZ == 2) {
        u32 h = *(const uint16_t*)(p + b);
        w[b >> 2] |= h << ((b & 2) * 8);
      } else if (ESZ == 4) {
        w[b >> 2] = *(const u32*)(p + b);
      } else {
        u64 d = *(const u64*)(p + b);
        w[b >> 2] = (u32)d;
        w[(b >> 2) + 1] = (u32)(d >> 32);
      }
    }
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
  }
  return v;
}

template <int ESZ, bool NT>
__device__ __forceinline__ void storeUser(char* p, v4u v, long valid, int pieceBytes, bool aligned) {
  if (valid >= pieceBytes && aligned) {
    if (pieceBytes == 16) {
      if (NT) stNt16(p, v);
      else *(v4u*)p = v;
    } else {
      v2u t; t.x = v.x; t.y = v.y;
      if (NT) stNt8(p, t);
      else *(v2u*)p = t;
    }
  } else if (valid > 0) {
    u32 w[4] = {v.x, v.y, v.z, v.w};
    int nb = valid < pieceBytes ? (int)valid : pieceBytes;
    for (int b = 0; b < nb; b += ESZ) {
      if (ESZ == 2) {
        *(uint16_t*)(p + b) = (uint16_t)(w[b >> 2] >> ((b & 2) * 8));
      } else if (ESZ == 4) {
        *(u32*)(p + b) = w[b >> 2];
      } else {
        *(u64*)(p + b) = (u64)w[b >> 2] | ((u64)w[(b >> 2) + 1] << 32);
      }
    }
  }
}

// ------------------------------------------------------------- flags
// Scope of an edge: workgroup when producer and consumer share the
// workgroup, agent otherwise.

// Counter comparisons use the low 32 bits, modulo 2^32: the two ends of one
// FIFO are never further apart than its depth (at most 8 slots), so the sign
// of the 32-bit difference decides.  The scalar unit compares 32-bit values
// in one instruction and has no ordered 64-bit compare (a u64 comparison of
// uniform values costs two moves to vector registers, a vector compare and a
// mask test): every wait and credit check of every step pays for it, and the
// waves of a workgroup step in lockstep, sharing their SIMDs' issue slots.
__device__ __forceinline__ bool reached(u32 have, u32 target) { return (int)(have - target) >= 0; }

__device__ __forceinline__ u32 ldCounter32(const u64* p, bool agent) {
  const u32* q = (const u32*)p;   // the low word (little-endian)
  u32 v = agent ? __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                : __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ u64 ldCounter(const u64* p, bool agent) {
  u64 v = agent ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                : __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  // every lane read the same word; make the value provably uniform
  u32 lo = __builtin_amdgcn_readfirstlane((u32)v);
  u32 hi = __builtin_amdgcn_readfirstlane((u32)(v >> 32));
  return ((u64)hi << 32) | lo;
}
__device__ __forceinline__ void stRelaxed64(u64* p, u64 v, bool agent) {
  if (agent) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ u64 ldRelaxed64(const u64* p, bool agent) {
  return agent ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               : __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Edges inside a workgroup order their payload with workgroup-scope
// release/acquire, which gfx950 compiles to ordered loads and stores with no
// cache maintenance.
//
// Edges between workgroups never use agent-scope fences: on gfx950 an
// agent-scope release writes back, and an acquire invalidates, the whole L2
// of the XCD (buffer_wbl2 sc1 / buffer_inv sc1), which at every ring step
// stalls every wavefront on that XCD.  Instead every byte that crosses such
// an edge -- slot payload, LL words, LL128 flags, counters -- is moved by a
// relaxed agent-scope atomic, which gfx950 issues as a plain load or store
// with the sc1 bit: it is served at the device's coherence point rather than
// by one XCD's L2, so it is coherent on its own.  What a release adds on top
// is order: the producer waits until its payload stores have completed
// (vmcnt(0)) before it stores the counter or flag that publishes them.  On
// the consumer the payload loads are issued only after the counter or flag
// read has returned the awaited value, as every wait loop branches on it.
__device__ __forceinline__ void stCoh16(char* p, v4u v) {
  __hip_atomic_store((u64*)p, ((u64)v.y << 32) | v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store((u64*)p + 1, ((u64)v.w << 32) | v.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stCoh8(char* p, v2u v) {
  __hip_atomic_store((u64*)p, ((u64)v.y << 32) | v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ v4u ldCoh16(const char* p) {
  const u64 a = __hip_atomic_load((const u64*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const u64 b = __hip_atomic_load((const u64*)p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v4u{(u32)a, (u32)(a >> 32), (u32)b, (u32)(b >> 32)};
}
__device__ __forceinline__ v2u ldCoh8(const char* p) {
  const u64 a = __hip_atomic_load((const u64*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v2u{(u32)a, (u32)(a >> 32)};
}

// Before publishing what this wavefront stored for its peer.  Workgroup
// edge: a workgroup-scope release.  Agent edge: the release keeps the
// compiler from sinking the payload stores below the publishing store, and
// s_waitcnt vmcnt(0) (gfx9 encoding 0x0F70: vmcnt 0, expcnt and lgkmcnt
// untouched) holds the wavefront until they have completed.
__device__ __forceinline__ void releaseEdge(bool agent) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (agent) __builtin_amdgcn_s_waitcnt(0x0F70);
}
// After a counter or flag read returned the awaited value, before touching
// what it publishes (or, for a credit, before overwriting the slot).  Both
// kinds of edge need only the compiler ordering of a workgroup-scope acquire:
// an agent edge's payload loads are device-coherent by themselves.
__device__ __forceinline__ void acquireEdge() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup"); }

// Credit: the receiver has drained a slot.  Its loads of the slot returned
// before this point (their values were used by the stores that precede it).
__device__ __forceinline__ void stCounterRelease(u64* p, u64 v, bool agent) {
  if (agent) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    stRelaxed64(p, v, true);
  } else {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// Bounded waiting.  Every spin sleeps briefly; every 4096 spins the abort
// word and the wall clock are checked, and a hard cap on spins backs the
// clock up.  The clock starts at the first of those checks: reading it is a
// scalar memory access of about a microsecond, and the usual wait in a ring
// or tree chain (a neighbour a few hundred nanoseconds behind) ends long
// before, so it must not pay for one.  The abort word is in host memory, a
// PCIe round trip per read: an LDS poll spins in about 100 ns, and with a
// check every 256 spins the thousands of wavefronts waiting in a ring cut
// into workgroups read it often enough to stall one another (32 ranks x
// 64 MiB: 10 of 36 calls 1.1-3.4x slower; none at 4096).  On give-up the
// member records why and the caller returns, so every wavefront of the
// kernel always exits.  The reason goes to the host-visible status word and
// to the comm's failed word in device memory: a member that gave up left its
// counters (and LL / LL128 lines) in the middle of a call, so a later call
// must not start from them; every kernel reads the failed word on entry and
// does nothing once it is set.
//
// A waiting wavefront drops to the lowest issue priority until its wait
// ends; the kernels run at kWorkPrio otherwise.  Up to 15 members of a
// workgroup can be polling while the one the chain waits on works on the same
// CU, and at equal priority their polls take its issue slots (16 ranks, 4 KiB
// per rank: 104 us at equal priority, 75 us with the pollers lowered).
constexpr int kWorkPrio = 2;
struct Waiter {
  u32 spins = 0;
  u64 t0 = 0;
  __device__ __forceinline__ ~Waiter() {
    if (spins != 0) __builtin_amdgcn_s_setprio(kWorkPrio);
  }
};

__device__ __forceinline__ bool keepWaiting(const KernelArgs& a, Waiter& w) {
  if (w.spins == 0) __builtin_amdgcn_s_setprio(0);
  ++w.spins;
  __builtin_amdgcn_s_sleep(2);
  if ((w.spins & 4095u) == 0) {
    const u64 now = wall_clock64();
    if (w.spins == 4096u) w.t0 = now;
    u32 ab = __hip_atomic_load(&a.ctrl->abortFlag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    u32 code = 0;
    if (__builtin_amdgcn_readfirstlane(ab) != 0) code = kStatusAbort;
    else if (now - w.t0 > a.timeoutTicks || w.spins >= (1u << 30)) code = kStatusTimeout;
    if (code != 0) {
      __hip_atomic_store(a.failed, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl->status, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      return false;
    }
  }
  return true;
}

// Nonzero once a member of an earlier call (or of this one) gave up.  Read
// once per wavefront on entry, before anything of the call is touched.
__device__ __forceinline__ u32 callFailed(const KernelArgs& a) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(a.failed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Wait until *p >= target.
__device__ __forceinline__ bool waitGeq(const KernelArgs& a, const u64* p, u64 target, bool agent) {
  const u32 t = (u32)target;
  if (reached(ldCounter32(p, agent), t)) return true;
  Waiter w;
  while (true) {
    if (!keepWaiting(a, w)) return false;
    if (reached(ldCounter32(p, agent), t)) return true;
  }
}

// Counters of the edges inside one workgroup live in LDS: member wave w's
// tail (what its predecessor has published into its FIFO) at w, its head
// (what it has consumed) at kLdsHead + w.  The FIFO slots themselves stay
// in HBM; only the handshake moves.  A wavefront's vector memory operations
// complete in issue order, so a counter polled with global loads waits
// behind every load the member issued before it (its local operand from
// HBM, above all); an LDS poll completes on its own counter.  Ordering is
// unchanged: the producer's slot stores and the LDS counter store are
// ordered by the same workgroup-scope release as before, which gfx950
// compiles to no wait at all (every wavefront of the workgroup shares the
// CU's vector memory path), and the consumer loads the slot only after the
// counter read returned.  Global copies are written back when a call ends,
// so the next call starts every edge at the same step.
constexpr int kLdsHead = kMaxMembersPerGroup;
__device__ __forceinline__ u64* ldsCounters() {
  __shared__ u64 c[2 * kMaxMembersPerGroup];
  return c;
}
__device__ __forceinline__ u32 ldLds32(int i) {
  const u32 v = __hip_atomic_load((u32*)&ldsCounters()[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(v);
}
// A counter of an edge inside the workgroup is read as its low word only,
// so a step publishes just that word; every lane of the wavefront stores the
// same value (one LDS write, and no execution-mask change around it).
__device__ __forceinline__ void stLds32(int i, u32 v) {
  __hip_atomic_store((u32*)&ldsCounters()[i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void stLds32Release(int i, u32 v) {
  __hip_atomic_store((u32*)&ldsCounters()[i], v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void stLds(int i, u64 v) {
  __hip_atomic_store(&ldsCounters()[i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void stLdsRelease(int i, u64 v) {
  __hip_atomic_store(&ldsCounters()[i], v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// FIFO slots of the edges of a Simple ring that lies inside one workgroup,
// when they live in LDS too (dynamic LDS sized at launch): member wave w's
// nSlots slots, written by its predecessor, at w * nSlots * slot bytes.  A
// handoff is then an LDS store, the counter store and an LDS load, and the
// ring's device-memory traffic is its inputs and outputs alone.
extern __shared__ __align__(16) char ldsFifoBase[];

__device__ __forceinline__ bool waitLdsGeq(const KernelArgs& a, int i, u64 target) {
  const u32 t = (u32)target;
  if (reached(ldLds32(i), t)) return true;
  Waiter w;
  while (true) {
    if (!keepWaiting(a, w)) return false;
    if (reached(ldLds32(i), t)) return true;
  }
}

// LL receive: every live 16-byte line {d0, flag, d1, flag} of this lane's U
// pieces is polled until both of its 8-byte words carry `flag`.  Each poll
// issues every piece's loads back to back and only then compares them (with
// selects, no branch per piece): a branch per piece made the compiler wait
// for one piece's loads before issuing the next piece's, one L2 round trip
// per piece per poll.  Each word is one 64-bit atomic load, so its data and
// flag are seen together; a line already seen is read again harmlessly (its
// slot is not reused before this step releases it).
template <int U>
__device__ __forceinline__ bool pollLL(const KernelArgs& a, const char* slot, const int (&wireOff)[U],
                                       const int (&payOff)[U], long valid, u32 flag, bool agent, v4u (&in)[U]) {
  bool done[U];
#pragma unroll
  for (int u = 0; u < U; ++u) { done[u] = payOff[u] >= valid; in[u] = v4u{0u, 0u, 0u, 0u}; }
  Waiter w;
  while (true) {
    u64 w0[U], w1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {   // a piece already seen is not read again
      const u64* line = (const u64*)(slot + wireOff[u]);
      w0[u] = done[u] ? 0 : ldRelaxed64(line, agent);
      w1[u] = done[u] ? 0 : ldRelaxed64(line + 1, agent);
    }
    bool all = true;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool now = !done[u] && (u32)(w0[u] >> 32) == flag && (u32)(w1[u] >> 32) == flag;
      in[u].x = now ? (u32)w0[u] : in[u].x;
      in[u].y = now ? (u32)w1[u] : in[u].y;
      done[u] = done[u] || now;
      all = all && done[u];
    }
    if (__all(all)) return true;
    if (!keepWaiting(a, w)) return false;
  }
}

// LL128 receive, first half: the flag lane of every 128-byte line (lane 7
// of each group of 8) polls the 8-byte flag of each live line of its U
// pieces, all U loads in flight at once, until every one carries `flag`.
template <int U>
__device__ __forceinline__ bool pollLL128Flags(const KernelArgs& a, const char* slot, const int (&wireOff)[U], int lane,
                                               long valid, u64 flag, bool agent) {
  const bool flagLane = (lane & 7) == 7;
  bool done[U];
#pragma unroll
  for (int u = 0; u < U; ++u) done[u] = !flagLane || u * kLL128UnitPayload >= valid;
  Waiter w;
  while (true) {
    bool all = true;
    if (flagLane) {
      u64 f[U];
#pragma unroll
      for (int u = 0; u < U; ++u)   // a flag already seen is not read again
        f[u] = done[u] ? flag : ldRelaxed64((const u64*)(slot + wireOff[u] + 8), agent);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        done[u] = done[u] || f[u] == flag;
        all = all && done[u];
      }
    }
    if (__all(all)) return true;
    if (!keepWaiting(a, w)) return false;
  }
}

// LL128 receive on an edge inside the workgroup, in one round trip: every
// lane loads its line's 8-byte flag with a workgroup-scope acquire and then
// its payload piece, with no wait in between, and keeps the payload only if
// every live line's flag matched (otherwise it polls again).  Each lane's
// acquire orders its own payload load after its flag load: if the flag is
// the sender's (published after its payload stores by a workgroup-scope
// release), the payload is that step's.  gfx950 implements a workgroup-scope
// acquire load as the plain load itself (the wavefronts of a workgroup share
// the CU's in-order vector memory path), so the payload loads issue right
// behind the flag loads and one L2 round trip serves both.  Across
// workgroups the payload is read only after the flags returned
// (pollLL128Flags), as device-coherent loads carry no such order.
template <int U>
__device__ __forceinline__ bool pollLL128Lines(const KernelArgs& a, const char* slot, const int (&wireOff)[U], int lane,
                                               long valid, u64 flag, v4u (&in)[U]) {
  const int lineOff = (lane >> 3) * kLL128LineBytes + kLL128LinePayload;   // this lane's line's flag word
  Waiter w;
  while (true) {
    // Every unit is read, live or not: skipping the units past the step's
    // bytes (a branch around their loads) measured 4-10% slower.
    u64 f[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      f[u] = __hip_atomic_load((const u64*)(slot + u * kLL128UnitBytes + lineOff), __ATOMIC_ACQUIRE,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    // every lane loads its whole 16-byte piece (no branch, so nothing waits
    // between these loads and the flags'); the flag lane's upper half is the
    // flag itself, which no store of that lane (8 payload bytes) ever writes
#pragma unroll
    for (int u = 0; u < U; ++u) in[u] = *(const v4u*)(slot + wireOff[u]);
    bool all = true;
#pragma unroll
    for (int u = 0; u < U; ++u) all = all && (u * kLL128UnitPayload >= valid || f[u] == flag);
    if (__all(all)) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u * kLL128UnitPayload >= valid) in[u] = v4u{0u, 0u, 0u, 0u};
      return true;
    }
    if (!keepWaiting(a, w)) return false;
  }
}

// Workgroup -> (lane id L, group g).  With several groups per lane, the
// groups of one lane get workgroup ids congruent mod 8, i.e. the same XCD
// under round-robin dispatch, so their edges stay in one L2: a locality hint
// only, the edges between workgroups are device-coherent wherever the groups
// run.  a.groupSpread gives them consecutive ids instead, i.e. different
// XCDs, which exercises exactly that.
__device__ __forceinline__ void laneAndGroup(const KernelArgs& a, int& L, int& g) {
  if (a.nGroups == 1) {
    L = blockIdx.x;
    g = 0;
  } else if (a.groupSpread) {
    g = blockIdx.x % a.nGroups;
    L = blockIdx.x / a.nGroups;
  } else {
    const int x = blockIdx.x % 8;
    g = (blockIdx.x / 8) % a.nGroups;
    L = (blockIdx.x / (8 * a.nGroups)) * 8 + x;
  }
}

// ------------------------------------------------------------- one member

struct Member {
  int lane;
  char* rfifo;        // my FIFO (predecessor writes it)
  char* sfifo;        // successor's FIFO (I write it)
  Conn* self;
  Conn* succ;
  u64 recvStep;       // slots consumed from my FIFO so far (== self->head)
  u64 sendStep;       // slots written into the successor's FIFO (== succ->tail)
  u32 recvSlot;       // recvStep % nSlots
  u32 sendSlot;       // sendStep % nSlots
  u32 succHead;       // low word of the last value read from succ->head; head
                      // only grows, so a stale copy never over-reports free slots
  int selfW;          // my wavefront in the workgroup: my LDS counters
  int succW;          // the successor's, when it shares the workgroup
  bool recvAgent;
  bool sendAgent;
  bool aligned;
  bool direct;
};

// CACHED: skip the poll while the last credit read still covers this slot.
template <bool CACHED, bool XWG>
__device__ __forceinline__ bool waitCredit(const KernelArgs& a, Member& m) {
  // slot sendStep % nSlots is free once the successor consumed step
  // sendStep - nSlots (modulo 2^32: before the first nSlots steps of a FIFO
  // the target is "negative" and any head reaches it)
  const u32 need = (u32)m.sendStep + 1u - (u32)a.nSlots;
  const bool agent = XWG && m.sendAgent;
  if (CACHED) {
    if (reached(m.succHead, need)) return true;   // ordered by the acquire after that read
    m.succHead = agent ? ldCounter32(&m.succ->head, true) : ldLds32(kLdsHead + m.succW);
    if (!reached(m.succHead, need)) {
      Waiter w;
      do {
        if (!keepWaiting(a, w)) return false;
        m.succHead = agent ? ldCounter32(&m.succ->head, true) : ldLds32(kLdsHead + m.succW);
      } while (!reached(m.succHead, need));
    }
  } else if (agent ? !waitGeq(a, &m.succ->head, need, true) : !waitLdsGeq(a, kLdsHead + m.succW, need)) {
    return false;
  }
  acquireEdge();
  return true;
}

__device__ __forceinline__ void advanceSend(const KernelArgs& a, Member& m) {
  ++m.sendStep;
  if (++m.sendSlot == (u32)a.nSlots) m.sendSlot = 0;
}
template <bool XWG>
__device__ __forceinline__ void finishRecv(const KernelArgs& a, Member& m) {
  ++m.recvStep;
  if (XWG && m.recvAgent) {
    if (m.lane == 0) stCounterRelease(&m.self->head, m.recvStep, true);
  } else {
    stLds32Release(kLdsHead + m.selfW, (u32)m.recvStep);
  }
  if (++m.recvSlot == (u32)a.nSlots) m.recvSlot = 0;
}

// One FIFO step of kind KIND (kKindAtRunTime: of kind `kindRt`); `valid`
// payload bytes start at inp / outp (and at
// succOutp in the successor's output, for a direct all-gather step).
// LINES: every edge of the launch is inside one workgroup, so an LL128
// receive reads flags and payload in one poll (pollLL128Lines); kernels with
// edges between workgroups keep the two-phase read, which needs fewer
// registers (their grids must be co-resident).
// LDSQ (Simple): the FIFO slots of the edges inside the workgroup are in
// LDS (an edge between workgroups keeps its device FIFO); the all-gather
// goes through them too (never direct), so each member writes its own
// output once and reads nothing back.
template <int PROTO, int DT, int OP, int U, bool XWG, int KIND, bool LINES = false, bool LDSQ = false>
__device__ __forceinline__ bool step(const KernelArgs& a, Member& m, int kindRt, const char* inp, char* outp,
                                     char* succOutp, long valid) {
  constexpr int ESZ = DT == arUint64 ? 8 : (DT == arFloat16 || DT == arBfloat16) ? 2 : 4;
  constexpr int SLOT = PROTO == kSimple ? U * kWave * 16 : PROTO == kLL ? kLLSlotBytes : U * kLL128UnitBytes;
  const int kind = KIND != kKindAtRunTime ? KIND : kindRt;
  const bool hasLocal = (kind & kLocalBit) != 0;
  const bool hasRecv = (kind & kRecvBit) != 0;
  const bool hasSend = (kind & kSendBit) != 0;
  const bool hasOut = (kind & kOutBit) != 0;
  // Direct all-gather (Simple): the member that finishes a chunk and every
  // member forwarding it write the successor's output buffer instead of its
  // FIFO, so the all-gather half moves no FIFO bytes; the receiver then
  // reads the finished chunk from its own output.  [The pages' FIFO slot
  // descriptor can carry a pointer, and a work item can be flagged direct.]
  // An edge between workgroups always goes through the FIFO (both of its
  // ends see the same sendAgent / recvAgent, so they agree on it).
  const bool directSend = PROTO == kSimple && !LDSQ && m.direct && !(XWG && m.sendAgent) && hasSend && hasOut;
  const bool directRecv = PROTO == kSimple && !LDSQ && m.direct && !(XWG && m.recvAgent) && hasRecv && hasOut &&
                          !hasLocal;
  const int lane = m.lane;

  // piece geometry of this lane: payload offset, payload bytes, wire offset
  int payOff[U], payBytes[U], wireOff[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (PROTO == kSimple) {
      payOff[u] = (u * kWave + lane) * 16; payBytes[u] = 16; wireOff[u] = payOff[u];
    } else if (PROTO == kLL) {
      payOff[u] = (u * kWave + lane) * 8; payBytes[u] = 8; wireOff[u] = (u * kWave + lane) * 16;
    } else {
      const int line = lane >> 3, j = lane & 7;
      payOff[u] = u * kLL128UnitPayload + (j < 7 ? (line * 7 + j) * 16 : 896 + line * 8);
      payBytes[u] = j < 7 ? 16 : 8;
      wireOff[u] = u * kLL128UnitBytes + lane * 16;
    }
  }

  // EARLY: the local operand depends on no flag, so start its loads before
  // the credit wait and keep the last credit read.  Measured on 8 ranks: LL
  // steps 7% shorter; the 8 KiB Simple slot 0.5% faster at 256 MiB per rank
  // (104 VGPRs, no spill); LL128 steps longer (its 1 KiB units hold more
  // registers across the wait) and small Simple slots 3% slower on short
  // messages, so those keep the plain order.
  constexpr bool EARLY = PROTO == kLL || (PROTO == kSimple && U == 8);
  // LEAN: LDS-FIFO kernels with slots of at most 2 KiB, whose steps are short
  // enough for a few instructions to show (the plans of latency-bound sizes):
  // they keep the last credit read, and move whole LDS slots.  Measured on
  // the 4 KiB headline slot, the same changes cost 2%; it keeps the others.
  constexpr bool LEAN = LDSQ && U <= 2;
  if (!EARLY && hasSend && !directSend && !waitCredit<LEAN, XWG>(a, m)) return false;

  v4u v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    v[u] = hasLocal ? loadUser<ESZ, true>(inp + payOff[u], valid - payOff[u], payBytes[u], m.aligned)
                    : v4u{0u, 0u, 0u, 0u};
  }
  if (EARLY && hasSend && !directSend && !waitCredit<true, XWG>(a, m)) return false;

  if (hasRecv) {
    const char* slot = m.rfifo + (size_t)m.recvSlot * SLOT;
    v4u in[U];
    if (PROTO == kSimple) {
      if ((XWG && m.recvAgent) ? !waitGeq(a, &m.self->tail, m.recvStep + 1, true)
                               : !waitLdsGeq(a, m.selfW, m.recvStep + 1))
        return false;
      acquireEdge();
      const char* ls = ldsFifoBase + ((size_t)m.selfW * (size_t)a.nSlots + m.recvSlot) * SLOT;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (LEAN && !(XWG && m.recvAgent))   // past the payload: stale, never stored
          in[u] = *(const v4u*)(ls + wireOff[u]);
        else if (LDSQ && !(XWG && m.recvAgent))
          in[u] = payOff[u] < valid ? *(const v4u*)(ls + wireOff[u]) : v4u{0u, 0u, 0u, 0u};
        else if (directRecv)   // the predecessor wrote it into my output
          in[u] = kind == kRecvCopySend
                      ? loadUser<ESZ, false>(outp + payOff[u], valid - payOff[u], 16, m.aligned)
                      : v4u{0u, 0u, 0u, 0u};
        else
          in[u] = payOff[u] < valid ? ((XWG && m.recvAgent) ? ldCoh16(slot + wireOff[u]) : *(const v4u*)(slot + wireOff[u]))
                                    : v4u{0u, 0u, 0u, 0u};
      }
    } else if (PROTO == kLL) {
      if (!pollLL<U>(a, slot, wireOff, payOff, valid, (u32)(m.recvStep + 1), XWG && m.recvAgent, in)) return false;
    } else if (LINES) {   // LL128, every edge inside the workgroup: flags and payload in one poll
      if (!pollLL128Lines<U>(a, slot, wireOff, lane, valid, m.recvStep + 1, in)) return false;
    } else {  // LL128: poll the flag of every live line, then read payload
      if (!pollLL128Flags<U>(a, slot, wireOff, lane, valid, m.recvStep + 1, XWG && m.recvAgent)) return false;
      acquireEdge();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        in[u] = v4u{0u, 0u, 0u, 0u};
        if (u * kLL128UnitPayload < valid) {
          if (payBytes[u] == 16) {
            in[u] = (XWG && m.recvAgent) ? ldCoh16(slot + wireOff[u]) : *(const v4u*)(slot + wireOff[u]);
          } else {
            v2u t = (XWG && m.recvAgent) ? ldCoh8(slot + wireOff[u]) : *(const v2u*)(slot + wireOff[u]);
            in[u].x = t.x; in[u].y = t.y;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = hasLocal ? combine<DT, OP>(in[u], v[u]) : in[u];
  }

  // A Simple send across workgroups waits for its payload stores to complete
  // before publishing them, and gfx9 counts stores and loads on one counter,
  // so there the output store comes after the send (nothing downstream waits
  // for it) instead of being waited for too.  Elsewhere it comes first: LL128
  // rings cut into workgroups measured 8% slower with it last.
  constexpr bool OUT_LAST = PROTO == kSimple && XWG;
  if (!OUT_LAST && hasOut && !directRecv) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      storeUser<ESZ, true>(outp + payOff[u], v[u], valid - payOff[u], payBytes[u], m.aligned);
  }

  if (hasSend) {
    char* slot = m.sfifo + (size_t)m.sendSlot * SLOT;
    if (PROTO == kSimple) {
      if (directSend) {
        // the successor reads this back at its next stage: keep it cacheable
#pragma unroll
        for (int u = 0; u < U; ++u)
          storeUser<ESZ, false>(succOutp + payOff[u], v[u], valid - payOff[u], 16, m.aligned);
      } else if (LDSQ && !(XWG && m.sendAgent)) {
        // LEAN: the whole slot (lanes past the payload carry values no one stores)
        char* ls = ldsFifoBase + ((size_t)m.succW * (size_t)a.nSlots + m.sendSlot) * SLOT;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (LEAN || payOff[u] < valid) *(v4u*)(ls + wireOff[u]) = v[u];
      } else if ((XWG && m.sendAgent)) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (payOff[u] < valid) stCoh16(slot + wireOff[u], v[u]);
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (payOff[u] < valid) *(v4u*)(slot + wireOff[u]) = v[u];
      }
      releaseEdge((XWG && m.sendAgent));
      if (XWG && m.sendAgent) {
        if (lane == 0) stRelaxed64(&m.succ->tail, m.sendStep + 1, true);
      } else {
        stLds32(m.succW, (u32)m.sendStep + 1u);
      }
    } else if (PROTO == kLL) {
      const u64 flag = (u64)(u32)(m.sendStep + 1) << 32;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (payOff[u] < valid) {
          u64* line = (u64*)(slot + wireOff[u]);
          stRelaxed64(line, flag | v[u].x, (XWG && m.sendAgent));
          stRelaxed64(line + 1, flag | v[u].y, (XWG && m.sendAgent));
        }
      }
    } else {  // LL128: payload, release, then the flag word of each live line
      const bool flagLane = (lane & 7) == 7;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (u * kLL128UnitPayload < valid) {
          if (payBytes[u] == 16) {
            if ((XWG && m.sendAgent)) stCoh16(slot + wireOff[u], v[u]);
            else *(v4u*)(slot + wireOff[u]) = v[u];
          } else {
            v2u t; t.x = v[u].x; t.y = v[u].y;
            if ((XWG && m.sendAgent)) stCoh8(slot + wireOff[u], t);
            else *(v2u*)(slot + wireOff[u]) = t;
          }
        }
      }
      releaseEdge((XWG && m.sendAgent));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (flagLane && u * kLL128UnitPayload < valid)
          stRelaxed64((u64*)(slot + wireOff[u] + 8), m.sendStep + 1, (XWG && m.sendAgent));
    }
    advanceSend(a, m);
  }

  if (OUT_LAST && hasOut && !directRecv) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      storeUser<ESZ, true>(outp + payOff[u], v[u], valid - payOff[u], payBytes[u], m.aligned);
  }

  if (hasRecv) finishRecv<XWG>(a, m);
  return true;
}

// One collective of the ring schedule over one member's (channel, lane)
// share of `count` elements per rank; false when a wait gave up.
template <int PROTO, int DT, int OP, int U, int COLL, bool XWG, bool SPEC, bool LINES, bool LDSQ>
__device__ __forceinline__ bool ringPass(const KernelArgs& a, Member& m, int r, int ch, int k, u64 count,
                                         const char* in, char* out, char* succOut) {
  constexpr int ESZ = DT == arUint64 ? 8 : (DT == arFloat16 || DT == arBfloat16) ? 2 : 4;
  constexpr u64 A = 16 / ESZ;   // 16-byte grain in elements
  constexpr int PAYLOAD = PROTO == kSimple ? U * kWave * 16
                        : PROTO == kLL ? kLLSlotPayload : U * kLL128UnitPayload;
  const int N = a.nranks;
  if (N < 2) return true;   // one rank never launches a kernel: its result is a copy
  const int succ = r + 1 == N ? 0 : r + 1;
  // channel share [pages: contiguous split per channel, 16-byte grain]
  const u64 per = alignUp(divUp(count, (u64)a.nChannels), A);
  const u64 lo = umin((u64)ch * per, count);
  const u64 hi = umin(lo + per, count);
  const u64 len = hi - lo;
  if (len == 0) return true;

  const u64 C = a.chunkElems;
  const u64 loopSize = (u64)N * C;
  const int lastSendStage = 2 * N - 3;

  // Pipelining.  A member's share of a chunk is cut into slot-sized
  // columns; a batch of at most nSlots/2 columns goes through all 2N-1 stages
  // before the next batch starts (the pages size a chunk to half the FIFO for
  // the same reason).  A member then never has more than nSlots/2 sends that
  // its successor has not matched with receives, so no FIFO can fill up
  // around the whole ring and the pipeline cannot deadlock, whatever the
  // chunk size.  The order in which ranks are folded into an element is that
  // of the stage schedule and does not depend on the batching.
  const u64 batch = (u64)(a.nSlots / 2 > 0 ? a.nSlots / 2 : 1);
  if (COLL == kCollAllReduce) {
    for (u64 off = 0; off < len; off += loopSize) {
      const u64 rem = len - off;
      // shrunk chunk on the last partial loop [pages: getNextSendAddr]
      const u64 cur = rem < loopSize ? alignUp(divUp(rem, (u64)N), A) : C;
      // no lane share of any chunk in this loop exceeds sub0 (chunk 0 is the
      // longest chunk and a share is at most the per-lane split of its chunk)
      const u64 sub0 = alignUp(divUp(umin(cur, rem), (u64)a.lanes), A);
      const u64 nCols = divUp(sub0 * ESZ, (u64)PAYLOAD);
      // a whole chunk's lane share, so that only a shortened chunk divides
      const u64 subCur = alignUp(divUp(cur, (u64)a.lanes), A);
      // chunks [0, cWhole) hold `cur` elements each (all N on a full loop):
      // their lane shares have one length, and chunk c's starts c * cur
      // elements after chunk 0's, so a stage over one of them needs no
      // multiply-and-clamp of its own (kernels with LDS FIFOs, whose steps
      // are short enough for it to matter; the others keep their registers)
      const int cWhole = !LDSQ ? 0 : rem >= loopSize ? N : (int)(rem / cur);
      const u64 sbWhole = umin((u64)k * subCur, cur);
      const u64 bytesWhole = (umin(sbWhole + subCur, cur) - sbWhole) * ESZ;
      const u64 firstWhole = (lo + off + sbWhole) * ESZ;
      const u64 curBytes = cur * ESZ;
      for (u64 jb = 0; jb < nCols; jb += batch) {
        const u64 je = umin(jb + batch, nCols);
        int cNext = r == 0 ? N - 1 : r - 1;   // (r - 1 - s) mod N, stepped down each stage
        // stage s of this batch, of kind KIND
        auto stage = [&](int s, auto kindTag, int kindRt) -> bool {
          constexpr int KIND = decltype(kindTag)::value;
          // chunk sent at stage s is (r - 1 - s) mod N; the final receive gets r + 1
          const int c = s <= lastSendStage ? cNext : succ;
          cNext = cNext == 0 ? N - 1 : cNext - 1;
          u64 bytes, first;
          if (LDSQ && c < cWhole) {
            bytes = bytesWhole;
            first = firstWhole + (u64)(u32)c * curBytes;
          } else {
            const u64 cb = (u64)c * cur;
            const u64 clen = cb < rem ? umin(cur, rem - cb) : 0;
            // lane k's share of the chunk (pipelining only: the order is per element)
            const u64 sub = clen == cur ? subCur : alignUp(divUp(clen, (u64)a.lanes), A);
            const u64 sb = umin((u64)k * sub, clen);
            const u64 se = umin(sb + sub, clen);
            bytes = (se - sb) * ESZ;
            first = (lo + off + cb + sb) * ESZ;
          }
          if constexpr (LDSQ && U <= 2) {   // a lane's share of one chunk is at most a chunk: 32 bits
            const u32 bytes32 = (u32)bytes;
            for (u32 j = (u32)jb; j < (u32)je; ++j) {
              const u32 b = j * (u32)PAYLOAD;
              if (b >= bytes32) break;
              const long valid = (long)(bytes32 - b < (u32)PAYLOAD ? bytes32 - b : (u32)PAYLOAD);
              if (!step<PROTO, DT, OP, U, XWG, KIND, LINES, LDSQ>(a, m, kindRt, in + first + b, out + first + b,
                                                            succOut + first + b, valid))
                return false;
            }
          } else {
            for (u64 j = jb; j < je; ++j) {
              const u64 b = j * (u64)PAYLOAD;
              if (b >= bytes) break;
              const long valid = (long)umin((u64)PAYLOAD, bytes - b);
              if (!step<PROTO, DT, OP, U, XWG, KIND, LINES, LDSQ>(a, m, kindRt, in + first + b, out + first + b,
                                                            succOut + first + b, valid))
                return false;
            }
          }
          return true;
        };
        // send | recv-reduce-send x (N-2) | recv-reduce-copy-send |
        // recv-copy-send x (N-2) | recv
        if constexpr (SPEC) {
          if (!stage(0, KindTag<kSend>{}, 0)) return false;
          for (int s = 1; s < N - 1; ++s)
            if (!stage(s, KindTag<kRecvReduceSend>{}, 0)) return false;
          if (!stage(N - 1, KindTag<kRecvReduceCopySend>{}, 0)) return false;
          for (int s = N; s <= lastSendStage; ++s)
            if (!stage(s, KindTag<kRecvCopySend>{}, 0)) return false;
          if (!stage(2 * N - 2, KindTag<kRecv>{}, 0)) return false;
        } else {
          for (int s = 0; s <= 2 * N - 2; ++s) {
            const int kind = s == 0 ? kSend : s < N - 1 ? kRecvReduceSend : s == N - 1 ? kRecvReduceCopySend
                             : s <= lastSendStage ? kRecvCopySend : kRecv;
            if (!stage(s, KindTag<kKindAtRunTime>{}, kind)) return false;
          }
        }
      }
    }
  } else {
    // ReduceScatter / AllGather, the two halves of the ring on their own
    // [pages: nSteps = nRanks-1 for them].  Every stage works on the same
    // element range of a different rank block (block = `count` elements):
    //   ReduceScatter: send | recv-reduce-send x (N-2) | recv-reduce-copy, on
    //                  block (r - 1 - s) mod N, so block b ends at its owner b;
    //   AllGather:     copy-send | recv-copy-send x (N-2) | recv, on block
    //                  (r - s) mod N, so block b starts at its owner b.
    constexpr bool rs = COLL == kCollReduceScatter;
    const u64 blk = count * ESZ;
    for (u64 off = 0; off < len; off += C) {
      const u64 cur = umin(C, len - off);
      const u64 sub = alignUp(divUp(cur, (u64)a.lanes), A);
      const u64 sb = umin((u64)k * sub, cur);
      const u64 se = umin(sb + sub, cur);
      const u64 bytes = (se - sb) * ESZ;
      const u64 first = (lo + off + sb) * ESZ;   // byte offset inside a block
      const u64 nCols = divUp(bytes, (u64)PAYLOAD);
      for (u64 jb = 0; jb < nCols; jb += batch) {
        const u64 je = umin(jb + batch, nCols);
        auto stage = [&](int s, auto kindTag, int kindRt) -> bool {
          constexpr int KIND = decltype(kindTag)::value;
          const int blkIdx = rs ? (r - 1 - s + 2 * N) % N : (r - s + N) % N;
          // ReduceScatter reads block b of its input and writes its one
          // output block; AllGather reads its one input block and writes block b
          const u64 inOff = rs ? (u64)blkIdx * blk + first : first;
          const u64 outOff = rs ? first : (u64)blkIdx * blk + first;
          for (u64 j = jb; j < je; ++j) {
            const u64 b = j * (u64)PAYLOAD;
            const long valid = (long)umin((u64)PAYLOAD, bytes - b);
            if (!step<PROTO, DT, OP, U, XWG, KIND, LINES, LDSQ>(a, m, kindRt, in + inOff + b, out + outOff + b,
                                                          succOut + outOff + b, valid))
              return false;
          }
          return true;
        };
        if constexpr (SPEC && rs) {
          if (!stage(0, KindTag<kSend>{}, 0)) return false;
          for (int s = 1; s < N - 1; ++s)
            if (!stage(s, KindTag<kRecvReduceSend>{}, 0)) return false;
          if (!stage(N - 1, KindTag<kRecvReduceCopy>{}, 0)) return false;
        } else if constexpr (SPEC) {
          if (!stage(0, KindTag<kCopySend>{}, 0)) return false;
          for (int s = 1; s < N - 1; ++s)
            if (!stage(s, KindTag<kRecvCopySend>{}, 0)) return false;
          if (!stage(N - 1, KindTag<kRecv>{}, 0)) return false;
        } else {
          for (int s = 0; s <= N - 1; ++s) {
            const int kind = rs ? (s == 0 ? kSend : s < N - 1 ? kRecvReduceSend : kRecvReduceCopy)
                                : (s == 0 ? kCopySend : s < N - 1 ? kRecvCopySend : kRecv);
            if (!stage(s, KindTag<kKindAtRunTime>{}, kind)) return false;
          }
        }
      }
    }
  }
  return true;
}

// Every pass of one member: the (channel, lane) pairs of its FIFO set, or
// the tasks of a batched launch; false when a wait gave up.
template <int PROTO, int DT, int OP, int U, int COLL, bool BATCH, bool XWG, bool SPEC, bool LINES, bool LDSQ = false>
__device__ __forceinline__ bool memberPasses(const KernelArgs& a, Member& m, int L, int sets, int lanesTotal,
                                             int perTask, int r, int succ) {
  if (!BATCH) {
    for (int Lp = L; Lp < lanesTotal; Lp += sets) {
      if (!ringPass<PROTO, DT, OP, U, COLL, XWG, SPEC, LINES, LDSQ>(a, m, r, Lp / a.lanes, Lp % a.lanes, a.count,
                                                 (const char*)a.send[r], (char*)a.recv[r], (char*)a.recv[succ]))
        return false;
    }
    return true;
  }
  const int N = a.nranks;
  const int Lc = L % perTask;   // (channel, lane) inside the task
  const int ch = Lc / a.lanes;
  const int k = Lc % a.lanes;
  const size_t row = 1 + 2 * (size_t)N;
  for (int t = L / perTask; t < a.nTasks; t += a.taskSlots) {
    const u64* d = a.tasks + (size_t)t * row;
    if (!ringPass<PROTO, DT, OP, U, COLL, XWG, SPEC, LINES, LDSQ>(a, m, r, ch, k, d[0], (const char*)d[1 + r], (char*)d[1 + N + r],
                                               (char*)d[1 + N + succ]))
      return false;
  }
  return true;
}

// BATCH: the launch runs the a.nTasks AllReduces of one aggregate, each
// described by a row of a.tasks {count, send[N], recv[N]}.  a.taskSlots of
// them run at once, each on its own nChannels x lanes wavefront sets (and
// FIFOs); a set takes tasks slot, slot + taskSlots, ... in turn, so its FIFO
// steps simply continue from one task to the next.
//
// ONEWG: every ring of the launch lies inside one workgroup (the host picks
// this instantiation for such plans only), so no edge crosses workgroups; the
// Simple kernels of slots up to 4 KiB then also compile every step for its
// kind (8 ranks x 4 KiB: 19.5 -> 15.2 us; 16 x 4 KiB: 45.6 -> 34.2 us).  Not
// for 8 KiB slots, where the per-kind copies spill.  Rings cut into
// workgroups compile their steps per kind when their FIFO slots are in LDS
// (LDSQ): with the kind known, a copy step's LDS handoff no longer waits on
// the vector memory counter for a local load that kind never issues -- which
// on gfx9 meant waiting for the previous step's output store to complete --
// so the chain of hops inside a workgroup runs at LDS speed (72 ranks x
// 4 MiB: 391 -> 325 us; 128 x 1 MiB: 595 -> 487 us; 24 x 4 KiB: 92 -> 72 us,
// with the output store after the send on edges between workgroups).
// Those with HBM FIFOs keep one step for every kind: there the extra
// registers of the copies cost residency.
//
// PERKIND (with ONEWG): compile each step for its kind.  LL and LL128 get it
// too (8 ranks x 4 KiB: LL 24.0 -> 18.6 us, LL128 26.9 -> 20.4 us), but the
// copies raise LL128's registers from 80 to 91 (6 -> 5 wavefronts per SIMD),
// which costs a grid of several resident rounds (8 x 256 MiB: 2.34 -> 2.47
// ms), so the host picks it for LL128 only when the grid is one workgroup per
// CU at most.
//
// LDSQ (Simple; a ring cut into workgroups only in single calls): the FIFO
// slots of the edges inside a workgroup are in LDS (the launch gives members x nSlots x slot bytes of
// dynamic LDS).  With ONEWG too, every counter starts at step 0 and nothing
// is published when the call ends: no state of these edges outlives the
// workgroup, and the comm's device FIFOs and counters are not touched (they
// keep tail == head for whatever ran before or runs after).  A ring cut into
// workgroups keeps the usual carried counters (its edges between workgroups
// need them); only the slots of the edges inside a group move.
template <int PROTO, int DT, int OP, int U, int COLL, bool BATCH, bool ONEWG, bool PERKIND = ONEWG, bool LDSQ = false>
__global__ void __launch_bounds__(1024) ringAllReduceKernel(const KernelArgs a) {
  static_assert(!LDSQ || PROTO == kSimple, "LDS FIFOs: Simple");
  constexpr bool FRESH = LDSQ && ONEWG;   // no counter carries over
  // The 8 KiB slot kernels read the wavefront index through readfirstlane,
  // so every per-member value (pointers, counters, rank, channel) lives in
  // scalar registers: that keeps them at 101-120 VGPRs instead of spilling.
  // Smaller slots keep the plain index: with their register room, per-member
  // state in VGPRs measured faster on short messages (the CU's scalar unit
  // is shared by all of its wavefronts' polling loops).
  const int wave = (U == 8 || LDSQ) ? (int)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave) : (int)(threadIdx.x / kWave);
  __builtin_amdgcn_s_setprio(kWorkPrio);
  const int N = a.nranks;
  const int perTask = a.nChannels * a.lanes;
  const int lanesTotal = BATCH ? perTask * a.taskSlots : perTask;

  int L, g;   // FIFO set and group
  laneAndGroup(a, L, g);
  // A single call's workgroups may be fewer than its (channel, lane) pairs:
  // set L then runs pairs L, L + sets, L + 2 sets, ... on the same FIFOs,
  // whose steps simply continue from one pair to the next.
  const int sets = BATCH ? lanesTotal : a.laneSets;
  const int r = g * a.groupSize + wave;
  // every wavefront reaches the barrier below before any returns
  const bool live = L < sets && r < N;
  const int succ = r + 1 >= N ? 0 : r + 1;
  const int pred = r == 0 ? N - 1 : r - 1;

  Member m;
  m.lane = threadIdx.x % kWave;
  const size_t wSelf = (size_t)L * N + r, wSucc = (size_t)L * N + succ;
  m.rfifo = a.fifo + wSelf * a.fifoWorkerBytes;
  m.sfifo = a.fifo + wSucc * a.fifoWorkerBytes;
  m.self = a.conn + wSelf;
  m.succ = a.conn + wSucc;
  // The 8 KiB Simple kernel serves single-workgroup rings only (the host
  // never plans it for a ring cut into groups), so it carries no code for
  // edges between workgroups.
  constexpr bool GROUPED = !ONEWG && (PROTO != kSimple || U <= kGroupedSimpleUnrollMax);
  constexpr bool SPEC = ONEWG && PERKIND && (PROTO != kSimple || U <= kGroupedSimpleUnrollMax);
  constexpr bool LINES = ONEWG && PROTO == kLL128;
  m.recvAgent = GROUPED && pred / a.groupSize != g;
  m.sendAgent = GROUPED && succ / a.groupSize != g;
  m.selfW = wave;
  m.succW = succ - g * a.groupSize;   // used only when the successor shares the workgroup
  m.aligned = a.aligned16 != 0;
  m.direct = !LDSQ && a.direct != 0;
  // counters carry over from earlier calls (tail == head at call boundaries,
  // unless a member of an earlier call gave up: then nothing runs); with
  // freshSteps or LDS FIFOs every edge is in LDS and starts at step 0 instead
  const bool carry = live && a.freshSteps == 0 && !FRESH;
  const u32 failed = (FRESH ? live : carry) ? callFailed(a) : 0u;
  m.recvStep = carry ? ldCounter(&m.self->head, true) : 0;
  m.sendStep = carry ? ldCounter(&m.succ->tail, true) : 0;
  m.succHead = (u32)m.sendStep;   // at a call boundary the successor has consumed all we sent
  m.recvSlot = (u32)(m.recvStep % (u64)a.nSlots);
  m.sendSlot = (u32)(m.sendStep % (u64)a.nSlots);
  if (live && m.lane == 0) {
    stLds(wave, m.recvStep);
    stLds(kLdsHead + wave, m.recvStep);
  }
  __syncthreads();
  if (!live || r == a.deadRank || failed != 0) return;

  // A member with an edge to another workgroup runs the pass compiled with
  // that edge's code; every other member runs one with no trace of it (the
  // runtime checks alone cost short messages a few percent).
  bool ok;
  if constexpr (GROUPED) {
    ok = m.sendAgent || m.recvAgent
             ? memberPasses<PROTO, DT, OP, U, COLL, BATCH, true, LDSQ, false, LDSQ>(a, m, L, sets, lanesTotal, perTask, r,
                                                                              succ)
             : memberPasses<PROTO, DT, OP, U, COLL, BATCH, false, LDSQ, false, LDSQ>(a, m, L, sets, lanesTotal, perTask,
                                                                               r, succ);
  } else {
    ok = memberPasses<PROTO, DT, OP, U, COLL, BATCH, false, SPEC, LINES, LDSQ>(a, m, L, sets, lanesTotal, perTask, r,
                                                                             succ);
  }
  if (!ok) return;
  // Publish what only LDS (an edge inside the workgroup) or the LL / LL128
  // flags (which never touch the tail counter per slot) have counted, so the
  // next call starts both ends of every FIFO at the same step.
  if (m.lane == 0 && a.freshSteps == 0 && !FRESH) {
    if (!(GROUPED && m.recvAgent)) stRelaxed64(&m.self->head, m.recvStep, true);
    if (PROTO != kSimple || !(GROUPED && m.sendAgent)) stRelaxed64(&m.succ->tail, m.sendStep, true);
  }
}

// ------------------------------------------------------------- tree AllReduce
//
// The pages' second algorithm ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程",
// ch.4 "Ring 與 Tree：把搜尋結果變成演算法拓撲", ncclGetBtree / ncclGetDtree;
// "NCCL Tree拓扑介绍", single and double binary trees].  Each virtual rank is
// a tree node and, as in the ring, one wavefront per (rank, channel, lane).
// Reduce: a node folds the partials its children send (d0 first, then d1)
// and then its own value, OP(OP(p_d0, p_d1), x), and sends the result to its
// parent; the root's result is the answer, which it writes and sends back
// down; every other node receives it from its parent, writes it and forwards
// it to its children.  The first half of the channels runs on the first
// tree, the second half on the second (mirrored for an even rank count,
// shifted by one rank for an odd one).
//
// FIFOs: a node owns three, one per incoming edge (from d0, from d1, from its
// parent), at worker index (lane * N + rank) * 3 + edge, with the same slot
// and counter layout as the ring's.  A member works through its lane share
// in batches of nSlots columns: the reduce pass of a batch, then its
// broadcast pass.  A member starts batch b+1 only after its broadcast pass of
// batch b, which needs data its parent sent after consuming the member's
// batch-b columns and, in turn, after its children consumed its batch-b
// broadcast; so no edge ever holds more than one batch and neither pass can
// wait on the other: the tree cannot deadlock for any size.

// Binary tree over ranks [pages: ncclGetBtree]: with `bit` the lowest set
// bit of r (for the root r = 0, the first power of two >= n), the parent
// clears `bit` and sets the next bit up (or only clears it, if that is out
// of range); the children are r - bit/2 and r + h for the largest power of
// two h <= bit/2 with r + h < n.  The root's only child is bit/2, named d1.
__device__ __forceinline__ void btreeNode(int n, int r, int& up, int& d0, int& d1) {
  up = d0 = d1 = -1;
  if (r == 0) {
    if (n > 1) d1 = (int)((1u << (32 - __builtin_clz((u32)n - 1u))) >> 1);   // bit_ceil(n) / 2
    return;
  }
  const int bit = r & -r;
  up = (r & ~bit) | (bit << 1);
  if (up >= n) up = r & ~bit;
  const int h = bit >> 1;
  if (h == 0) return;
  d0 = r - h;
  const int room = n - 1 - r;   // r + h' < n  <=>  h' <= room
  if (room >= 1) d1 = r + (int)(1u << (31 - __builtin_clz((u32)(h < room ? h : room))));   // bit_floor
}

// Tree t of the double tree [pages: ncclGetDtree]: tree 1 relabels rank x as
// n-1-x (even n) or x-1 (odd n), takes the binary tree of the relabelled
// rank and maps every peer back.
__device__ __forceinline__ void dtreeNode(int n, int r, int t, int& up, int& d0, int& d1) {
  if (t == 0) {
    btreeNode(n, r, up, d0, d1);
    return;
  }
  const bool mirror = (n & 1) == 0;
  btreeNode(n, mirror ? n - 1 - r : (r == 0 ? n - 1 : r - 1), up, d0, d1);
  auto back = [&](int x) { return x < 0 ? -1 : mirror ? n - 1 - x : (x + 1 == n ? 0 : x + 1); };
  up = back(up);
  d0 = back(d0);
  d1 = back(d1);
}

// One end of one FIFO.
struct Edge {
  char* fifo;   // slot 0 (the FIFO is owned by the receiving end)
  Conn* conn;   // its counters
  u64 step;     // next step on this FIFO
  u32 slot;     // step % nSlots
  bool agent;   // the other end is in another workgroup
  int lds;      // LDS FIFOs: the FIFO's index in the workgroup's LDS (-1: device memory)
};

// A tree inside one workgroup with its FIFOs in LDS: every node but the root
// has one FIFO up to its parent (index 2r) and one down from it (2r + 1),
// nSlots slots each in the dynamic LDS, tail and head counters in
// treeLdsCounters (2 per FIFO, at most 16 nodes).
__device__ __forceinline__ u64* treeLdsCounters() {
  __shared__ u64 c[2 * 2 * kMaxMembersPerGroup];
  return c;
}
__device__ __forceinline__ u32 ldTreeLds32(int i) {
  const u32 v = __hip_atomic_load((u32*)&treeLdsCounters()[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ bool waitTreeLdsGeq(const KernelArgs& a, int i, u64 target) {
  const u32 t = (u32)target;
  if (reached(ldTreeLds32(i), t)) return true;
  Waiter w;
  while (true) {
    if (!keepWaiting(a, w)) return false;
    if (reached(ldTreeLds32(i), t)) return true;
  }
}
__device__ __forceinline__ Edge openLdsEdge(int fifoIndex) {
  Edge e;
  e.fifo = nullptr;
  e.conn = nullptr;
  e.step = 0;
  e.slot = 0;
  e.agent = false;
  e.lds = fifoIndex;
  return e;
}

__device__ __forceinline__ Edge openEdge(const KernelArgs& a, size_t worker, bool agent, bool recvEnd) {
  Edge e;
  e.fifo = a.fifo + worker * a.fifoWorkerBytes;
  e.conn = a.conn + worker;
  // counters carry over from earlier calls (tail == head at call boundaries)
  e.step = ldCounter(recvEnd ? &e.conn->head : &e.conn->tail, true);
  e.slot = (u32)(e.step % (u64)a.nSlots);
  e.agent = agent;
  e.lds = -1;
  return e;
}

template <int PROTO, int U>
struct Pieces {   // this lane's pieces of one slot (as in the ring's step)
  int payOff[U], payBytes[U], wireOff[U];
  __device__ __forceinline__ explicit Pieces(int lane) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (PROTO == kSimple) {
        payOff[u] = (u * kWave + lane) * 16; payBytes[u] = 16; wireOff[u] = payOff[u];
      } else if (PROTO == kLL) {
        payOff[u] = (u * kWave + lane) * 8; payBytes[u] = 8; wireOff[u] = (u * kWave + lane) * 16;
      } else {
        const int line = lane >> 3, j = lane & 7;
        payOff[u] = u * kLL128UnitPayload + (j < 7 ? (line * 7 + j) * 16 : 896 + line * 8);
        payBytes[u] = j < 7 ? 16 : 8;
        wireOff[u] = u * kLL128UnitBytes + lane * 16;
      }
    }
  }
};

template <int PROTO, int U, bool XWG, bool LINES = false, bool LDSQ = false>
__device__ __forceinline__ bool edgeRecv(const KernelArgs& a, const Edge& e, const Pieces<PROTO, U>& pc, int lane,
                                         long valid, v4u (&in)[U]) {
  constexpr int SLOT = PROTO == kSimple ? U * kWave * 16 : PROTO == kLL ? kLLSlotBytes : U * kLL128UnitBytes;
  // LDSQ: an edge inside the workgroup has its FIFO and counters in LDS
  // (every edge of a member compiled without edges between workgroups)
  if (LDSQ && (!XWG || e.lds >= 0)) {   // Simple
    if (!waitTreeLdsGeq(a, 2 * e.lds, e.step + 1)) return false;
    acquireEdge();
    const char* ls = ldsFifoBase + ((size_t)e.lds * (size_t)a.nSlots + e.slot) * SLOT;
    // slots of at most 2 KiB are moved whole, as in the ring (past the
    // payload: stale lanes that are never stored)
#pragma unroll
    for (int u = 0; u < U; ++u)
      in[u] = U <= 2 || pc.payOff[u] < valid ? *(const v4u*)(ls + pc.wireOff[u]) : v4u{0u, 0u, 0u, 0u};
    return true;
  }
  const char* slot = e.fifo + (size_t)e.slot * SLOT;
  if (PROTO == kSimple) {
    if (!waitGeq(a, &e.conn->tail, e.step + 1, (XWG && e.agent))) return false;
    acquireEdge();
#pragma unroll
    for (int u = 0; u < U; ++u)
      in[u] = pc.payOff[u] >= valid ? v4u{0u, 0u, 0u, 0u}
              : (XWG && e.agent)            ? ldCoh16(slot + pc.wireOff[u])
                                   : *(const v4u*)(slot + pc.wireOff[u]);
  } else if (PROTO == kLL) {
    if (!pollLL<U>(a, slot, pc.wireOff, pc.payOff, valid, (u32)(e.step + 1), XWG && e.agent, in)) return false;
  } else if (LINES) {   // LL128, every edge inside the workgroup: flags and payload in one poll
    if (!pollLL128Lines<U>(a, slot, pc.wireOff, lane, valid, e.step + 1, in)) return false;
  } else {
    if (!pollLL128Flags<U>(a, slot, pc.wireOff, lane, valid, e.step + 1, XWG && e.agent)) return false;
    acquireEdge();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      in[u] = v4u{0u, 0u, 0u, 0u};
      if (u * kLL128UnitPayload < valid) {
        if (pc.payBytes[u] == 16) {
          in[u] = (XWG && e.agent) ? ldCoh16(slot + pc.wireOff[u]) : *(const v4u*)(slot + pc.wireOff[u]);
        } else {
          const v2u t = (XWG && e.agent) ? ldCoh8(slot + pc.wireOff[u]) : *(const v2u*)(slot + pc.wireOff[u]);
          in[u].x = t.x; in[u].y = t.y;
        }
      }
    }
  }
  return true;
}

template <bool XWG, bool LDSQ = false>
__device__ __forceinline__ void edgeFinishRecv(const KernelArgs& a, Edge& e, int lane) {
  ++e.step;
  if (LDSQ && (!XWG || e.lds >= 0))   // the low word, by every lane (as the ring's LDS counters)
    __hip_atomic_store((u32*)&treeLdsCounters()[2 * e.lds + 1], (u32)e.step, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
  else if (lane == 0)
    stCounterRelease(&e.conn->head, e.step, (XWG && e.agent));
  if (++e.slot == (u32)a.nSlots) e.slot = 0;
}

template <int PROTO, int U, bool XWG, bool LDSQ = false>
__device__ __forceinline__ bool edgeSend(const KernelArgs& a, Edge& e, const Pieces<PROTO, U>& pc, int lane,
                                         long valid, const v4u (&v)[U]) {
  constexpr int SLOT = PROTO == kSimple ? U * kWave * 16 : PROTO == kLL ? kLLSlotBytes : U * kLL128UnitBytes;
  // slot step % nSlots is free once the receiver consumed step - nSlots
  // (modulo 2^32, as the ring's credit)
  const u32 need = (u32)e.step + 1u - (u32)a.nSlots;
  if (LDSQ && (!XWG || e.lds >= 0)) {   // Simple, FIFO and counters in LDS
    if (!waitTreeLdsGeq(a, 2 * e.lds + 1, need)) return false;
    acquireEdge();
    char* ls = ldsFifoBase + ((size_t)e.lds * (size_t)a.nSlots + e.slot) * SLOT;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (U <= 2 || pc.payOff[u] < valid) *(v4u*)(ls + pc.wireOff[u]) = v[u];
    releaseEdge(false);   // the LDS stores before the counter
    __hip_atomic_store((u32*)&treeLdsCounters()[2 * e.lds], (u32)e.step + 1u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
    ++e.step;
    if (++e.slot == (u32)a.nSlots) e.slot = 0;
    return true;
  }
  if (!waitGeq(a, &e.conn->head, need, (XWG && e.agent))) return false;
  acquireEdge();
  char* slot = e.fifo + (size_t)e.slot * SLOT;
  if (PROTO == kSimple) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (pc.payOff[u] < valid) {
        if ((XWG && e.agent)) stCoh16(slot + pc.wireOff[u], v[u]);
        else *(v4u*)(slot + pc.wireOff[u]) = v[u];
      }
    }
    releaseEdge((XWG && e.agent));
    if (lane == 0) stRelaxed64(&e.conn->tail, e.step + 1, (XWG && e.agent));
  } else if (PROTO == kLL) {
    const u64 flag = (u64)(u32)(e.step + 1) << 32;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (pc.payOff[u] < valid) {
        u64* line = (u64*)(slot + pc.wireOff[u]);
        stRelaxed64(line, flag | v[u].x, (XWG && e.agent));
        stRelaxed64(line + 1, flag | v[u].y, (XWG && e.agent));
      }
    }
  } else {
    const bool flagLane = (lane & 7) == 7;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u * kLL128UnitPayload < valid) {
        if (pc.payBytes[u] == 16) {
          if ((XWG && e.agent)) stCoh16(slot + pc.wireOff[u], v[u]);
          else *(v4u*)(slot + pc.wireOff[u]) = v[u];
        } else {
          v2u t; t.x = v[u].x; t.y = v[u].y;
          if ((XWG && e.agent)) stCoh8(slot + pc.wireOff[u], t);
          else *(v2u*)(slot + pc.wireOff[u]) = t;
        }
      }
    }
    releaseEdge((XWG && e.agent));
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (flagLane && u * kLL128UnitPayload < valid)
        stRelaxed64((u64*)(slot + pc.wireOff[u] + 8), e.step + 1, (XWG && e.agent));
  }
  ++e.step;
  if (++e.slot == (u32)a.nSlots) e.slot = 0;
  return true;
}

// A tree node's FIFO ends and peers (independent of the data).
struct TreeNode {
  int up, d[2];
  Edge fromChild[2], toChild[2], fromParent, toParent;
};

// One AllReduce over one member's (channel, lane) share of `count` elements
// per rank: batches of nSlots columns, each a reduce pass then (below the
// root) a broadcast pass; false when a wait gave up.
// A tree member's role as a constant: which of its peers exist, as bits
// kRoleD0 (child d0), kRoleD1 (child d1), kRoleParent.  A binary tree's root
// has d1 only; every other node with children has d0, and maybe d1.
// kRoleAtRunTime: read it from the node.
constexpr int kRoleD0 = 1, kRoleD1 = 2, kRoleParent = 4, kRoleAtRunTime = -1;
template <int PROTO, int DT, int OP, int U, bool XWG, int ROLE = kRoleAtRunTime, bool LINES = false,
          bool LDSQ = false>
__device__ __forceinline__ bool treePass(const KernelArgs& a, TreeNode& nd, int ch, int k, int lane, u64 count,
                                         const char* inBase, char* outBase) {
  constexpr int ESZ = DT == arUint64 ? 8 : (DT == arFloat16 || DT == arBfloat16) ? 2 : 4;
  constexpr u64 A = 16 / ESZ;
  constexpr int PAYLOAD = PROTO == kSimple ? U * kWave * 16
                        : PROTO == kLL ? kLLSlotPayload : U * kLL128UnitPayload;
  const u64 per = alignUp(divUp(count, (u64)a.nChannels), A);
  const u64 lo = umin((u64)ch * per, count);
  const u64 len = umin(lo + per, count) - lo;
  const u64 sub = alignUp(divUp(len, (u64)a.lanes), A);
  const u64 sb = umin((u64)k * sub, len);
  const u64 bytes = (umin(sb + sub, len) - sb) * ESZ;
  if (bytes == 0) return true;

  const bool leaf = ROLE != kRoleAtRunTime ? (ROLE & (kRoleD0 | kRoleD1)) == 0 : nd.d[0] < 0 && nd.d[1] < 0;
  const bool hasUp = ROLE != kRoleAtRunTime ? (ROLE & kRoleParent) != 0 : nd.up >= 0;
  auto hasChild = [&](int i) { return ROLE != kRoleAtRunTime ? ((ROLE >> i) & 1) != 0 : nd.d[i] >= 0; };
  const char* in = inBase + (lo + sb) * ESZ;
  char* out = outBase + (lo + sb) * ESZ;
  const bool aligned = a.aligned16 != 0;
  const Pieces<PROTO, U> pc(lane);
  const u64 nCols = divUp(bytes, (u64)PAYLOAD);
  const u64 batch = (u64)a.nSlots;
  v4u acc[U], x[U];
  for (u64 jb = 0; jb < nCols; jb += batch) {
    const u64 je = umin(jb + batch, nCols);
    // reduce pass: children's partials, then my own value; up (or, at the
    // root, straight into the broadcast)
    for (u64 j = jb; j < je; ++j) {
      const u64 b = j * (u64)PAYLOAD;
      const long valid = (long)umin((u64)PAYLOAD, bytes - b);
#pragma unroll
      for (int u = 0; u < U; ++u)
        x[u] = loadUser<ESZ, true>(in + b + pc.payOff[u], valid - pc.payOff[u], pc.payBytes[u], aligned);
      if (leaf) {
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = x[u];
      } else {
        bool have = false;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (!hasChild(i)) continue;
          v4u got[U];
          if (!edgeRecv<PROTO, U, XWG, LINES, LDSQ>(a, nd.fromChild[i], pc, lane, valid, got)) return false;
          edgeFinishRecv<XWG, LDSQ>(a, nd.fromChild[i], lane);
#pragma unroll
          for (int u = 0; u < U; ++u) acc[u] = have ? combine<DT, OP>(acc[u], got[u]) : got[u];
          have = true;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = combine<DT, OP>(acc[u], x[u]);
      }
      if (hasUp) {
        if (!edgeSend<PROTO, U, XWG, LDSQ>(a, nd.toParent, pc, lane, valid, acc)) return false;
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
          storeUser<ESZ, true>(out + b + pc.payOff[u], acc[u], valid - pc.payOff[u], pc.payBytes[u], aligned);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (hasChild(i) && !edgeSend<PROTO, U, XWG, LDSQ>(a, nd.toChild[i], pc, lane, valid, acc)) return false;
      }
    }
    if (!hasUp) continue;
    // broadcast pass: the result from the parent, to my output and children
    for (u64 j = jb; j < je; ++j) {
      const u64 b = j * (u64)PAYLOAD;
      const long valid = (long)umin((u64)PAYLOAD, bytes - b);
      if (!edgeRecv<PROTO, U, XWG, LINES, LDSQ>(a, nd.fromParent, pc, lane, valid, acc)) return false;
      edgeFinishRecv<XWG, LDSQ>(a, nd.fromParent, lane);
#pragma unroll
      for (int u = 0; u < U; ++u)
        storeUser<ESZ, true>(out + b + pc.payOff[u], acc[u], valid - pc.payOff[u], pc.payBytes[u], aligned);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (hasChild(i) && !edgeSend<PROTO, U, XWG, LDSQ>(a, nd.toChild[i], pc, lane, valid, acc)) return false;
    }
  }
  return true;
}

// Every pass of one tree member: its one call, or the tasks of a batched
// launch; false when a wait gave up.
template <int PROTO, int DT, int OP, int U, bool BATCH, bool XWG, int ROLE = kRoleAtRunTime, bool LINES = false,
          bool LDSQ = false>
__device__ __forceinline__ bool treePasses(const KernelArgs& a, TreeNode& nd, int L, int perTask, int ch, int k,
                                           int lane, int r) {
  if (!BATCH)
    return treePass<PROTO, DT, OP, U, XWG, ROLE, LINES, LDSQ>(a, nd, ch, k, lane, a.count, (const char*)a.send[r],
                                                             (char*)a.recv[r]);
  const int N = a.nranks;
  const size_t row = 1 + 2 * (size_t)N;
  for (int i = L / perTask; i < a.nTasks; i += a.taskSlots) {
    const u64* d = a.tasks + (size_t)i * row;
    if (!treePass<PROTO, DT, OP, U, XWG, ROLE, LINES, LDSQ>(a, nd, ch, k, lane, d[0], (const char*)d[1 + r],
                                                           (char*)d[1 + N + r]))
      return false;
  }
  return true;
}

// BATCH as for the ring kernel: a.nTasks AllReduces from a.tasks, a.taskSlots
// of them at once.
//
// ONEWG: every tree of the launch lies inside one workgroup (the host picks
// this instantiation for such plans only); the Simple kernels then also
// compile a member's pass for its role (parent or root, number of children).
//
// LDSQ (Simple, ONEWG): every FIFO of the tree and its counters are in LDS
// (the launch gives 2N x nSlots x slot bytes of dynamic LDS); the counters
// start at 0 in each launch and the comm's device FIFOs are not touched.
template <int PROTO, int DT, int OP, int U, bool BATCH, bool ONEWG, bool LDSQ = false>
__global__ void __launch_bounds__(1024) treeAllReduceKernel(const KernelArgs a) {
  static_assert(!LDSQ || (PROTO == kSimple && (ONEWG || !BATCH)), "LDS FIFOs: Simple trees (cut into groups: single calls)");
  // as in the ring kernel: scalar member state for the largest (4 KiB) slot
  const int wave = (U == 4 || LDSQ) ? (int)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave)
                                    : (int)(threadIdx.x / kWave);
  __builtin_amdgcn_s_setprio(kWorkPrio);
  const int lane = threadIdx.x % kWave;
  const int N = a.nranks;
  const int perTask = a.nChannels * a.lanes;
  const int lanesTotal = BATCH ? perTask * a.taskSlots : perTask;

  int L, g;   // (lane id, group), as in the ring kernel
  laneAndGroup(a, L, g);
  const int r = g * a.groupSize + wave;
  if constexpr (LDSQ) {   // every wavefront clears the counters and meets the others before any returns
    for (int i = (int)threadIdx.x; i < 4 * kMaxMembersPerGroup; i += (int)blockDim.x)
      __hip_atomic_store(&treeLdsCounters()[i], (u64)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
  }
  if (L >= lanesTotal) return;
  if (r >= N || r == a.deadRank) return;
  // an earlier call left its edges mid-call when a member gave up
  if (callFailed(a) != 0) return;
  const int Lc = BATCH ? L % perTask : L;   // (channel, lane) inside the task
  const int ch = Lc / a.lanes;
  const int k = Lc % a.lanes;

  // this member's place in its channel's tree
  TreeNode nd;
  const int t = a.nChannels > 1 && 2 * ch >= a.nChannels ? 1 : 0;
  dtreeNode(N, r, t, nd.up, nd.d[0], nd.d[1]);
  auto worker = [&](int node, int edge) { return ((size_t)L * N + node) * 3 + edge; };
  auto cross = [&](int node) { return node / a.groupSize != g; };
  if constexpr (LDSQ) {
    // An edge inside the workgroup: node x's FIFO up is 2x, its FIFO down
    // 2x + 1, x its index in the workgroup.  An edge to another workgroup
    // keeps its FIFO and carried counters in device memory.
    const int base = g * a.groupSize;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (nd.d[i] >= 0) {
        if (!cross(nd.d[i])) {
          nd.fromChild[i] = openLdsEdge(2 * (nd.d[i] - base));
          nd.toChild[i] = openLdsEdge(2 * (nd.d[i] - base) + 1);
        } else {
          nd.fromChild[i] = openEdge(a, worker(r, i), true, true);
          nd.toChild[i] = openEdge(a, worker(nd.d[i], 2), true, false);
        }
      }
    }
    if (nd.up >= 0) {
      if (!cross(nd.up)) {
        nd.fromParent = openLdsEdge(2 * (r - base) + 1);
        nd.toParent = openLdsEdge(2 * (r - base));
      } else {
        int pu, p0, p1;
        dtreeNode(N, nd.up, t, pu, p0, p1);
        nd.fromParent = openEdge(a, worker(r, 2), true, true);
        nd.toParent = openEdge(a, worker(nd.up, r == p0 ? 0 : 1), true, false);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (nd.d[i] >= 0) {
        nd.fromChild[i] = openEdge(a, worker(r, i), cross(nd.d[i]), true);
        nd.toChild[i] = openEdge(a, worker(nd.d[i], 2), cross(nd.d[i]), false);
      }
    }
    if (nd.up >= 0) {
      int pu, p0, p1;
      dtreeNode(N, nd.up, t, pu, p0, p1);
      nd.fromParent = openEdge(a, worker(r, 2), cross(nd.up), true);
      nd.toParent = openEdge(a, worker(nd.up, r == p0 ? 0 : 1), cross(nd.up), false);
    }
  }

  bool ok;
  if constexpr (ONEWG && PROTO == kSimple) {
    const int role = (nd.up >= 0 ? kRoleParent : 0) | (nd.d[0] >= 0 ? kRoleD0 : 0) | (nd.d[1] >= 0 ? kRoleD1 : 0);
    switch (role) {
#define AR_ROLE(R) treePasses<PROTO, DT, OP, U, BATCH, false, R, false, LDSQ>(a, nd, L, perTask, ch, k, lane, r)
      case kRoleParent: ok = AR_ROLE(kRoleParent); break;                                      // leaf
      case kRoleParent | kRoleD0: ok = AR_ROLE(kRoleParent | kRoleD0); break;                  // one child
      case kRoleParent | kRoleD0 | kRoleD1: ok = AR_ROLE(kRoleParent | kRoleD0 | kRoleD1); break;
      case kRoleD1: ok = AR_ROLE(kRoleD1); break;                                              // the root
      default: ok = AR_ROLE(kRoleAtRunTime); break;   // any other shape reads its peers at run time
#undef AR_ROLE
    }
  } else if constexpr (ONEWG) {   // LL / LL128, every edge inside the workgroup
    ok = treePasses<PROTO, DT, OP, U, BATCH, false, kRoleAtRunTime, PROTO == kLL128>(a, nd, L, perTask, ch, k, lane, r);
  } else {
    // as in the ring kernel: only a member with an edge to another workgroup
    // runs the pass compiled with that edge's code
    bool xwg = nd.up >= 0 && nd.toParent.agent;
#pragma unroll
    for (int i = 0; i < 2; ++i) xwg = xwg || (nd.d[i] >= 0 && nd.toChild[i].agent);
    if constexpr (PROTO == kSimple && !BATCH) {
      // Simple trees cut into workgroups: the members whose edges all stay
      // inside the workgroup run a pass compiled for their role too
      const int role = (nd.up >= 0 ? kRoleParent : 0) | (nd.d[0] >= 0 ? kRoleD0 : 0) | (nd.d[1] >= 0 ? kRoleD1 : 0);
      if (xwg) {
        ok = treePasses<PROTO, DT, OP, U, BATCH, true, kRoleAtRunTime, false, LDSQ>(a, nd, L, perTask, ch, k, lane, r);
      } else {
        switch (role) {
#define AR_ROLE(R) treePasses<PROTO, DT, OP, U, BATCH, false, R, false, LDSQ>(a, nd, L, perTask, ch, k, lane, r)
          case kRoleParent: ok = AR_ROLE(kRoleParent); break;
          case kRoleParent | kRoleD0: ok = AR_ROLE(kRoleParent | kRoleD0); break;
          case kRoleParent | kRoleD0 | kRoleD1: ok = AR_ROLE(kRoleParent | kRoleD0 | kRoleD1); break;
          default: ok = AR_ROLE(kRoleAtRunTime); break;
#undef AR_ROLE
        }
      }
    } else {
      ok = xwg ? treePasses<PROTO, DT, OP, U, BATCH, true>(a, nd, L, perTask, ch, k, lane, r)
               : treePasses<PROTO, DT, OP, U, BATCH, false>(a, nd, L, perTask, ch, k, lane, r);
    }
  }
  if (!ok) return;
  // LL / LL128 never touch the tail counter per slot: publish it once so the
  // next call starts both ends of each FIFO at the same step.
  if (PROTO != kSimple && lane == 0) {
    if (nd.up >= 0) stRelaxed64(&nd.toParent.conn->tail, nd.toParent.step, true);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (nd.d[i] >= 0) stRelaxed64(&nd.toChild[i].conn->tail, nd.toChild[i].step, true);
  }
}

// ------------------------------------------------------------- dispatch

// The ring kernel for one collective, element type and op (AllGather has no
// arithmetic: one kernel per element size).
template <int PROTO, int U, int COLL, bool BATCH, bool ONEWG = false, bool PERKIND = ONEWG, bool LDSQ = false>
KernelFn pickRing(int dtype, int op) {
  if (COLL == kCollAllGather) {
    switch (dtype) {
      case arInt32: case arFloat32:
        return ringAllReduceKernel<PROTO, arInt32, arSum, U, COLL, BATCH, ONEWG, PERKIND, LDSQ>;
      case arFloat16: case arBfloat16:
        return ringAllReduceKernel<PROTO, arBfloat16, arSum, U, COLL, BATCH, ONEWG, PERKIND, LDSQ>;
      case arUint64: return ringAllReduceKernel<PROTO, arUint64, arProbe, U, COLL, BATCH, ONEWG, PERKIND, LDSQ>;
    }
    return nullptr;
  }
#define AR_RING(DT, OP) ringAllReduceKernel<PROTO, DT, OP, U, COLL, BATCH, ONEWG, PERKIND, LDSQ>
  switch (dtype) {
    case arInt32: return op == arSum ? AR_RING(arInt32, arSum) : op == arMax ? AR_RING(arInt32, arMax)
                       : op == arMin ? AR_RING(arInt32, arMin) : nullptr;
    case arFloat32: return op == arSum ? AR_RING(arFloat32, arSum) : op == arMax ? AR_RING(arFloat32, arMax)
                         : op == arMin ? AR_RING(arFloat32, arMin) : nullptr;
    case arFloat16: return op == arSum ? AR_RING(arFloat16, arSum) : op == arMax ? AR_RING(arFloat16, arMax)
                         : op == arMin ? AR_RING(arFloat16, arMin) : nullptr;
    case arBfloat16: return op == arSum ? AR_RING(arBfloat16, arSum) : op == arMax ? AR_RING(arBfloat16, arMax)
                          : op == arMin ? AR_RING(arBfloat16, arMin) : nullptr;
    case arUint64: return op == arProbe ? AR_RING(arUint64, arProbe) : nullptr;
  }
#undef AR_RING
  return nullptr;
}

template <int PROTO, int U, bool BATCH, bool ONEWG = false, bool LDSQ = false>
KernelFn pickTree(int dtype, int op) {
#define AR_TREE(DT, OP) treeAllReduceKernel<PROTO, DT, OP, U, BATCH, ONEWG, LDSQ>
  switch (dtype) {
    case arInt32: return op == arSum ? AR_TREE(arInt32, arSum) : op == arMax ? AR_TREE(arInt32, arMax)
                       : op == arMin ? AR_TREE(arInt32, arMin) : nullptr;
    case arFloat32: return op == arSum ? AR_TREE(arFloat32, arSum) : op == arMax ? AR_TREE(arFloat32, arMax)
                         : op == arMin ? AR_TREE(arFloat32, arMin) : nullptr;
    case arFloat16: return op == arSum ? AR_TREE(arFloat16, arSum) : op == arMax ? AR_TREE(arFloat16, arMax)
                         : op == arMin ? AR_TREE(arFloat16, arMin) : nullptr;
    case arBfloat16: return op == arSum ? AR_TREE(arBfloat16, arSum) : op == arMax ? AR_TREE(arBfloat16, arMax)
                          : op == arMin ? AR_TREE(arBfloat16, arMin) : nullptr;
    case arUint64: return op == arProbe ? AR_TREE(arUint64, arProbe) : nullptr;
  }
#undef AR_TREE
  return nullptr;
}

// Protocol and slot size: the ring's Simple slot is 1, 2, 4 or 8 KiB (at
// most 4 KiB for a ring cut into workgroups), the tree's 1, 2 or 4 KiB; LL
// has one slot geometry, LL128 two (2 KiB, and 4 KiB for single calls).
template <int COLL, bool BATCH>
KernelFn pickRingSimple(const Plan& plan, int dtype, int op) {
  // rings inside one workgroup get the instantiation compiled for them, with
  // FIFO slots in LDS when the plan says so (single calls)
  const bool one = plan.nGroups == 1;
  if (one && plan.ldsFifo) {   // single calls and batched launches
    switch (plan.unroll) {
      case 1: return pickRing<kSimple, 1, COLL, BATCH, true, true, true>(dtype, op);
      case 2: return pickRing<kSimple, 2, COLL, BATCH, true, true, true>(dtype, op);
      case 4: return pickRing<kSimple, 4, COLL, BATCH, true, true, true>(dtype, op);
    }
    return nullptr;
  }
  if constexpr (!BATCH) {
    if (plan.ldsFifo) {   // a ring cut into workgroups: LDS slots on the edges inside each
      switch (plan.unroll) {
        case 1: return pickRing<kSimple, 1, COLL, false, false, false, true>(dtype, op);
        case 2: return pickRing<kSimple, 2, COLL, false, false, false, true>(dtype, op);
        case 4: return pickRing<kSimple, 4, COLL, false, false, false, true>(dtype, op);
      }
      return nullptr;
    }
  }
  switch (plan.unroll) {
    case 1: return one ? pickRing<kSimple, 1, COLL, BATCH, true>(dtype, op) : pickRing<kSimple, 1, COLL, BATCH>(dtype, op);
    case 2: return one ? pickRing<kSimple, 2, COLL, BATCH, true>(dtype, op) : pickRing<kSimple, 2, COLL, BATCH>(dtype, op);
    case 4: return one ? pickRing<kSimple, 4, COLL, BATCH, true>(dtype, op) : pickRing<kSimple, 4, COLL, BATCH>(dtype, op);
    case 8: return pickRing<kSimple, 8, COLL, BATCH>(dtype, op);
  }
  return nullptr;
}

// LL and LL128; single calls whose rings lie inside one workgroup get the
// instantiation compiled for them (no code for edges between workgroups; an
// LL128 receive in one poll).
template <int COLL, bool BATCH>
KernelFn pickRingLLOnly(const Plan& plan, int dtype, int op) {
  if (plan.proto != kLL) return nullptr;
  if (!BATCH && plan.nGroups == 1) return pickRing<kLL, kLLUnroll, COLL, false, true>(dtype, op);
  return pickRing<kLL, kLLUnroll, COLL, BATCH>(dtype, op);
}

template <int COLL, bool BATCH>
KernelFn pickRingLL128Only(const Plan& plan, int dtype, int op) {
  if (plan.proto != kLL128) return nullptr;
  const bool one = !BATCH && plan.nGroups == 1;
  if (plan.unroll == kLL128Unroll) {
    if (!one) return pickRing<kLL128, kLL128Unroll, COLL, BATCH>(dtype, op);
    return plan.perKind ? pickRing<kLL128, kLL128Unroll, COLL, false, true, true>(dtype, op)
                        : pickRing<kLL128, kLL128Unroll, COLL, false, true, false>(dtype, op);
  }
  if constexpr (!BATCH) {   // large LL128 slots: single calls only
    if (plan.unroll == kLL128UnrollLarge) {
      if (!one) return pickRing<kLL128, kLL128UnrollLarge, COLL, false>(dtype, op);
      return plan.perKind ? pickRing<kLL128, kLL128UnrollLarge, COLL, false, true, true>(dtype, op)
                          : pickRing<kLL128, kLL128UnrollLarge, COLL, false, true, false>(dtype, op);
    }
  }
  return nullptr;
}

template <int COLL, bool BATCH>
KernelFn pickRingLL(const Plan& plan, int dtype, int op) {
  return plan.proto == kLL ? pickRingLLOnly<COLL, BATCH>(plan, dtype, op) : pickRingLL128Only<COLL, BATCH>(plan, dtype, op);
}

template <int COLL, bool BATCH>
KernelFn pickRingProto(const Plan& plan, int dtype, int op) {
  return plan.proto == kSimple ? pickRingSimple<COLL, BATCH>(plan, dtype, op) : pickRingLL<COLL, BATCH>(plan, dtype, op);
}

template <bool BATCH>
KernelFn pickTreeProto(const Plan& plan, int dtype, int op) {
  // single calls whose trees lie inside one workgroup get the instantiation
  // compiled for them (batched LL / LL128 launches keep the general one)
  const bool oneLL = !BATCH && plan.nGroups == 1;
  switch (plan.proto) {
    case kLL: return oneLL ? pickTree<kLL, kLLUnroll, false, true>(dtype, op) : pickTree<kLL, kLLUnroll, BATCH>(dtype, op);
    case kLL128:
      if (plan.unroll != kLL128Unroll) return nullptr;
      return oneLL ? pickTree<kLL128, kLL128Unroll, false, true>(dtype, op)
                   : pickTree<kLL128, kLL128Unroll, BATCH>(dtype, op);
    case kSimple: {
      // trees inside one workgroup get the instantiation compiled for them,
      // with their FIFOs in LDS when the plan says so
      const bool one = plan.nGroups == 1;
      if (one && plan.ldsFifo) {
        switch (plan.unroll) {
          case 1: return pickTree<kSimple, 1, BATCH, true, true>(dtype, op);
          case 2: return pickTree<kSimple, 2, BATCH, true, true>(dtype, op);
          case 4: return pickTree<kSimple, 4, BATCH, true, true>(dtype, op);
        }
        return nullptr;
      }
      if (plan.ldsFifo) {   // a tree cut into workgroups, its inside edges in LDS (single calls)
        if constexpr (!BATCH) {
          switch (plan.unroll) {
            case 1: return pickTree<kSimple, 1, false, false, true>(dtype, op);
            case 2: return pickTree<kSimple, 2, false, false, true>(dtype, op);
            case 4: return pickTree<kSimple, 4, false, false, true>(dtype, op);
          }
        }
        return nullptr;
      }
      switch (plan.unroll) {
        case 1: return one ? pickTree<kSimple, 1, BATCH, true>(dtype, op) : pickTree<kSimple, 1, BATCH>(dtype, op);
        case 2: return one ? pickTree<kSimple, 2, BATCH, true>(dtype, op) : pickTree<kSimple, 2, BATCH>(dtype, op);
        case 4: return one ? pickTree<kSimple, 4, BATCH, true>(dtype, op) : pickTree<kSimple, 4, BATCH>(dtype, op);
      }
      break;
    }
  }
  return nullptr;
}

}  // namespace
}  // namespace ar
