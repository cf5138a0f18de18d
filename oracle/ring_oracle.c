/*
 * ring_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, single-threaded CPU implementation of the ring AllReduce that the
 * HIP library computes, written to be checked by eye against the pages.  It
 * shares no code, header, table or helper with the HIP path; only the tests,
 * the package's smoke check and the benchmark's CPU-baseline leg may load it.
 *
 * What it computes (all citations are to the web pages the method comes from):
 *
 *  - Channel split.  A collective is cut into one contiguous share per channel
 *    ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.2 §2.2 "通道 channel",
 *    walkthrough step 3 "資料切分"].  The pages leave the exact rounding open;
 *    the share is rounded up to the 16-byte grain the chunk formula uses:
 *        P = alignUp(divUp(count, nChannels), 16/elemSize)
 *        channel ch covers [min(ch*P, count), min((ch+1)*P, count)).
 *
 *  - Loops and chunks.  Inside a channel the ring walks loops of
 *    nRanks*chunkElems elements.  When fewer elements than a full loop remain,
 *    the chunk shrinks to alignUp(divUp(rem, nRanks), 16/elemSize) and chunk k
 *    covers [k*cur, min((k+1)*cur, rem)), empty once k*cur >= rem
 *    [same book, ch.2 §2.3 "演算法 algorithm", RingARAlgorithm::getNextSendAddr].
 *
 *  - Summation order.  At ring stage s the member at ring index r sends chunk
 *    (r + nRanks - 1 - s) mod nRanks [same passage, the chunkId formula].  So
 *    chunk c leaves member c+1 raw, is combined at c+2, c+3, ... and is
 *    finished at member c after nRanks-1 reduce steps; the all-gather half then
 *    copies the finished chunk around the ring [same section, the
 *    reduce-scatter / all-gather walkthrough and nStepsPerLoop = 2(nRanks-1)].
 *    With the identity ring used for every channel, member index == rank, so
 *        acc = x[(c+1) mod N][e];  acc = OP(acc, x[(c+k) mod N][e]), k=2..N
 *    and every rank receives acc.
 *
 *  - OP.  Sum on int32 wraps (two's complement).  Sum on float32 is one IEEE
 *    binary32 add, round-to-nearest-even.  Sum on float16/bfloat16 widens both
 *    operands exactly to binary32, adds, and rounds back to the 16-bit type with
 *    round-to-nearest-even, because the partial crosses the ring in its own
 *    type at every hop.  Max is acc = (x > acc) ? x : acc and Min is
 *    acc = (x < acc) ? x : acc with acc the incoming partial and x the local
 *    value.  The pages fix none of these; they are the readings this library
 *    takes and both sides implement them independently.
 *
 *  - A debug-only uint64 "probe" op, acc = acc*16 + x, is not commutative, so a
 *    folded value spells out the order in which ranks were visited.
 *
 *  - ReduceScatter and AllGather, the two halves of the same ring [same book,
 *    ch.5 §三: nSteps is 2(nRanks-1) for AllReduce and nRanks-1 for the
 *    others; ch.6 §三: their traffic is nRanks times the count, and AllGather
 *    moves bytes with no reduction].  With the collective's usual meaning
 *    (rank r's ReduceScatter output is the reduction of block r of every
 *    rank's input; AllGather's output is every rank's input in rank order),
 *    the reduce-scatter half of the ring gives block b the order
 *        acc = x[b+1][b-th block]; acc = OP(acc, x[b+k][b-th block]), k=2..N
 *    (it leaves rank b+1 raw and is finished at its owner b), whatever the
 *    channel and chunk split.
 *
 *  - Tree AllReduce, the pages' second algorithm.  The binary tree over the
 *    ranks ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.4 "Ring 與
 *    Tree：把搜尋結果變成演算法拓撲", ncclGetBtree]: a rank's parent and children
 *    follow from its lowest set bit (see ar_oracle_btree).  The double tree
 *    [same passage, ncclGetDtree; "NCCL Tree拓扑介绍", "Double Binary Tree"]
 *    adds a second tree: the first mirrored (rank -> N-1-rank) when N is even,
 *    shifted by one rank when N is odd; every peer the btree gives for the
 *    mirrored or shifted rank is mapped back the same way (the pages elide
 *    this mapping; it is the inverse of the relabelling).  One tree is bound
 *    to one channel and the first half of the data goes to the first tree,
 *    the rest to the second; here channel ch of nCh runs on the second tree
 *    when 2*ch >= nCh (with one channel, only the first tree is used).
 *    Reduce phase: a node combines what it received from its children with
 *    its own data and passes the result to its parent; the root ends with the
 *    full reduction, which the broadcast phase copies down to every rank
 *    ["NCCL Tree拓扑介绍", "Single Binary Tree"].  The pages do not fix the
 *    order inside a node; the reading here, like the ring's OP(incoming,
 *    local), folds the received partials first, in the order the tree names
 *    the children (d0, then d1), and the node's own value last:
 *        partial(v) = OP(OP(partial(d0), partial(d1)), x[v])
 *    (a missing child drops out; a leaf's partial is x[v]).  Chunking and
 *    pipelining never change this per-element expression.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math; x86-64 SSE
 * arithmetic, default MXCSR, so no flush-to-zero).
 */
#include <stdint.h>
#include <stdlib.h>
#include <stddef.h>
#include <string.h>

enum { ORC_INT32 = 0, ORC_FLOAT32 = 1, ORC_FLOAT16 = 2, ORC_BFLOAT16 = 3, ORC_UINT64 = 4 };
enum { ORC_SUM = 0, ORC_MAX = 1, ORC_MIN = 2, ORC_PROBE = 3 };

static size_t elem_size(int dtype) {
  switch (dtype) {
    case ORC_INT32: return 4;
    case ORC_FLOAT32: return 4;
    case ORC_FLOAT16: return 2;
    case ORC_BFLOAT16: return 2;
    case ORC_UINT64: return 8;
    default: return 0;
  }
}

static size_t div_up(size_t x, size_t y) { return (x + y - 1) / y; }
static size_t align_up(size_t x, size_t a) { return div_up(x, a) * a; }
static size_t min_sz(size_t a, size_t b) { return a < b ? a : b; }

/* ---------------- 16-bit float conversions (written from IEEE 754) ---------- */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 is the top half of a binary32; widening is exact. */
static float bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even.  NaN stays a quiet NaN
 * with its sign; overflow rounds to infinity through the carry. */
static uint16_t f32_to_bf16(float f) {
  uint32_t u = f32_to_bits(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lower = u & 0xffffu;          /* the 16 bits dropped */
  uint32_t upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

/* binary16 -> binary32, exact (every half value is a float). */
static float f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h >> 15) & 1u;
  uint32_t expo = (uint32_t)(h >> 10) & 0x1fu;
  uint32_t mant = (uint32_t)h & 0x3ffu;
  float mag;
  if (expo == 0) {
    mag = (float)mant * (1.0f / 16777216.0f);          /* mant * 2^-24, exact */
  } else if (expo == 31) {
    return bits_to_f32((sign << 31) | 0x7f800000u | (mant << 13));
  } else {
    mag = bits_to_f32(((expo - 15u + 127u) << 23) | (mant << 13));
  }
  return sign ? -mag : mag;
}

/* binary32 -> binary16, round to nearest, ties to even, with subnormal results
 * and overflow to infinity.  Done on the exact binary32 significand. */
static uint16_t f32_to_f16(float f) {
  uint32_t u = f32_to_bits(f);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t expo = (u >> 23) & 0xffu;
  uint32_t mant = u & 0x7fffffu;
  if (expo == 0xffu) {                                  /* inf or NaN */
    if (mant == 0) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | 0x7e00u | (mant >> 13));
  }
  if (expo == 0) return sign;        /* binary32 subnormals are far below half's range */
  int e = (int)expo - 127;           /* unbiased exponent of the value */
  uint32_t sig = mant | 0x800000u;   /* 24-bit significand, value = sig * 2^(e-23) */
  /* The half result is q * 2^(he) with q an integer; find how many low bits of
   * sig fall below the half's last place. */
  int shift;                         /* bits to drop from sig */
  if (e >= -14) shift = 13;          /* normal half: 11-bit significand */
  else shift = 13 + (-14 - e);       /* subnormal half: fixed scale 2^-24 */
  if (shift > 25) return sign;       /* below half the smallest subnormal */
  uint32_t q = sig >> shift;
  uint32_t rem = sig & ((1u << shift) - 1u);
  uint32_t halfway = 1u << (shift - 1);
  if (rem > halfway || (rem == halfway && (q & 1u))) q += 1u;
  uint32_t bits;
  if (e >= -14) {
    /* q is 1.xxx with the implicit bit at 2^10; a carry may bump the exponent */
    uint32_t he = (uint32_t)(e + 15);
    if (q >= 0x800u) { q >>= 1; he += 1; }
    if (he >= 31) return (uint16_t)(sign | 0x7c00u);
    bits = (he << 10) | (q & 0x3ffu);
  } else {
    bits = q;                         /* q == 0x400 becomes the smallest normal */
  }
  return (uint16_t)(sign | bits);
}

/* ---------------- the per-element combine, one dtype at a time -------------- */

static void fold_i32(int op, int32_t* acc, const int32_t* x, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    if (op == ORC_SUM) acc[i] = (int32_t)((uint32_t)acc[i] + (uint32_t)x[i]);
    else if (op == ORC_MAX) acc[i] = (x[i] > acc[i]) ? x[i] : acc[i];
    else acc[i] = (x[i] < acc[i]) ? x[i] : acc[i];
  }
}

static void fold_f32(int op, float* acc, const float* x, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    if (op == ORC_SUM) acc[i] = acc[i] + x[i];
    else if (op == ORC_MAX) acc[i] = (x[i] > acc[i]) ? x[i] : acc[i];
    else acc[i] = (x[i] < acc[i]) ? x[i] : acc[i];
  }
}

static void fold_half(int op, int is_bf16, uint16_t* acc, const uint16_t* x, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    float a = is_bf16 ? bf16_to_f32(acc[i]) : f16_to_f32(acc[i]);
    float b = is_bf16 ? bf16_to_f32(x[i]) : f16_to_f32(x[i]);
    if (op == ORC_SUM) {
      float s = a + b;
      acc[i] = is_bf16 ? f32_to_bf16(s) : f32_to_f16(s);
    } else if (op == ORC_MAX) {
      if (b > a) acc[i] = x[i];
    } else {
      if (b < a) acc[i] = x[i];
    }
  }
}

static void fold_u64_probe(uint64_t* acc, const uint64_t* x, size_t n) {
  for (size_t i = 0; i < n; ++i) acc[i] = acc[i] * 16u + x[i];
}

static int fold(int dtype, int op, void* acc, const void* x, size_t n) {
  switch (dtype) {
    case ORC_INT32: fold_i32(op, (int32_t*)acc, (const int32_t*)x, n); return 0;
    case ORC_FLOAT32: fold_f32(op, (float*)acc, (const float*)x, n); return 0;
    case ORC_FLOAT16: fold_half(op, 0, (uint16_t*)acc, (const uint16_t*)x, n); return 0;
    case ORC_BFLOAT16: fold_half(op, 1, (uint16_t*)acc, (const uint16_t*)x, n); return 0;
    case ORC_UINT64: fold_u64_probe((uint64_t*)acc, (const uint64_t*)x, n); return 0;
    default: return -1;
  }
}

static int check_args(int nranks, int dtype, int op, int nchannels, size_t chunk_elems) {
  size_t esz = elem_size(dtype);
  if (nranks < 1 || nchannels < 1 || esz == 0) return -1;
  if (op < ORC_SUM || op > ORC_PROBE) return -1;
  if ((op == ORC_PROBE) != (dtype == ORC_UINT64)) return -1;
  size_t grain = 16 / esz;
  if (chunk_elems == 0 || chunk_elems % grain != 0) return -1;
  return 0;
}

/* Locate element idx: its channel, loop, chunk and the chunk's element range
 * [first, first+len) in the rank buffer.  Returns -1 if idx >= count. */
int ar_oracle_locate(int nranks, size_t count, int dtype, int nchannels, size_t chunk_elems,
                     size_t idx, int* channel, long long* loop, int* chunk,
                     size_t* first, size_t* len) {
  size_t esz = elem_size(dtype);
  if (esz == 0 || nranks < 1 || nchannels < 1 || idx >= count) return -1;
  size_t grain = 16 / esz;
  size_t per_ch = align_up(div_up(count, (size_t)nchannels), grain);
  size_t ch = idx / per_ch;
  size_t lo = min_sz(ch * per_ch, count);
  size_t hi = min_sz((ch + 1) * per_ch, count);
  size_t loop_size = (size_t)nranks * chunk_elems;
  size_t in_ch = idx - lo;
  size_t l = in_ch / loop_size;
  size_t off = l * loop_size;
  size_t rem = (hi - lo) - off;
  size_t cur = rem < loop_size ? align_up(div_up(rem, (size_t)nranks), grain) : chunk_elems;
  size_t c = (in_ch - off) / cur;
  size_t b = c * cur;
  size_t e = min_sz(b + cur, rem);
  if (channel) *channel = (int)ch;
  if (loop) *loop = (long long)l;
  if (chunk) *chunk = (int)c;
  if (first) *first = lo + off + b;
  if (len) *len = e - b;
  return 0;
}

/* Full ring AllReduce: out[r][0..count) for every rank r.  in and out are
 * arrays of nranks host pointers; out[r] may equal in[r] only if the caller
 * does not need the inputs afterwards (the fold reads in[] chunk by chunk
 * before writing that chunk). */
int ar_oracle_allreduce(int nranks, size_t count, int dtype, int op, int nchannels,
                        size_t chunk_elems, const void* const* in, void* const* out) {
  if (check_args(nranks, dtype, op, nchannels, chunk_elems) != 0) return -1;
  size_t esz = elem_size(dtype);
  size_t grain = 16 / esz;
  if (count == 0) return 0;
  if (nranks == 1) {
    if (out[0] != in[0]) memcpy(out[0], in[0], count * esz);
    return 0;
  }
  size_t per_ch = align_up(div_up(count, (size_t)nchannels), grain);
  size_t loop_size = (size_t)nranks * chunk_elems;
  /* accumulator for one chunk, in the element type */
  enum { TMP_BYTES = 1 << 16 };
  unsigned char acc[TMP_BYTES];
  size_t tmp_elems = TMP_BYTES / esz;
  for (int ch = 0; ch < nchannels; ++ch) {
    size_t lo = min_sz((size_t)ch * per_ch, count);
    size_t hi = min_sz((size_t)(ch + 1) * per_ch, count);
    size_t len = hi - lo;
    for (size_t off = 0; off < len; off += loop_size) {
      size_t rem = len - off;
      size_t cur = rem < loop_size ? align_up(div_up(rem, (size_t)nranks), grain) : chunk_elems;
      for (int c = 0; c < nranks; ++c) {
        size_t b = (size_t)c * cur;
        if (b >= rem) continue;                       /* empty chunk */
        size_t e = min_sz(b + cur, rem);
        size_t first = lo + off + b;
        /* walk the chunk in pieces that fit the accumulator */
        for (size_t p = first; p < lo + off + e; p += tmp_elems) {
          size_t n = min_sz(tmp_elems, lo + off + e - p);
          int start = (c + 1) % nranks;               /* member c+1 sends it raw */
          memcpy(acc, (const unsigned char*)in[start] + p * esz, n * esz);
          for (int k = 2; k <= nranks; ++k) {
            int r = (c + k) % nranks;                 /* last one is r == c */
            fold(dtype, op, acc, (const unsigned char*)in[r] + p * esz, n);
          }
          for (int r = 0; r < nranks; ++r)
            memcpy((unsigned char*)out[r] + p * esz, acc, n * esz);
        }
      }
    }
  }
  return 0;
}

/* One output element, computed on its own (for sampled checks at full size). */
int ar_oracle_element(int nranks, size_t count, int dtype, int op, int nchannels,
                      size_t chunk_elems, const void* const* in, size_t idx, void* result) {
  if (check_args(nranks, dtype, op, nchannels, chunk_elems) != 0) return -1;
  size_t esz = elem_size(dtype);
  int c = 0;
  if (ar_oracle_locate(nranks, count, dtype, nchannels, chunk_elems, idx, NULL, NULL, &c, NULL, NULL) != 0)
    return -1;
  unsigned char acc[8];
  int start = nranks == 1 ? 0 : (c + 1) % nranks;
  memcpy(acc, (const unsigned char*)in[start] + idx * esz, esz);
  for (int k = 2; k <= nranks; ++k) {
    int r = (c + k) % nranks;
    fold(dtype, op, acc, (const unsigned char*)in[r] + idx * esz, 1);
  }
  memcpy(result, acc, esz);
  return 0;
}

/* Batched form of ar_oracle_element over an index list. */
int ar_oracle_elements(int nranks, size_t count, int dtype, int op, int nchannels,
                       size_t chunk_elems, const void* const* in, const int64_t* idx,
                       size_t nidx, void* results) {
  size_t esz = elem_size(dtype);
  for (size_t i = 0; i < nidx; ++i) {
    if (idx[i] < 0) return -1;
    int rc = ar_oracle_element(nranks, count, dtype, op, nchannels, chunk_elems, in,
                               (size_t)idx[i], (unsigned char*)results + i * esz);
    if (rc != 0) return rc;
  }
  return 0;
}

/* ReduceScatter: in[r] holds nranks*count elements (block q at q*count),
 * out[r] receives count elements: the ring fold of block r over all ranks. */
int ar_oracle_reduce_scatter(int nranks, size_t count, int dtype, int op, const void* const* in,
                             void* const* out) {
  if (check_args(nranks, dtype, op, 1, 16 / (elem_size(dtype) ? elem_size(dtype) : 1)) != 0) return -1;
  size_t esz = elem_size(dtype);
  if (count == 0) return 0;
  enum { TMP_BYTES = 1 << 16 };
  unsigned char acc[TMP_BYTES];
  size_t tmp_elems = TMP_BYTES / esz;
  for (int b = 0; b < nranks; ++b) {              /* block b is finished at rank b */
    size_t base = (size_t)b * count;
    for (size_t p = 0; p < count; p += tmp_elems) {
      size_t n = min_sz(tmp_elems, count - p);
      int start = nranks == 1 ? 0 : (b + 1) % nranks;
      memcpy(acc, (const unsigned char*)in[start] + (base + p) * esz, n * esz);
      for (int k = 2; k <= nranks; ++k) {
        int r = (b + k) % nranks;
        fold(dtype, op, acc, (const unsigned char*)in[r] + (base + p) * esz, n);
      }
      memcpy((unsigned char*)out[b] + p * esz, acc, n * esz);
    }
  }
  return 0;
}

/* AllGather: in[r] holds count elements of elem_bytes each; out[r] receives
 * nranks*count elements, rank q's input at q*count. */
int ar_oracle_all_gather(int nranks, size_t count, size_t elem_bytes, const void* const* in,
                         void* const* out) {
  if (nranks < 1 || elem_bytes == 0) return -1;
  for (int r = 0; r < nranks; ++r)
    for (int q = 0; q < nranks; ++q)
      memcpy((unsigned char*)out[r] + (size_t)q * count * elem_bytes, in[q], count * elem_bytes);
  return 0;
}

/* Conversions exposed so tests can pin them against numpy / torch. */
void ar_oracle_f32_to_bf16(const float* x, uint16_t* y, size_t n) {
  for (size_t i = 0; i < n; ++i) y[i] = f32_to_bf16(x[i]);
}
void ar_oracle_f32_to_f16(const float* x, uint16_t* y, size_t n) {
  for (size_t i = 0; i < n; ++i) y[i] = f32_to_f16(x[i]);
}
void ar_oracle_f16_to_f32(const uint16_t* x, float* y, size_t n) {
  for (size_t i = 0; i < n; ++i) y[i] = f16_to_f32(x[i]);
}
void ar_oracle_bf16_to_f32(const uint16_t* x, float* y, size_t n) {
  for (size_t i = 0; i < n; ++i) y[i] = bf16_to_f32(x[i]);
}

/* ---------------- tree AllReduce ------------------------------------------ */

/* Binary tree over ranks 0..nranks-1 [pages: ch.4, ncclGetBtree; "NCCL Tree
 *拓扑介绍", the binary tree drawn over the ranks].  The tree is the in-order
 * tree of the ranks' binary numbering, built here from that definition over
 * spans of ranks:
 *  - rank 0 is the root and has one child, the root of the span [1, nranks)
 *    (the pages name it d1);
 *  - the root of a non-empty span [lo, hi) is its rank with the largest lowest
 *    set bit (the "roundest" number); its first child (d0, child_type 0) is
 *    the root of [lo, root) and its second (d1, child_type 1) the root of
 *    [root + 1, hi).
 * Every rank but 0 is the root of exactly one span, so each query builds the
 * whole tree (O(nranks), recursion depth log2 nranks) and reads its entry. */
static int span_root(int lo, int hi) {   /* the rank in [lo, hi) with the largest lowest set bit */
  int p = 1;
  while (p * 2 <= hi) p *= 2;            /* from the largest power of two below hi down */
  for (; p >= 1; p /= 2) {
    int m = (lo + p - 1) / p * p;        /* the first multiple of p at or above lo */
    if (m < hi) return m;
  }
  return -1;
}

static int span_tree(int lo, int hi, int parent, int side, int* up, int* d0, int* d1, int* type) {
  if (lo >= hi) return -1;
  int r = span_root(lo, hi);
  up[r] = parent;
  type[r] = side;
  d0[r] = span_tree(lo, r, r, 0, up, d0, d1, type);
  d1[r] = span_tree(r + 1, hi, r, 1, up, d0, d1, type);
  return r;
}

int ar_oracle_btree(int nranks, int rank, int* up, int* d0, int* d1, int* child_type) {
  if (nranks < 1 || rank < 0 || rank >= nranks) return -1;
  int* a = (int*)malloc(4 * sizeof(int) * (size_t)nranks);
  if (a == NULL) return -1;
  int *u = a, *c0 = a + nranks, *c1 = a + 2 * nranks, *t = a + 3 * nranks;
  u[0] = -1;
  c0[0] = -1;
  t[0] = 0;
  c1[0] = span_tree(1, nranks, 0, 1, u, c0, c1, t);
  if (up) *up = u[rank];
  if (d0) *d0 = c0[rank];
  if (d1) *d1 = c1[rank];
  if (child_type) *child_type = rank == 0 ? 0 : t[rank];
  free(a);
  return 0;
}

/* Tree `tree` (0 or 1) of the double binary tree [pages: ch.4, ncclGetDtree]. */
int ar_oracle_dtree(int nranks, int rank, int tree, int* up, int* d0, int* d1) {
  if (nranks < 1 || rank < 0 || rank >= nranks || tree < 0 || tree > 1) return -1;
  if (tree == 0) return ar_oracle_btree(nranks, rank, up, d0, d1, NULL);
  int peer[3];
  if (nranks % 2 == 0) {                 /* mirror: relabel r -> N-1-r */
    ar_oracle_btree(nranks, nranks - 1 - rank, &peer[0], &peer[1], &peer[2], NULL);
    for (int i = 0; i < 3; ++i) peer[i] = peer[i] < 0 ? -1 : nranks - 1 - peer[i];
  } else {                               /* shift: relabel r -> r-1 */
    ar_oracle_btree(nranks, (rank - 1 + nranks) % nranks, &peer[0], &peer[1], &peer[2], NULL);
    for (int i = 0; i < 3; ++i) peer[i] = peer[i] < 0 ? -1 : (peer[i] + 1) % nranks;
  }
  if (up) *up = peer[0];
  if (d0) *d0 = peer[1];
  if (d1) *d1 = peer[2];
  return 0;
}

/* The tree a channel is bound to: the first half of the channels (the first
 * half of the data) on tree 0, the rest on tree 1. */
int ar_oracle_tree_of_channel(int nchannels, int ch) {
  if (nchannels < 1 || ch < 0 || ch >= nchannels) return -1;
  return 2 * ch >= nchannels && nchannels > 1 ? 1 : 0;
}

enum { TREE_TMP_ELEMS_BYTES = 1 << 13 };

/* partial(v) over elements [p, p+n) of tree `tree`, into acc (n elements). */
static void tree_partial(int nranks, int tree, int v, int dtype, int op, const void* const* in,
                         size_t p, size_t n, unsigned char* acc) {
  size_t esz = elem_size(dtype);
  int d[2];
  ar_oracle_dtree(nranks, v, tree, NULL, &d[0], &d[1]);
  int have = 0;
  for (int i = 0; i < 2; ++i) {
    if (d[i] < 0) continue;
    if (!have) {
      tree_partial(nranks, tree, d[i], dtype, op, in, p, n, acc);
      have = 1;
    } else {
      unsigned char tmp[TREE_TMP_ELEMS_BYTES];
      tree_partial(nranks, tree, d[i], dtype, op, in, p, n, tmp);
      fold(dtype, op, acc, tmp, n);
    }
  }
  const unsigned char* x = (const unsigned char*)in[v] + p * esz;
  if (have) fold(dtype, op, acc, x, n);
  else memcpy(acc, x, n * esz);
}

static int tree_root(int nranks, int tree) {
  for (int r = 0; r < nranks; ++r) {
    int u;
    ar_oracle_dtree(nranks, r, tree, &u, NULL, NULL);
    if (u < 0) return r;
  }
  return -1;
}

/* Full double-tree AllReduce: out[r][0..count) for every rank r (channel
 * split as for the ring; the tree follows from the channel). */
int ar_oracle_tree_allreduce(int nranks, size_t count, int dtype, int op, int nchannels,
                             const void* const* in, void* const* out) {
  size_t esz = elem_size(dtype);
  if (check_args(nranks, dtype, op, nchannels, 16 / (esz ? esz : 1)) != 0) return -1;
  if (count == 0) return 0;
  size_t grain = 16 / esz;
  size_t per_ch = align_up(div_up(count, (size_t)nchannels), grain);
  size_t tmp_elems = TREE_TMP_ELEMS_BYTES / esz;
  unsigned char acc[TREE_TMP_ELEMS_BYTES];
  for (int ch = 0; ch < nchannels; ++ch) {
    size_t lo = min_sz((size_t)ch * per_ch, count);
    size_t hi = min_sz((size_t)(ch + 1) * per_ch, count);
    int tree = ar_oracle_tree_of_channel(nchannels, ch);
    int root = tree_root(nranks, tree);
    for (size_t p = lo; p < hi; p += tmp_elems) {
      size_t n = min_sz(tmp_elems, hi - p);
      tree_partial(nranks, tree, root, dtype, op, in, p, n, acc);
      for (int r = 0; r < nranks; ++r) memcpy((unsigned char*)out[r] + p * esz, acc, n * esz);
    }
  }
  return 0;
}

/* The tree fold for a list of single elements (sampled checks at full size). */
int ar_oracle_tree_elements(int nranks, size_t count, int dtype, int op, int nchannels,
                            const void* const* in, const int64_t* idx, size_t nidx, void* results) {
  size_t esz = elem_size(dtype);
  if (check_args(nranks, dtype, op, nchannels, 16 / (esz ? esz : 1)) != 0) return -1;
  size_t per_ch = align_up(div_up(count, (size_t)nchannels), 16 / esz);
  for (size_t i = 0; i < nidx; ++i) {
    if (idx[i] < 0 || (size_t)idx[i] >= count) return -1;
    int tree = ar_oracle_tree_of_channel(nchannels, (int)((size_t)idx[i] / per_ch));
    tree_partial(nranks, tree, tree_root(nranks, tree), dtype, op, in, (size_t)idx[i], 1,
                 (unsigned char*)results + i * esz);
  }
  return 0;
}
