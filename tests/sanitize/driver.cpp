// Host-code driver for the AddressSanitizer + UndefinedBehaviorSanitizer
// build (tests/test_sanitize_cpu.py): exercises the CPU oracle
// (oracle/ring_oracle.c), the tuner (ar_tune.cpp: cost model, measured time
// table, AR_TUNE_FILE parsing) and the group aggregation rule (ar_group.cpp)
// over many argument combinations, bad ones included, and checks a few
// invariants that need no reference.  Exit status 0 and no sanitizer report
// is a pass.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "ar.h"

extern "C" {
int ar_oracle_allreduce(int nranks, size_t count, int dtype, int op, int nchannels, size_t chunk_elems,
                        const void* const* in, void* const* out);
int ar_oracle_elements(int nranks, size_t count, int dtype, int op, int nchannels, size_t chunk_elems,
                       const void* const* in, const int64_t* idx, size_t nidx, void* results);
int ar_oracle_reduce_scatter(int nranks, size_t count, int dtype, int op, const void* const* in, void* const* out);
int ar_oracle_all_gather(int nranks, size_t count, size_t elem_bytes, const void* const* in, void* const* out);
int ar_oracle_btree(int nranks, int rank, int* up, int* d0, int* d1, int* child_type);
int ar_oracle_dtree(int nranks, int rank, int tree, int* up, int* d0, int* d1);
int ar_oracle_tree_allreduce(int nranks, size_t count, int dtype, int op, int nchannels, const void* const* in,
                             void* const* out);
}

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static size_t esz(int dt) { return dt == arUint64 ? 8 : (dt == arFloat16 || dt == arBfloat16) ? 2 : 4; }

// Ring and tree oracles on small random inputs of every type and op; int32
// sums, maxima and minima must equal a plain fold in any order.
static void oracles(std::mt19937& rng) {
  const int dts[] = {arInt32, arFloat32, arFloat16, arBfloat16};
  for (int n : {1, 2, 3, 5, 8, 13, 16, 17}) {
    for (size_t count : {(size_t)0, (size_t)1, (size_t)7, (size_t)33, (size_t)1000}) {
      for (int dt : dts) {
        for (int op : {arSum, arMax, arMin}) {
          const size_t e = esz(dt);
          std::vector<std::vector<uint8_t>> in(n), out(n), tout(n);
          std::vector<const void*> ip(n);
          std::vector<void*> op_(n), tp(n);
          for (int r = 0; r < n; ++r) {
            in[r].resize(count * e + 1);
            for (auto& b : in[r]) b = (uint8_t)(rng() & 0x3f);   // small exponents: no NaN or inf
            out[r].assign(count * e + 1, 0);
            tout[r].assign(count * e + 1, 0);
            ip[r] = in[r].data();
            op_[r] = out[r].data();
            tp[r] = tout[r].data();
          }
          for (int nch : {1, 3, 64}) {
            CHECK(ar_oracle_allreduce(n, count, dt, op, nch, 16 + 16 * (rng() % 4), ip.data(), op_.data()) == 0);
            CHECK(ar_oracle_tree_allreduce(n, count, dt, op, nch, ip.data(), tp.data()) == 0);
          }
          if (dt == arInt32 && count > 0) {
            for (size_t i = 0; i < count; ++i) {
              int32_t want = 0, got;
              for (int r = 0; r < n; ++r) {
                int32_t x;
                memcpy(&x, in[r].data() + 4 * i, 4);
                want = r == 0 ? x : op == arSum ? (int32_t)((uint32_t)want + (uint32_t)x)
                                    : op == arMax ? (x > want ? x : want) : (x < want ? x : want);
              }
              memcpy(&got, out[0].data() + 4 * i, 4);
              CHECK(got == want);
              memcpy(&got, tout[0].data() + 4 * i, 4);
              CHECK(got == want);
            }
          }
          std::vector<int64_t> idx;
          for (size_t i = 0; i < count; i += 1 + count / 5) idx.push_back((int64_t)i);
          std::vector<uint8_t> res(idx.size() * e + 1);
          CHECK(ar_oracle_elements(n, count, dt, op, 2, 32, ip.data(), idx.data(), idx.size(), res.data()) == 0);
        }
      }
    }
  }
  // the two halves, and argument errors
  for (int n : {1, 2, 4, 7}) {
    const size_t count = 45;
    std::vector<std::vector<float>> in(n, std::vector<float>(count * n)), out(n, std::vector<float>(count * n));
    std::vector<const void*> ip(n);
    std::vector<void*> op_(n);
    for (int r = 0; r < n; ++r) {
      for (auto& x : in[r]) x = (float)(rng() % 1000) / 7.0f;
      ip[r] = in[r].data();
      op_[r] = out[r].data();
    }
    CHECK(ar_oracle_reduce_scatter(n, count, arFloat32, arSum, ip.data(), op_.data()) == 0);
    CHECK(ar_oracle_all_gather(n, count, 4, ip.data(), op_.data()) == 0);
  }
  std::vector<float> x(16);
  const void* ip1[1] = {x.data()};
  void* op1[1] = {x.data()};
  CHECK(ar_oracle_allreduce(0, 16, arFloat32, arSum, 1, 16, ip1, op1) != 0);
  CHECK(ar_oracle_allreduce(1, 16, 99, arSum, 1, 16, ip1, op1) != 0);
  CHECK(ar_oracle_allreduce(1, 16, arFloat32, 99, 1, 16, ip1, op1) != 0);
  CHECK(ar_oracle_allreduce(1, 16, arFloat32, arSum, 0, 16, ip1, op1) != 0);
}

// Tree shapes: every child names its parent back, ranks 1..N-1 have one.
static void trees() {
  for (int n = 1; n <= 130; ++n) {
    for (int t = 0; t < 2; ++t) {
      std::vector<int> up(n), d0(n), d1(n);
      for (int r = 0; r < n; ++r) CHECK(ar_oracle_dtree(n, r, t, &up[r], &d0[r], &d1[r]) == 0);
      int roots = 0;
      for (int r = 0; r < n; ++r) {
        if (up[r] < 0) ++roots;
        else CHECK(up[r] < n && (d0[up[r]] == r || d1[up[r]] == r));
        if (d0[r] >= 0) CHECK(d0[r] < n && up[d0[r]] == r);
        if (d1[r] >= 0) CHECK(d1[r] < n && up[d1[r]] == r);
      }
      CHECK(roots == 1);
    }
    int a, b, c, d;
    CHECK(ar_oracle_btree(n, n, &a, &b, &c, &d) != 0);
  }
}

// Cost model and table over a sweep of sizes, ranks and channel caps.
static void tuner() {
  arTuneModel_t m[3] = {{8.f, 0.6f, 20.f, 60.f}, {9.f, 0.8f, 25.f, 300.f}, {10.f, 1.f, 30.f, 700.f}};
  for (int n : {1, 2, 3, 8, 17, 72, 128, 200}) {
    for (int ch : {0, 1, 7, 64, 65}) {
      for (size_t b = 0; b <= ((size_t)1 << 34); b = b ? b * 5 : 1) {
        arProto_t p;
        arAlgo_t al;
        int nch = 0;
        float us = 0.f;
        const arResult_t r = arTuneEval(n, ch, b, m, 7u, &p, &nch, &us);
        if (r == arSuccess && !(p >= arProtoLL && p <= arProtoSimple && nch >= (n > 1) && nch <= ch)) {
          fprintf(stderr, "check failed: arTuneEval n=%d ch=%d b=%zu -> proto %d nch %d\n", n, ch, b, (int)p, nch);
          ++failures;
        }
        for (int f = 0; f < 3; ++f)
          (void)arTuneEvalColl((arFunc_t)f, n, ch, b, m, (unsigned)(b % 8), &p, &nch, &us);
        (void)arTuneEvalAlgo(arFuncAllReduce, n, ch, b, m, m, 3u, 7u, &al, &p, &nch, &us);
        (void)arTuneEvalAlgo(arFuncAllReduce, n, ch, b, m, nullptr, 1u, 7u, &al, &p, &nch, &us);
        for (int a2 = 0; a2 < 2; ++a2)
          for (int p2 = 0; p2 < 3; ++p2)
            if (arTuneTableTime(n, b, (arAlgo_t)a2, (arProto_t)p2, &us) == arSuccess) CHECK(us > 0.f);
      }
    }
  }
  arProto_t p;
  int nch;
  float us;
  CHECK(arTuneEval(8, 64, 1024, nullptr, 7u, &p, &nch, &us) != arSuccess);
  CHECK(arTuneEval(8, 64, 1024, m, 0u, &p, &nch, &us) != arSuccess);
  CHECK(arTuneTableTime(8, 1024, (arAlgo_t)5, arProtoSimple, &us) != arSuccess);
}

// Group aggregation: a permutation, launches numbered from 0, consecutive.
static void groups(std::mt19937& rng) {
  for (int trial = 0; trial < 300; ++trial) {
    const int n = (int)(rng() % 40);
    std::vector<int> keys(n), iso(n), order(n, -1), launchOf(n, -1);
    std::vector<size_t> bytes(n);
    for (int i = 0; i < n; ++i) {
      keys[i] = (int)(rng() % 4);
      bytes[i] = (size_t)1 << (rng() % 30);
      iso[i] = rng() % 7 == 0;
    }
    int nl = -1;
    CHECK(arGroupAggregate(n, keys.data(), bytes.data(), iso.data(), order.data(), launchOf.data(), &nl) ==
          arSuccess);
    std::vector<int> seen(n, 0);
    for (int i = 0; i < n; ++i) {
      CHECK(order[i] >= 0 && order[i] < n);
      if (order[i] >= 0 && order[i] < n) ++seen[order[i]];
      CHECK(launchOf[i] >= 0 && launchOf[i] < nl);
      if (i > 0 && order[i] >= 0 && order[i - 1] >= 0)
        CHECK(launchOf[order[i]] == launchOf[order[i - 1]] || launchOf[order[i]] == launchOf[order[i - 1]] + 1);
    }
    for (int i = 0; i < n; ++i) CHECK(seen[i] == 1);
  }
  int nl;
  CHECK(arGroupAggregate(-1, nullptr, nullptr, nullptr, nullptr, nullptr, &nl) != arSuccess);
  CHECK(arGroupAggregate(3, nullptr, nullptr, nullptr, nullptr, nullptr, &nl) != arSuccess);
}

int main() {
  std::mt19937 rng(20261202);
  oracles(rng);
  trees();
  tuner();
  groups(rng);
  printf("sanitized host code: %d check failures\n", failures);
  return failures == 0 ? 0 : 1;
}
