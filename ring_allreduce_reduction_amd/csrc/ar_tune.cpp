// ar_tune.cpp -- the ring and tree cost models and algorithm / protocol /
// channel selection.
//
// Model form ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.5 §三 ring.cc]:
//   busBw = bw * nChannels; LL: min(llMaxBw, 0.5 * busBw) (half of every LL
//   line is flag); LL128: min(0.92 * busBw, cap) (120 of 128 bytes payload);
//   algBw = busBw * nRanks / nSteps with nSteps = 2(nRanks - 1) for AllReduce;
//   lat = baseLat + nSteps * stepLat (one node: every step is intra).
// Time ["NCCL 源码解析：从硬件拓扑到集合通信选型的完整链路", §五]:
//   time = lat * latCount + nBytes / (1000 * bw)   (us, GB/s), latCount = 1.
// Selection [same book, ch.5 §一]: one rank short-cuts to Simple with 0
// channels; otherwise the argmin over the candidates, protocols visited in the
// order the reference's head-inserted list yields (Simple, LL128, LL) with a
// strict <, so protocol ties keep Simple.  The pages name no channel rule
// beyond "interpolate by size"; candidates here are the powers of two up to
// the maximum whose share is at least the planner's 32 KiB minimum traffic per
// channel [same book, ch.6 §五].  Within a protocol a channel-count tie keeps
// the larger count: every channel runs in the same single launch here, and on
// MI355X extra channels past the bandwidth cap still spread the work better.
// Tree model [same book, ch.5 §四, tree.cc]: AllReduce only; busBw = bw * nChannels
// * 0.92, then LL x 1/3.8 and LL128 x 120/128 (the multi-node factor: every
// virtual rank is its own tree node here), capped; the pages give the tree
// no nRanks/nSteps ratio, so algBw = busBw; lat = baseLat + 2 * log2i(N) *
// stepLat (N / nNodes - 1 = 0 intra-node steps, log2i(nNodes) tree levels each
// way); and for AllReduce bw *= treeCorrectionFactor[proto][log2i(nBytes >>
// 6)] when that index is in [0, 23).  Candidates are visited ring first (its
// Simple, LL128, LL), then tree, with a strict <: ties keep the ring, the
// order the pages' head-inserted candidate list gives when the ring's
// candidates are registered after the tree's.
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <array>
#include <mutex>
#include <vector>

#include "ar.h"
#include "ar_tune_table.h"

#include "ar_tune_table.inc"

namespace {

constexpr size_t kMinBytesPerChannel = 32 * 1024;

float candidateTime(const arTuneModel_t& m, int proto, int nranks, int nSteps, int nch, size_t nBytes) {
  float busBw = m.bwPerChGBs * (float)nch;
  if (proto == arProtoLL) busBw = busBw * 0.5f;
  else if (proto == arProtoLL128) busBw = busBw * 0.92f;
  if (busBw > m.maxBwGBs) busBw = m.maxBwGBs;
  const float algBw = busBw * (float)nranks / (float)nSteps;
  const float lat = m.baseLatUs + (float)nSteps * m.stepLatUs;
  return lat * 1.0f + (float)nBytes / (1000.0f * algBw);
}

bool validModel(const arTuneModel_t& m) {
  return m.bwPerChGBs > 0.0f && m.maxBwGBs > 0.0f && m.baseLatUs >= 0.0f && m.stepLatUs >= 0.0f;
}

// The pages' empirical tree efficiency by message size, rows LL, LL128,
// Simple; column i covers 64 B * 2^i [same book, ch.5 §四, the
// treeCorrectionFactor table of cost_model.cc].
const float kTreeCorrection[3][24] = {
    {1.0f, 1.0f, 1.0f, 1.0f, .9f, .8f, .7f, .7f, .7f, .7f, .6f, .5f, .4f, .4f, .5f, .6f, .7f, .8f, .9f, 1.0f,
     1.0f, 1.0f, 1.0f, 1.0f},
    {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, .9f, .8f, .8f, .8f, .7f, .6f, .6f, .6f, .6f, .6f, .6f, .8f, .9f, .9f, .9f,
     .9f, 1.0f, 1.0f, 1.0f},
    {.9f, .9f, .9f, .9f, .9f, .9f, .9f, .8f, .7f, .6f, .6f, .5f, .5f, .5f, .5f, .6f, .7f, .8f, .7f, .7f, .8f,
     .9f, .9f, .9f}};

int log2i(uint64_t n) {   // floor(log2(n)), -1 for 0
  int l = -1;
  while (n) {
    n >>= 1;
    ++l;
  }
  return l;
}

float treeTime(const arTuneModel_t& m, int proto, int nranks, int nch, size_t nBytes) {
  float busBw = m.bwPerChGBs * (float)nch * 0.92f;
  if (proto == arProtoLL) busBw = busBw * (1.0f / 3.8f);
  else if (proto == arProtoLL128) busBw = busBw * (120.0f / 128.0f);
  if (busBw > m.maxBwGBs) busBw = m.maxBwGBs;
  const int logSize = log2i((uint64_t)nBytes >> 6);
  if (logSize >= 0 && logSize < 23) busBw *= kTreeCorrection[proto][logSize];
  const float lat = m.baseLatUs + 2.0f * (float)log2i((uint64_t)nranks) * m.stepLatUs;
  return lat * 1.0f + (float)nBytes / (1000.0f * busBw);
}

}  // namespace

extern "C" arResult_t arTuneEvalAlgo(arFunc_t func, int nranks, int maxChannels, size_t nBytes,
                                     const arTuneModel_t* ringModels, const arTuneModel_t* treeModels,
                                     unsigned algoMask, unsigned protoMask, arAlgo_t* algo, arProto_t* proto,
                                     int* nChannels, float* predictedUs) {
  if (nranks < 1 || maxChannels < 1) return arInvalidArgument;
  if (func != arFuncAllReduce && func != arFuncReduceScatter && func != arFuncAllGather) return arInvalidArgument;
  if ((protoMask & 7u) == 0 || (algoMask & 3u) == 0) return arInvalidArgument;
  if (((algoMask & 1u) && ringModels == nullptr) || ((algoMask & 2u) && treeModels == nullptr))
    return arInvalidArgument;
  // ring steps per call [ch.5 §三]: 2(N-1) for AllReduce, N-1 for the halves
  const int nSteps = func == arFuncAllReduce ? 2 * (nranks - 1) : nranks - 1;
  if (nranks == 1) {
    if (algo) *algo = arAlgoRing;
    if (proto) *proto = arProtoSimple;
    if (nChannels) *nChannels = 0;
    if (predictedUs) *predictedUs = 0.0f;
    return arSuccess;
  }
  static const int order[3] = {arProtoSimple, arProtoLL128, arProtoLL};
  float best = FLT_MAX;
  int bestAlgo = -1, bestProto = -1, bestCh = 0;
  for (int al = arAlgoRing; al <= arAlgoTree; ++al) {
    if (!(algoMask & (1u << al))) continue;
    if (al == arAlgoTree && func != arFuncAllReduce) continue;   // the tree serves AllReduce only
    const arTuneModel_t* models = al == arAlgoRing ? ringModels : treeModels;
    for (int i = 0; i < 3; ++i) {
      const int p = order[i];
      if (!(protoMask & (1u << p)) || !validModel(models[p])) continue;
      float bestP = FLT_MAX;
      int bestChP = 0;
      for (int nch = 1; nch <= maxChannels; nch *= 2) {
        if (nch > 1 && nBytes / (size_t)nch < kMinBytesPerChannel) break;
        const float t = al == arAlgoRing ? candidateTime(models[p], p, nranks, nSteps, nch, nBytes)
                                         : treeTime(models[p], p, nranks, nch, nBytes);
        if (t <= bestP) {
          bestP = t;
          bestChP = nch;
        }
      }
      if (bestP < best) {
        best = bestP;
        bestAlgo = al;
        bestProto = p;
        bestCh = bestChP;
      }
    }
  }
  if (bestProto < 0) return arInvalidUsage;
  if (algo) *algo = (arAlgo_t)bestAlgo;
  if (proto) *proto = (arProto_t)bestProto;
  if (nChannels) *nChannels = bestCh;
  if (predictedUs) *predictedUs = best;
  return arSuccess;
}

extern "C" arResult_t arTuneEvalColl(arFunc_t func, int nranks, int maxChannels, size_t nBytes,
                                     const arTuneModel_t* models, unsigned protoMask, arProto_t* proto,
                                     int* nChannels, float* predictedUs) {
  if (models == nullptr) return arInvalidArgument;
  return arTuneEvalAlgo(func, nranks, maxChannels, nBytes, models, nullptr, 1u << arAlgoRing, protoMask, nullptr,
                        proto, nChannels, predictedUs);
}

extern "C" arResult_t arTuneEval(int nranks, int maxChannels, size_t nBytes, const arTuneModel_t* models,
                                 unsigned protoMask, arProto_t* proto, int* nChannels, float* predictedUs) {
  return arTuneEvalColl(arFuncAllReduce, nranks, maxChannels, nBytes, models, protoMask, proto, nChannels,
                        predictedUs);
}

// ---------------------------------------------------------------- the tuner's time table
//
// The pages let a tuner plugin see the cost of every (algorithm, protocol)
// candidate and override it before the argmin ["NCCL 原始碼解讀：一個
// AllReduce 的 GPU 旅程", ch.5 §一, step 3; "NCCL 源码解析：从硬件拓扑到集合通信
// 选型的完整链路", §五, the tuner plugin].  The overriding costs here are
// times measured on MI355X: one line per (ranks, bytes per rank) with the six
// candidates' microseconds, compiled in from the calibration record
// (ar_tune_table.txt) or read from the file AR_TUNE_FILE names.  A query
// between lines is interpolated log-log in bytes along each rank count's
// lines, then log-log between the two nearest rank counts; past a rank
// count's largest size the time grows in proportion to the bytes.  Rank
// counts outside the table are not covered (the cost model decides).

namespace {

struct TableRank {
  int nranks;
  std::vector<uint64_t> bytes;        // ascending
  std::vector<std::array<float, 6>> us;   // < 0: that candidate cannot run
};

struct TuneTable {
  std::vector<TableRank> ranks;       // ascending nranks
  bool haveModels[2][3] = {};
  arTuneModel_t models[2][3] = {};    // [algo][proto], from "model" lines
};

void addRow(TuneTable& t, int n, uint64_t bytes, const float us[6]) {
  auto it = std::find_if(t.ranks.begin(), t.ranks.end(), [&](const TableRank& r) { return r.nranks >= n; });
  if (it == t.ranks.end() || it->nranks != n) {
    TableRank r;
    r.nranks = n;
    it = t.ranks.insert(it, r);
  }
  auto jt = std::lower_bound(it->bytes.begin(), it->bytes.end(), bytes);
  const size_t j = (size_t)(jt - it->bytes.begin());
  std::array<float, 6> a;
  for (int k = 0; k < 6; ++k) a[k] = us[k];
  if (jt != it->bytes.end() && *jt == bytes) {
    it->us[j] = a;
  } else {
    it->bytes.insert(jt, bytes);
    it->us.insert(it->us.begin() + (ptrdiff_t)j, a);
  }
}

// Parse a table file; false (with a warning) if it holds a malformed line or no line.
bool parseTableFile(const char* path, TuneTable& t) {
  FILE* f = fopen(path, "r");
  if (f == nullptr) {
    fprintf(stderr, "[ar] WARN AR_TUNE_FILE=%s cannot be opened; using the compiled table\n", path);
    return false;
  }
  char line[1024];
  int lineNo = 0, rows = 0;
  bool ok = true;
  while (ok && fgets(line, sizeof(line), f) != nullptr) {
    ++lineNo;
    if (char* h = strchr(line, '#')) *h = 0;
    char* tok[16];
    int nt = 0;
    for (char* p = strtok(line, " \t\r\n"); p != nullptr && nt < 16; p = strtok(nullptr, " \t\r\n")) tok[nt++] = p;
    if (nt == 0) continue;
    if (!strcmp(tok[0], "model")) {
      const int al = nt == 7 ? (!strcmp(tok[1], "ring") ? 0 : !strcmp(tok[1], "tree") ? 1 : -1) : -1;
      const int pr = nt == 7 ? (!strcmp(tok[2], "ll") ? 0 : !strcmp(tok[2], "ll128") ? 1 : !strcmp(tok[2], "simple") ? 2 : -1)
                             : -1;
      if (al < 0 || pr < 0) {
        ok = false;
        break;
      }
      arTuneModel_t m = {(float)atof(tok[3]), (float)atof(tok[4]), (float)atof(tok[5]), (float)atof(tok[6])};
      if (!(m.bwPerChGBs > 0.0f) || !(m.maxBwGBs > 0.0f) || m.baseLatUs < 0.0f || m.stepLatUs < 0.0f) {
        ok = false;
        break;
      }
      t.models[al][pr] = m;
      t.haveModels[al][pr] = true;
      continue;
    }
    if (nt != 8) {
      ok = false;
      break;
    }
    const long n = strtol(tok[0], nullptr, 10);
    const unsigned long long b = strtoull(tok[1], nullptr, 10);
    float us[6];
    for (int k = 0; k < 6; ++k) us[k] = !strcmp(tok[2 + k], "-") ? -1.0f : (float)atof(tok[2 + k]);
    if (n < 2 || n > AR_MAX_RANKS || b == 0) {
      ok = false;
      break;
    }
    addRow(t, (int)n, (uint64_t)b, us);
    ++rows;
  }
  fclose(f);
  if (!ok || rows == 0) {
    fprintf(stderr, "[ar] WARN AR_TUNE_FILE=%s: bad line %d (or no table line); using the compiled table\n", path,
            lineNo);
    return false;
  }
  return true;
}

// The table in force, read once per process: AR_TUNE_FILE if it parses, else
// the compiled one [the reference's parameter cache, ch.3 §3.5].
const TuneTable& table() {
  static TuneTable t;
  static std::once_flag once;
  std::call_once(once, [] {
    TuneTable f;
    for (int p = 0; p < 3; ++p) {   // the compiled constants, unless the file names others
      f.models[0][p] = kCompiledRingModels[p];
      f.models[1][p] = kCompiledTreeModels[p];
      f.haveModels[0][p] = f.haveModels[1][p] = true;
    }
    const char* path = getenv("AR_TUNE_FILE");
    if (path != nullptr && *path != 0) {
      TuneTable g = f;
      if (parseTableFile(path, g)) {
        t = g;
        return;
      }
    }
    for (const ar::TuneRow& r : kCompiledTuneRows) addRow(f, r.nranks, r.bytes, r.us);
    t = f;
  });
  return t;
}

// One rank count's time for a candidate at `bytes`, or a negative value where
// a line it needs marks the candidate as unable to run.
float rankTime(const TableRank& r, uint64_t bytes, int k) {
  const size_t m = r.bytes.size();
  size_t hi = 0;   // first line with at least `bytes`
  while (hi < m && r.bytes[hi] < bytes) ++hi;
  if (hi == 0) return r.us[0][(size_t)k];             // at or below the smallest size: its time
  const size_t lo = hi - 1;
  const float tl = r.us[lo][(size_t)k];
  if (hi == m)                                        // past the largest: in proportion to the bytes
    return tl < 0.0f ? -1.0f : tl * (float)((double)bytes / (double)r.bytes[lo]);
  const float th = r.us[hi][(size_t)k];
  if (r.bytes[hi] == bytes) return th;
  if (tl < 0.0f || th < 0.0f) return -1.0f;
  const double w = (log((double)bytes) - log((double)r.bytes[lo])) / (log((double)r.bytes[hi]) - log((double)r.bytes[lo]));
  return (float)exp((1.0 - w) * log((double)tl) + w * log((double)th));
}

}  // namespace

bool ar::tuneTableTime(int nranks, uint64_t nBytes, int algo, int proto, float* us) {
  const TuneTable& t = table();
  if (algo < 0 || algo > 1 || proto < 0 || proto > 2 || nBytes == 0 || t.ranks.empty()) return false;
  if (nranks < t.ranks.front().nranks || nranks > t.ranks.back().nranks) return false;
  const int k = algo * 3 + proto;
  size_t i = 0;
  while (t.ranks[i].nranks < nranks) ++i;   // first rank count >= nranks
  float v;
  if (t.ranks[i].nranks == nranks) {
    v = rankTime(t.ranks[i], nBytes, k);
  } else {
    const TableRank& a = t.ranks[i - 1];
    const TableRank& b = t.ranks[i];
    const float ta = rankTime(a, nBytes, k), tb = rankTime(b, nBytes, k);
    if (ta < 0.0f || tb < 0.0f) return false;
    const double w = (log((double)nranks) - log((double)a.nranks)) / (log((double)b.nranks) - log((double)a.nranks));
    v = (float)exp((1.0 - w) * log((double)ta) + w * log((double)tb));
  }
  if (v < 0.0f) return false;
  *us = v;
  return true;
}

bool ar::tuneTableCovers(int nranks) {
  const TuneTable& t = table();
  return !t.ranks.empty() && nranks >= t.ranks.front().nranks && nranks <= t.ranks.back().nranks;
}

void ar::tuneTableModels(arTuneModel_t ring[3], arTuneModel_t tree[3]) {
  const TuneTable& t = table();
  for (int p = 0; p < 3; ++p) {
    if (t.haveModels[0][p]) ring[p] = t.models[0][p];
    if (t.haveModels[1][p]) tree[p] = t.models[1][p];
  }
}

extern "C" arResult_t arTuneTableTime(int nranks, size_t nBytes, arAlgo_t algo, arProto_t proto, float* predictedUs) {
  if (predictedUs == nullptr || nranks < 1 || nBytes == 0) return arInvalidArgument;
  if (algo != arAlgoRing && algo != arAlgoTree) return arInvalidArgument;
  if (proto != arProtoLL && proto != arProtoLL128 && proto != arProtoSimple) return arInvalidArgument;
  return ar::tuneTableTime(nranks, (uint64_t)nBytes, (int)algo, (int)proto, predictedUs) ? arSuccess : arInvalidUsage;
}
