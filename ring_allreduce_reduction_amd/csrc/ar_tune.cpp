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
#include <stddef.h>
#include <stdint.h>

#include "ar.h"

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
