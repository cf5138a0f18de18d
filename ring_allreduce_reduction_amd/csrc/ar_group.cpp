// ar_group.cpp -- which collectives of a group share one launch.
//
// ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.6 §四 ncclPrepareTasks]:
// the tasks of a group leave the sorter largest traffic first; they are
// bucketed by (function, op, data type), buckets visited in index order;
// inside a bucket, consecutive tasks of similar size are aggregated into one
// launch unless a task is isolated (aggIsolate).  The pages print the size
// test as aggEnd < 4 * aggBeg, which every task of a descending list passes;
// with "similar size (within 4x)" stated beside it, the reading here is that
// a task joins while 4 * its traffic exceeds the first task's.
#include <stddef.h>

#include <algorithm>
#include <map>
#include <numeric>
#include <vector>

#include "ar.h"

extern "C" arResult_t arGroupAggregate(int nTasks, const int* keys, const size_t* bytes, const int* isolate,
                                       int* order, int* launchOf, int* nLaunches) {
  if (nTasks < 0 || (nTasks > 0 && (keys == nullptr || bytes == nullptr || order == nullptr ||
                                    launchOf == nullptr)) || nLaunches == nullptr)
    return arInvalidArgument;
  std::vector<int> sorted((size_t)nTasks);
  std::iota(sorted.begin(), sorted.end(), 0);
  // largest first; equal sizes keep call order
  std::stable_sort(sorted.begin(), sorted.end(), [&](int x, int y) { return bytes[x] > bytes[y]; });
  std::map<int, std::vector<int>> buckets;
  for (int i : sorted) buckets[keys[i]].push_back(i);
  int launch = 0, pos = 0;
  for (auto& kv : buckets) {
    const std::vector<int>& list = kv.second;
    for (size_t i = 0; i < list.size();) {
      const int beg = list[i];
      size_t j = i + 1;
      if (!(isolate && isolate[beg]))
        while (j < list.size() && !(isolate && isolate[list[j]]) && bytes[list[j]] * 4 > bytes[beg]) ++j;
      for (size_t q = i; q < j; ++q) {
        order[pos++] = list[q];
        launchOf[list[q]] = launch;
      }
      ++launch;
      i = j;
    }
  }
  *nLaunches = launch;
  return arSuccess;
}
