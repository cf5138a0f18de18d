// ar_tune_table.h -- the tuner's measured time table (ar_tune.cpp), as used
// by the comm's selection in ar_comm.cpp.  Nothing here is in the C ABI
// beyond arTuneTableTime.
#pragma once

#include <stdint.h>

#include "ar.h"

namespace ar {

// One line of the table: microseconds per AllReduce of ring LL, LL128,
// Simple and tree LL, LL128, Simple (< 0: that candidate cannot run there).
struct TuneRow {
  int nranks;
  uint64_t bytes;
  float us[6];
};

// The table's time of (algo, proto) for `nranks` ranks and nBytes per rank
// (interpolated); false where the table does not cover them.
bool tuneTableTime(int nranks, uint64_t nBytes, int algo, int proto, float* us);

// Whether the table holds rank counts on both sides of (or equal to) nranks.
bool tuneTableCovers(int nranks);

// The cost-model constants that come with the table in force (compiled, or
// the "model" lines of AR_TUNE_FILE): each entry the table names is written.
void tuneTableModels(arTuneModel_t ring[3], arTuneModel_t tree[3]);

}  // namespace ar
