// Launch descriptors of the grouped decode-and-multiply kernel (internal to libsage).
#pragma once

#include "sage_internal.hpp"

namespace sage {

constexpr int kWaves = 4;                     // row tiles (wavefronts) per workgroup
constexpr int kMaxGroupsPerSplit = 8;         // column groups one workgroup handles
constexpr int kMaxJobs = 16;
constexpr int kWholeXMax = 16384;           // inputs up to this width are staged whole in LDS

// One product y = W x, possibly repeated over `inst` instances (routed experts). The matrix comes
// either from the direct fields or, when `table` is set, from table[ids[instance]*tstride + toff]
// in device memory.
struct Job {
  const uint8_t* packed;
  const uint16_t* codebook;
  const int32_t* pi;
  const sage_matrix_t* table;
  const int32_t* ids;
  const uint16_t* x;
  uint16_t* y;
  float* partial;
  uint32_t* counters;
  int64_t x_stride;        // elements between the inputs of consecutive instances
  int64_t y_stride;        // elements between the outputs of consecutive instances
  int64_t partial_stride;  // floats of split-K partials per instance
  int32_t tstride, toff, n_experts;
  int32_t log2K;
  int32_t d_out, d_in;
  int32_t rt, ng, wgr;     // row tiles, column groups, workgroup rows (= ceil(rt / kWaves))
  int32_t S, gs;           // column splits and groups per split
  int32_t wg_begin, wg_per_inst, inst;
  int32_t counters_stride;
};

struct JobTable {
  int32_t wg_begin[kMaxJobs];  // first workgroup of each job (unused entries: INT32_MAX)
  int32_t n;
  int32_t total_wg;
  Job jobs[kMaxJobs];
};

static_assert(sizeof(JobTable) <= 3072, "kernel argument block too large");

}  // namespace sage
