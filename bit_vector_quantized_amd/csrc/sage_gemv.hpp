// Launch descriptors of the grouped decode-and-multiply kernel (internal to libsage).
#pragma once

#include "sage_internal.hpp"

namespace sage {

// Workgroup shape: kTiles row tiles x kParts column parts, one wavefront each. The kParts waves of
// a row tile split the workgroup's columns and add their partial sums in LDS.
constexpr int kTiles = 4;
constexpr int kParts = 4;
constexpr int kWaves = kTiles * kParts;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxGroupsPerSplit = 8;                         // column groups per workgroup
constexpr int kMaxUnits = 2 * kMaxGroupsPerSplit / kParts;    // half-groups per wavefront
constexpr int kMaxJobs = 16;
constexpr int kWholeXMax = 16384;  // inputs up to this width are staged whole in LDS

// One launch piece: row tiles [tile0, tile0 + rt) of a product y = W x, possibly repeated over
// `inst` instances (routed experts). The matrix comes either from the direct fields or, when
// `table` is set, from table[ids[instance] * tstride + toff] in device memory.
struct Job {
  const uint8_t* packed;
  const uint16_t* codebook;
  const int32_t* pi;
  const sage_matrix_t* table;
  const int32_t* ids;
  const uint16_t* x;
  uint16_t* y;
  float* partial;           // split-K partials [inst][S][rt * 64]
  uint32_t* counters;       // arrival counters [inst][rq]
  int64_t x_stride;         // elements between the inputs of consecutive instances
  int64_t y_stride;         // elements between the outputs of consecutive instances
  int64_t partial_stride;   // floats of split-K partials per instance
  int32_t tstride, toff, n_experts;
  int32_t log2K;
  int32_t d_out, d_in;      // the whole matrix
  int32_t tile0, rt, rq;    // first row tile, row tiles, row quads (ceil(rt / kTiles)) of the piece
  int32_t ng;               // column groups of the matrix
  int32_t S, gs;            // column splits and groups per split
  int32_t wg_per_inst, inst;
  int32_t counters_stride;
  // Fused two-stage launches (SwiGLU MLP). A producer piece also writes its rows in fp32 to
  // out32 with coherent stores and signals sync[0] once per finished row group; a consumer piece
  // (src_gate set) waits until sync[0] reaches signal_total, then takes its input from
  // fp16(silu(fp16(gate)) * fp16(up)) of the producers' fp32 rows. sync[1] counts consumers that
  // passed the wait (the last one resets sync[0..1]); sync[2] counts waits that timed out.
  float* out32;
  const float* src_gate;
  const float* src_up;
  uint32_t* sync;
  uint16_t* h_out;          // optional fp16 copy of the consumer input (one workgroup writes it)
  int32_t signal_total;
  int32_t consumer_wgs;
};

// Kernel argument: blockIdx.y selects the piece, blockIdx.x the workgroup inside it.
struct JobTable {
  Job jobs[kMaxJobs];
};

static_assert(sizeof(JobTable) <= 4096, "kernel argument block too large");

}  // namespace sage
