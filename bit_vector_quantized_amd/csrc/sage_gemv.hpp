// Launch descriptors of the grouped decode-and-multiply kernel (internal to libsage).
#pragma once

#include "sage_internal.hpp"

namespace sage {

// Workgroup shapes: T row tiles x (16 / T) column parts, one wavefront each (16 waves, 1024
// threads). The parts of a row tile split the workgroup's columns and add their partial sums in
// LDS. T = 4 is the general shape; T = 2 and T = 1 put more parts on a tile, so fewer workgroups
// of other compute units have to combine split-K partials (planner in sage_gemv.hip).
constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
template <int T>
struct WgShape {
  static constexpr int kTiles = T;
  static constexpr int kParts = kWaves / T;
  static constexpr int kMaxGS = T == 4 ? 8 : (T == 2 ? 20 : 24);           // groups per workgroup
  static constexpr int kMaxUnits = (2 * kMaxGS + kParts - 1) / kParts;     // half-groups per wave
};
__host__ __device__ constexpr int shape_max_gs(int T) { return T == 4 ? 8 : (T == 2 ? 20 : 24); }
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
  int32_t tile0, rt, rq;    // first row tile, row tiles, tile blocks (ceil(rt / T)) of the piece
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
