// Launch descriptors of the grouped decode-and-multiply kernel (internal to libsage).
#pragma once

#include "sage_internal.hpp"

namespace sage {

// Workgroup shapes: T row tiles x (16 / T) column parts, one wavefront each (16 waves, 1024
// threads). The parts of a row tile split the workgroup's columns and add their partial sums in
// LDS. T = 4 is the general shape; T = 2 and T = 1 put more parts on a tile, so fewer workgroups
// of other compute units have to combine split-K partials (planner in sage_gemv.hip).
// T = 0 is the chunked shape for unsplit launches: the workgroup owns Q chunks of 16 rows (not
// tied to 64-row tiles) and each 16-lane group of a wave works on one chunk, so a launch can
// spread its rows over every compute unit without split-K.
constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
__host__ __device__ constexpr int shape_max_gs(int T) {
  return T == 4 ? 8 : (T == 2 ? 20 : (T == 0 ? 32 : 24));
}
template <int T>
struct WgShape {
  static constexpr int kTiles = T == 0 ? 1 : T;
  static constexpr int kParts = kWaves / kTiles;
  static constexpr int kMaxGS = shape_max_gs(T);                              // groups per workgroup
  static constexpr int kMaxUnits = T == 0 ? 5 : (2 * kMaxGS + kParts - 1) / kParts;  // per wave
};
constexpr int kChunkRows = 16;
constexpr int kMaxChunkUnits = 5;   // half-groups per lane group in the chunked shape
constexpr int kStreamSteps = 2;     // half-group steps per wave and block of the persistent shape
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
  // chunked shape: chunks per workgroup, first chunk and chunks of the piece
  int32_t cq, chunk0, nchunk;
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

// Work map of the chunked shape, built by the planner (the same for every piece of a launch).
//   lane_group[4 w + g]  lane group g of wave w: chunk (bits 0-3), half-groups (bits 4-7), first
//                        half-group (bits 8-15)
//   wave[w]              bits 0-7: half-group steps of wave w (its longest lane group); bits
//                        8-15: lane groups of wave w that share a chunk and add up inside the
//                        wave first (0 none, 1 g and g + 2, 2 all four)
//   red[c]               contributors to chunk c after that: lane groups first + i * step for
//                        i < count (bits 0-5 first, 6-11 step, 12-19 count), added in that order
struct ChunkMap {
  uint16_t lane_group[kWaves * 4];
  uint32_t wave[kWaves];
  uint32_t red[8];
};

// Kernel argument: blockIdx.y selects the piece, blockIdx.x the workgroup inside it.
struct JobTable {
  Job jobs[kMaxJobs];
  ChunkMap cmap;
};

static_assert(sizeof(JobTable) <= 4096, "kernel argument block too large");

}  // namespace sage
