// Small-batch product Y = X W_hat^T for SAGE-packed weights on gfx950 matrix cores (SAGE paper §3.5
// and App. A.1: each weight is decoded once per output tile and reused across the activation rows).
//
// MFMA mapping. A wavefront owns 16 weight rows and computes D = A * B with
// v_mfma_f32_16x16x32_f16: B is 32 input channels x 16 weight rows, A is 16 activation rows x the
// same 32 channels. In the B operand a lane supplies 8 consecutive input channels of one weight row,
// which is exactly one subvector, so the lane decodes its subvector straight into the operand:
// w_i = r_hat * (+-c_z,i), r_hat = mu + q*delta computed in fp32, the product formed in fp16. Lanes
// 16u..16u+15 of MFMA step kk supply subvector 4u + kk of their row, so A reads the same channels;
// the channel order inside the 32-wide contraction is the same for A and B. One decoded subvector
// feeds NT = 1, 2 or 4 MFMAs (16, 32 or 64 activation rows).
//
// Workgroup: 16 wavefronts = T weight tiles of 64 rows (4 waves of 16 rows each) x 4/T column
// parts. It owns a range of column groups (split-K over workgroups) and one chunk of activation
// rows; the column parts add their accumulators in LDS. Up to 16 rows the activations of its
// columns are staged once in LDS (gathered through pi below 8 rows, §3.2) and shared by the tiles;
// from 17 rows they stream through LDS one column group per part at a time (1 x 4), so a 64-row
// tile can take every group of its row without split-K. All packed-weight loads of a wave are
// issued up front through range-checked buffer loads, as in the batch-one kernel.
#include <algorithm>
#include <mutex>

#include "sage_internal.hpp"

namespace sage {
namespace {

// Small-batch workgroup shapes: T 64-row weight tiles (four 16-row quarter waves each) x 4/T
// column parts, 16 waves. T = 2 is the general shape; T = 1 gives each tile 4 parts, so a row
// tile can take all its column groups without split-K.
constexpr int kGWaves = 16;
constexpr int kGThreads = kGWaves * 64;              // 1024
template <int T>
struct GShape {
  static constexpr int kTiles = T;
  static constexpr int kParts = 4 / T;
  static constexpr int kMaxGS = T == 2 ? 8 : 20;                            // groups per split
  static constexpr int kMaxUnits = (kMaxGS + kParts - 1) / kParts;          // groups per wave
};
inline int gshape_max_gs(int T) { return T == 2 ? 8 : 20; }
constexpr int kPermuteMinRows = 8;                   // from this many rows on, X is permuted once
constexpr int kDirectRows = kPermuteMinRows;         // rows gathered straight from X below that
constexpr int kPrefillMinRows = 128;                 // prefill kernel candidates from this many rows
constexpr uint32_t kNowhere = 1u << 30;              // an offset past every range

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct GemmArgs {
  const uint8_t* packed;
  const uint16_t* codebook;
  const int32_t* pi;
  const uint16_t* X;
  uint16_t* Y;
  float* partial;       // [mchunk][split][mrows_chunk][rt * 64]
  uint32_t* counters;   // [mchunk][rpairs] (rpairs = tile blocks of the shape)
  int64_t ldx, ldy;
  int32_t d_out, d_in, M, L;
  int32_t rt, rpairs, ng, S, gs, mchunks;
  int32_t mrows_chunk;  // activation rows per workgroup = 16 * NT
  int32_t vec_x;        // X rows are 16-byte aligned and already in permuted order (kVec)
  int32_t tiles;        // workgroup shape (GShape<tiles>)
  int32_t stream;       // activations streamed through LDS a group at a time (1 x 4 shape)
};

__device__ inline __amdgpu_buffer_rsrc_t view(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// X[:, pi] for M rows into a dense [M][d_in] buffer (the reorder the paper does once per
// projection before prefill, §3.5). A workgroup copies kR whole rows of X into LDS (all its
// 16-byte loads issued before any is stored), then each thread gathers 8 consecutive outputs of
// the workgroup's column range (blockIdx.y, `units` 8-column units each) through pi from LDS, pi
// read once for all kR rows, and writes them as one 16-byte store. kR * J <= 16, J = row loads
// per thread = ceil(d_in / 2048).
constexpr int kPermLoads = 16;
constexpr int kPermLdsMinRows = 128;

template <int kR>
__global__ void __launch_bounds__(256) permute_rows_kernel(const uint16_t* __restrict__ X,
                                                           int64_t ldx,
                                                           const int32_t* __restrict__ pi,
                                                           int d_in, int M, int units,
                                                           uint16_t* __restrict__ Xp) {
  constexpr int kJ = kPermLoads / kR;
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * kR;
  const int nr = min(M - m0, kR);
  const int row_units = d_in >> 3;
  const uint32_t last = (uint32_t)d_in - 1u;
  const int c0 = blockIdx.y * units + tid;
  const int c1 = min(row_units, (int)(blockIdx.y + 1) * units);
  // Every load is issued unconditionally through a range-checked view (an offset outside the view
  // reads zeros without touching memory), so all of them are in flight together: the permutation
  // entries of the thread's first two 8-column units and its 16-byte chunks of the kR rows.
  const __amdgpu_buffer_rsrc_t pi_rs = view(pi, pi ? (uint32_t)d_in * 4u : 0u);
  u32x4 pv[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = c0 + i * 256;
    const uint32_t off = c < c1 ? (uint32_t)c * 32u : kNowhere;
    pv[i][0] = __builtin_amdgcn_raw_buffer_load_b128(pi_rs, off, 0, 0);
    pv[i][1] = __builtin_amdgcn_raw_buffer_load_b128(pi_rs, off + 16u, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t x_rs =
      view(X + (int64_t)m0 * ldx, (uint32_t)(((int64_t)(nr - 1) * ldx + d_in) * 2));
  u32x4 v[kR][kJ];
#pragma unroll
  for (int r = 0; r < kR; ++r)
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int cc = tid + j * 256;
      const uint32_t off =
          (r < nr && cc < row_units) ? (uint32_t)(((int64_t)r * ldx + cc * 8) * 2) : kNowhere;
      v[r][j] = __builtin_amdgcn_raw_buffer_load_b128(x_rs, off, 0, 0);
    }
#pragma unroll
  for (int r = 0; r < kR; ++r)
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int cc = tid + j * 256;
      if (r < nr && cc < row_units) *reinterpret_cast<u32x4*>(xs + r * d_in + cc * 8) = v[r][j];
    }
  int idx[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = c0 + i * 256;
      idx[i][j] = pi ? (int)min(pv[i][j >> 2][j & 3], last) : c * 8 + j;
    }
  __syncthreads();
  for (int c = c0, i = 0; c < c1; c += 256, ++i) {
    int id[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      id[j] = i < 2 ? idx[i & 1][j] : (pi ? (int)min((uint32_t)pi[c * 8 + j], last) : c * 8 + j);
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      if (r >= nr) break;
      const uint16_t* xr = xs + r * d_in;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)xr[id[2 * j]] | ((uint32_t)xr[id[2 * j + 1]] << 16);
      *reinterpret_cast<uint4*>(Xp + (int64_t)(m0 + r) * d_in + c * 8) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Permute launch: rows per workgroup kR (a power of two with kR * J <= 16, at most M / CUs) and
// column ranges, so the grid reaches about two workgroups per compute unit while each workgroup
// still writes at least 256 columns (every workgroup stages its whole rows: few rows spread over
// more workgroups measured faster than one workgroup per row), and no thread gathers more than
// two 8-column units. kR = 0 (X not 16-byte aligned, or rows wider than 32768)
// selects the element-wise gather below, and so do fewer than kPermLdsMinRows rows (measured on
// 2560 and 9728 columns: at 16 and 64 rows the GEMM ran up to 1 us faster after the element-wise
// gather, at 1024 rows the staged reorder took 9 us instead of 37 us on 9728 columns).
struct PermPlan {
  int rows = 0, ranges = 1, units = 0;
};

PermPlan permute_plan(int d_in, int M, bool aligned16) {
  PermPlan P;
  const int J = ceil_div(d_in, 2048);
  if (!aligned16 || J > kPermLoads || M < kPermLdsMinRows) return P;
  const int cus = device_cu_count();
  const int want = std::max(1, std::min(kPermLoads / J, M / cus));
  P.rows = want >= 8 ? 8 : (want >= 4 ? 4 : (want >= 2 ? 2 : 1));
  const int wg_rows = ceil_div(M, P.rows);
  P.ranges = std::max(1, std::min(ceil_div(2 * cus, wg_rows), d_in / 256));
  P.ranges = std::max(P.ranges, ceil_div(d_in / 8, 512));  // at most two units per thread
  P.units = ceil_div(d_in / 8, P.ranges);
  P.ranges = ceil_div(d_in / 8, P.units);
  return P;
}

__global__ void __launch_bounds__(256) permute_gather_kernel(const uint16_t* __restrict__ X,
                                                             int64_t ldx,
                                                             const int32_t* __restrict__ pi,
                                                             int d_in, int M,
                                                             uint16_t* __restrict__ Xp) {
  // consecutive workgroups cover consecutive columns of one row (the gather stays inside a row)
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= d_in) return;
  const int src = pi ? (int)min((uint32_t)pi[p], (uint32_t)d_in - 1u) : p;
  for (int m = blockIdx.y; m < M; m += gridDim.y)
    Xp[(int64_t)m * d_in + p] = X[(int64_t)m * ldx + src];
}

// One fp16 pair c scaled by r: each half becomes fp16(c_i * r) with a single rounding of the exact
// product (v_fma_mix takes the fp16 half as its first operand, r in fp32, and rounds the fused
// result once to fp16: the weight the paper's kernel stores, App. A.1).
__device__ inline uint32_t scale_pair_mix(uint32_t c, float r) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(d)
      : "v"(c), "v"(r));
  return d;
}

// Table entry address of the sign-applied codeword halves (the batch-one kernel's table, built
// once per workgroup from the codebook): T[h][s][z] at ((h * 16 + s) * K + z) * 8 holds
// c_z[4h .. 4h+3] with element i negated when bit i of s is set.
template <int L>
struct TKeys {
  static constexpr uint32_t kKeyMask = ((1u << (4 + L)) - 1u) << 3;   // z and a sign nibble
  static constexpr uint32_t kSignMask = 15u << (3 + L);
  static constexpr uint32_t kTHi = 128u << L;
};
__device__ inline uint32_t rotr32(uint32_t v, uint32_t n) { return __builtin_amdgcn_alignbit(v, v, n); }

// LDS layout: the sign-applied codeword table [256 K bytes], 128 spare bytes, flag, then the X tile
// [NT*16][gs*128 + 8] fp16 (also the part-sum exchange once the products are done).
__host__ __device__ inline uint32_t gemm_xs_offset(int L) { return (1u << L) * 256u + 144u; }
// Streamed activations: two buffers of four 16 NT-row slabs (one per column part), each row one
// group's 128 channels (256 bytes, 16-byte chunk c of row R at slot c ^ (R % 16)), after the table.
__host__ __device__ inline uint32_t stream_xs_offset(int L) { return (1u << L) * 256u + 256u; }
__host__ __device__ inline uint32_t stream_lds(int L, int nt) {
  return stream_xs_offset(L) + 2u * 4u * (uint32_t)nt * 16u * 256u;
}

template <int L, int NT, bool kVec, int kGT, bool kStream>
__device__ void gemm_body(const GemmArgs& A, int rp, int split, int mchunk, uint8_t* smem) {
  static_assert(!kStream || (kVec && kGT == 1), "streamed activations need the 1 x 4 shape");
  constexpr uint32_t kK = 1u << L;
  constexpr int kGTiles = GShape<kGT>::kTiles;
  constexpr int kGParts = GShape<kGT>::kParts;
  constexpr int kGMaxUnits = GShape<kGT>::kMaxUnits;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 15;                 // weight row inside the wave's 16 (B), X row (A)
  const int u = lane >> 4;                 // channel quadrant
  const int quarter = wave % (kGTiles * 4);
  const int part = wave / (kGTiles * 4);
  const int rt = rp * kGTiles + quarter / 4;
  const bool tile_ok = rt < A.rt;
  const int wrow_in_tile = (quarter % 4) * 16 + j;
  const int wrow = rt * kTileRows + wrow_in_tile;
  const int g0 = split * A.gs;
  const int ngl = min(A.ng - g0, A.gs);
  const int gpp = (ngl + kGParts - 1) / kGParts;
  const int k0 = part * gpp;
  const int ngp = max(0, min(ngl - k0, gpp));   // groups of this wave
  const int m0 = mchunk * A.mrows_chunk;
  const int mrows = min(A.M - m0, NT * 16);
  const int c0 = g0 * kGroupCols;
  const int cols = ngl * kGroupCols;
  const int xstride = A.gs * kGroupCols + 8;     // fp16 elements per staged activation row

  uint8_t* cb = smem;
  uint32_t* flag = reinterpret_cast<uint32_t*>(smem + kK * 256 + 128);
  _Float16* xs = reinterpret_cast<_Float16*>(smem + (kStream ? stream_xs_offset(L) : gemm_xs_offset(L)));

  // 1. Loads: codebook, pi, activations, then every packed group of the wave.
  const __amdgpu_buffer_rsrc_t cb_rs = view(A.codebook, kK * 16u);
  const u32x4 cw = __builtin_amdgcn_raw_buffer_load_b128(cb_rs, tid * 16, 0, 0);
  const __amdgpu_buffer_rsrc_t x_rs =
      view(A.X + (int64_t)m0 * A.ldx, (uint32_t)((int64_t)mrows * A.ldx * 2));
  // 16-byte chunks per staged row (the shape's largest split) and per thread
  constexpr int kCpr = GShape<kGT>::kMaxGS * (kGroupCols / 8);
  constexpr int kVecLoads = (NT * 16 * kCpr + kGThreads - 1) / kGThreads;
  // columns per thread on the gathered path (more than one when a split exceeds 1024 columns)
  constexpr int kCpt = (GShape<kGT>::kMaxGS * kGroupCols + kGThreads - 1) / kGThreads;
  u32x4 xc[kVecLoads];
  uint16_t xv[kCpt][kDirectRows];
  const int nck = ngl * (kGroupCols / 8);
  // gathered path: pi goes out before the weights (it decides the activation addresses)
  uint32_t pv[kCpt];
  if constexpr (!kVec) {
    const __amdgpu_buffer_rsrc_t pi_rs =
        view(A.pi ? A.pi + c0 : nullptr, A.pi ? (uint32_t)cols * 4u : 0u);
#pragma unroll
    for (int q = 0; q < kCpt; ++q)
      pv[q] = __builtin_amdgcn_raw_buffer_load_b32(pi_rs, (tid + q * kGThreads) * 4, 0, 0);
  }
  // Streamed: iteration it needs group k0 + it of every column part. Its activations are 4 slabs
  // of 16 NT rows x 256 bytes = 16 NT pieces of 1 KiB (4 rows each); wave w loads pieces w, w + 16,
  // ... straight into LDS. Lane l of a piece fills row r0 + l / 16, slot l % 16, i.e. chunk
  // (l % 16) ^ (row % 16) of the row. Groups past a part's range read zeros.
  constexpr int kSlabRows = NT * 16;
  const int giters = (ngl + 3) / 4;
  auto stage = [&](int it) {
    if constexpr (kStream) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int piece = wave + 16 * t;
        const int spart = piece / (kSlabRows / 4);
        const int r0 = (piece % (kSlabRows / 4)) * 4;
        const int row = r0 + (lane >> 4);
        const int chunk = (lane & 15) ^ (row & 15);
        const int gi = spart * giters + it;
        const bool ok = it < giters && gi < ngl;
        const uint32_t off =
            ok ? (uint32_t)(((int64_t)row * A.ldx + c0 + gi * kGroupCols + chunk * 8) * 2)
               : kNowhere;
        uint8_t* dst = reinterpret_cast<uint8_t*>(xs) +
                       ((uint32_t)(((it & 1) * 4 + spart) * kSlabRows + r0) * 256u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rs, (__attribute__((address_space(3))) void*)dst,
                                                 16, off, 0, 0, 0);
      }
    }
  };
  if constexpr (kStream) {
    stage(0);
    stage(1);
  } else if constexpr (kVec) {
#pragma unroll
    for (int i = 0; i < kVecLoads; ++i) {
      const int e = tid + i * kGThreads;
      const int m = e / kCpr, ch = e % kCpr;
      const uint32_t off =
          ch < nck ? (uint32_t)(((int64_t)m * A.ldx + c0 + ch * 8) * 2) : kNowhere;
      xc[i] = __builtin_amdgcn_raw_buffer_load_b128(x_rs, off, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint8_t* blk0 = A.packed + ((int64_t)rt * A.ng + g0) * kBlockBytes;
  const __amdgpu_buffer_rsrc_t w_rs = view(blk0, tile_ok ? (uint32_t)(ngl * kBlockBytes) : 0u);
  u32x2 pp[kGMaxUnits], sd[kGMaxUnits];
  const uint32_t plane = (u < 2 ? kPlaneA : kPlaneB) + wrow_in_tile * 16 + (u & 1) * 8;
#pragma unroll
  for (int k = 0; k < kGMaxUnits; ++k) {
    const bool ok = k < ngp;
    const uint32_t blk = (uint32_t)(k0 + k) * kBlockBytes;
    pp[k] = __builtin_amdgcn_raw_buffer_load_b64(w_rs, ok ? blk + plane : kNowhere, 0, 2);
    sd[k] = __builtin_amdgcn_raw_buffer_load_b64(
        w_rs, ok ? blk + kSidePlane + wrow_in_tile * 8 : kNowhere, 0, 2);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!kVec) {
    // few rows in original order: gather through pi straight from X (rows >= mrows read zeros)
#pragma unroll
    for (int q = 0; q < kCpt; ++q) {
      const int c = tid + q * kGThreads;
      const uint32_t src = A.pi ? min(pv[q], (uint32_t)A.d_in - 1u) : (uint32_t)(c0 + c);
#pragma unroll
      for (int m = 0; m < kDirectRows; ++m)
        xv[q][m] = __builtin_amdgcn_raw_buffer_load_b16(
            x_rs, c < cols ? (uint32_t)(((int64_t)m * A.ldx + src) * 2) : kNowhere, 0, 0);
    }
  }

  // 2. LDS set-up: thread z < K writes the 32 sign-applied halves of codeword z.
  if (tid < (int)kK) {
#pragma unroll
    for (int hs = 0; hs < 32; ++hs) {
      const uint32_t h = (uint32_t)hs >> 4, sg = (uint32_t)hs & 15u;
      const uint32_t c01 = h ? cw[2] : cw[0];
      const uint32_t c23 = h ? cw[3] : cw[1];
      const uint32_t m01 = ((sg & 1u) << 15) | ((sg & 2u) << 30);
      const uint32_t m23 = ((sg & 4u) << 13) | ((sg & 8u) << 28);
      *reinterpret_cast<u32x2*>(cb + ((uint32_t)hs * kK + (uint32_t)tid) * 8u) =
          u32x2{c01 ^ m01, c23 ^ m23};
    }
  }
  if constexpr (kStream) {
    // nothing: the activations go straight to LDS
  } else if constexpr (kVec) {
#pragma unroll
    for (int i = 0; i < kVecLoads; ++i) {
      const int e = tid + i * kGThreads;
      const int m = e / kCpr, ch = e % kCpr;
      if (ch < nck && m < NT * 16) *reinterpret_cast<u32x4*>(xs + m * xstride + ch * 8) = xc[i];
    }
  } else {
#pragma unroll
    for (int q = 0; q < kCpt; ++q) {
      const int c = tid + q * kGThreads;
      if (c < cols) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
          xs[m * xstride + c] =
              m < kDirectRows ? __builtin_bit_cast(_Float16, xv[q][m]) : (_Float16)0.0f;
      }
    }
  }
  // (streamed: the first iteration's barrier covers the table)
  if constexpr (!kStream) __syncthreads();

  // 3. Decode once, multiply NT times.
  float4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  const bool row_ok = tile_ok && wrow < A.d_out;  // padded rows decode to zero weights anyway
  if constexpr (kStream) {
    // Iteration it: every wave waits for its own activation loads of the iteration (the counts are
    // the loads issued after them: iteration 1's loads and the 2 kGMaxUnits packed-word loads
    // before iteration 0, the packed-word loads before iteration 1, none later) and meets the
    // others at the barrier, after which the other buffer is free for iteration it + 1.
#pragma unroll
    for (int it = 0; it < kGMaxUnits; ++it) {
      if (it < giters) {
        if (it == 0)
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NT + 2 * kGMaxUnits)
                       : "memory");
        else if (it == 1)
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * kGMaxUnits)
                       : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (it >= 1 && it + 1 < giters) stage(it + 1);
        if (it < ngp) {
          const uint8_t* abase = reinterpret_cast<const uint8_t*>(xs) +
                                 (uint32_t)(((it & 1) * 4 + part) * kSlabRows) * 256u;
          const float mu = h2f(sd[it][1]);
          const float dl = h2f(sd[it][1] >> 16);
          using TK = TKeys<L>;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const uint32_t P = (kk < 2) ? pp[it][0] : pp[it][1];
            const uint32_t pair = 2u * (uint32_t)u + (uint32_t)(kk >> 1);
            uint32_t klo, khi, q;
            if ((kk & 1) == 0) {
              klo = P & TK::kKeyMask;
              khi = (rotr32(sd[it][0], (4u * pair + 29u - (uint32_t)L) & 31u) & TK::kSignMask) |
                    (klo & ~TK::kSignMask);
              q = (P >> (7 + L)) & ((1u << (10 - L)) - 1u);
            } else {
              const uint32_t R = rotr32(P, 14);
              klo = R & TK::kKeyMask;
              khi = (rotr32(P, 28 - L) & TK::kSignMask) | (klo & ~TK::kSignMask);
              q = (R >> (7 + L)) & ((1u << (10 - L)) - 1u);
            }
            const float r = fmaf((float)q, dl, mu);
            const u32x2 lo = *reinterpret_cast<const u32x2*>(cb + klo);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(cb + TK::kTHi + khi);
            uint32_t w[4];
            w[0] = scale_pair_mix(lo[0], r);
            w[1] = scale_pair_mix(lo[1], r);
            w[2] = scale_pair_mix(hi[0], r);
            w[3] = scale_pair_mix(hi[1], r);
            if (!row_ok) w[0] = w[1] = w[2] = w[3] = 0u;
            const half8_t b = __builtin_bit_cast(half8_t, make_uint4(w[0], w[1], w[2], w[3]));
            // activation row t * 16 + j, chunk 4 u + kk of the group, at slot chunk ^ j
            const uint32_t aoff = (uint32_t)j * 256u + (uint32_t)(((4 * u + kk) ^ j) * 16);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const half8_t a =
                  *reinterpret_cast<const half8_t*>(abase + (uint32_t)t * 4096u + aoff);
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
            }
          }
        }
      }
    }
  } else {
  // the SIMD's issue slots go to the oldest wave first; a wave's priority is its remaining groups
  // (3 down to 0), so the four waves of a SIMD advance together instead of one after another
  __builtin_amdgcn_s_setprio(3);
#pragma unroll
  for (int k = 0; k < kGMaxUnits; ++k) {
    if (k < ngp) {
      const int left = ngp - 1 - k;
      if (left == 2) __builtin_amdgcn_s_setprio(2);
      else if (left == 1) __builtin_amdgcn_s_setprio(1);
      else if (left == 0) __builtin_amdgcn_s_setprio(0);
      const int slot = k0 + k;
      const float mu = h2f(sd[k][1]);
      const float dl = h2f(sd[k][1] >> 16);
      using TK = TKeys<L>;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // subvector 4u + kk of the group: payload dword 2u + kk/2, half a (kk even) or b (kk odd);
        // its table keys come straight from the packed word (see the batch-one kernel): the low
        // sign nibble sits next to z, the high one is rotated into place from X (a) or P (b)
        const uint32_t P = (kk < 2) ? pp[k][0] : pp[k][1];
        const uint32_t pair = 2u * (uint32_t)u + (uint32_t)(kk >> 1);
        uint32_t klo, khi, q;
        if ((kk & 1) == 0) {
          klo = P & TK::kKeyMask;
          khi = (rotr32(sd[k][0], (4u * pair + 29u - (uint32_t)L) & 31u) & TK::kSignMask) |
                (klo & ~TK::kSignMask);
          q = (P >> (7 + L)) & ((1u << (10 - L)) - 1u);
        } else {
          const uint32_t R = rotr32(P, 14);
          klo = R & TK::kKeyMask;
          khi = (rotr32(P, 28 - L) & TK::kSignMask) | (klo & ~TK::kSignMask);
          q = (R >> (7 + L)) & ((1u << (10 - L)) - 1u);
        }
        const float r = fmaf((float)q, dl, mu);
        const u32x2 lo = *reinterpret_cast<const u32x2*>(cb + klo);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(cb + TK::kTHi + khi);
        uint32_t w[4];
        w[0] = scale_pair_mix(lo[0], r);
        w[1] = scale_pair_mix(lo[1], r);
        w[2] = scale_pair_mix(hi[0], r);
        w[3] = scale_pair_mix(hi[1], r);
        if (!row_ok) w[0] = w[1] = w[2] = w[3] = 0u;
        const half8_t b = __builtin_bit_cast(half8_t, make_uint4(w[0], w[1], w[2], w[3]));
        const int xcol = slot * kGroupCols + (4 * u + kk) * 8;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const half8_t a = *reinterpret_cast<const half8_t*>(xs + (t * 16 + j) * xstride + xcol);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
        }
      }
    }
  }

  __builtin_amdgcn_s_setprio(0);
  }
  // 4. The other column parts hand their sums to the first through LDS (the X tile is done);
  // part order is kept.
  __syncthreads();
  float4_t* red = reinterpret_cast<float4_t*>(xs);
  if (part > 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      red[(((part - 1) * kGTiles * 4 + quarter) * NT + t) * 64 + lane] = acc[t];
  }
  __syncthreads();
  if (part == 0) {
#pragma unroll
    for (int p = 1; p < kGParts; ++p)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] += red[(((p - 1) * kGTiles * 4 + quarter) * NT + t) * 64 + lane];
  }

  // 5. Output. D layout: lane holds weight row j and activation rows 4u .. 4u+3 of each tile.
  const int64_t rows_pad = (int64_t)A.rt * kTileRows;
  const bool out_ok = part == 0 && row_ok;
  if (A.S == 1) {
    if (out_ok) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = t * 16 + 4 * u + r;
          if (m < mrows) A.Y[(int64_t)(m0 + m) * A.ldy + wrow] = f2h(acc[t][r]);
        }
    }
    return;
  }
  float* pbuf = A.partial + (int64_t)mchunk * A.S * A.mrows_chunk * rows_pad;
  if (out_ok) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = t * 16 + 4 * u + r;
        if (m < mrows)
          store_coherent(pbuf + ((int64_t)split * A.mrows_chunk + m) * rows_pad + wrow, acc[t][r]);
      }
  }
  wait_stores();
  __syncthreads();
  uint32_t* counter = A.counters + (int64_t)mchunk * A.rpairs + rp;
  if (tid == 0) *flag = (counter_add(counter) == (uint32_t)(A.S - 1)) ? 1u : 0u;
  __syncthreads();
  if (*flag == 0u) return;
  // last workgroup: reduce the tiles for all rows of the chunk. Thread t owns elements
  // t + 1024 i (activation row e / R, row e % R of the tile block, R = 64 kGTiles); four splits in
  // flight.
  constexpr int kRows = kGTiles * kTileRows;
  constexpr int kPer = NT * 16 * kRows / kGThreads;
  const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(
      pbuf, (uint32_t)((int64_t)A.S * A.mrows_chunk * rows_pad * (int64_t)sizeof(float)));
  const int prow = rp * kRows + (tid % kRows);
  float sum[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) sum[i] = 0.0f;
  for (int sp0 = 0; sp0 < A.S; sp0 += 4) {
    float v[4][kPer];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int m = tid / kRows + (kGThreads / kRows) * i;
        const int sp = min(sp0 + q, A.S - 1);
        v[q][i] = load_coherent_at(
            rs, (uint32_t)((((int64_t)sp * A.mrows_chunk + m) * rows_pad + prow) * sizeof(float)));
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (sp0 + q < A.S) sum[i] += v[q][i];
  }
  if (prow < A.d_out) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = tid / kRows + (kGThreads / kRows) * i;
      if (m < mrows) A.Y[(int64_t)(m0 + m) * A.ldy + prow] = f2h(sum[i]);
    }
  }
  if (tid == 0) counter_reset(counter);
}

// One kernel per split (log2 K = L compiled in): a wave runs through a third of the code a switch
// over the split would give it (fewer instruction-cache misses while the workgroups start).
template <int NT, bool kVec, int kGT, bool kStream, int L>
__global__ void __launch_bounds__(kGThreads) gemm_kernel(GemmArgs A) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int per_chunk = A.rpairs * A.S;
  const int mchunk = blockIdx.x / per_chunk;
  const int local = blockIdx.x - mchunk * per_chunk;
  const int rp = local / A.S;
  const int split = local - rp * A.S;
  gemm_body<L, NT, kVec, kGT, kStream>(A, rp, split, mchunk, smem);
}

typedef void (*GemmFn)(GemmArgs);

template <int NT, bool kVec, int kGT, bool kStream = false>
GemmFn gemm_fn(int L) {
  switch (L) {
    case 4: return gemm_kernel<NT, kVec, kGT, kStream, 4>;
    case 5: return gemm_kernel<NT, kVec, kGT, kStream, 5>;
    case 6: return gemm_kernel<NT, kVec, kGT, kStream, 6>;
    case 7: return gemm_kernel<NT, kVec, kGT, kStream, 7>;
    default: return gemm_kernel<NT, kVec, kGT, kStream, 8>;
  }
}

// ------------------------------------------------------------------------------------------------
// Prefill-sized batches (SAGE paper §3.5 / Fig. 6b: decode each weight once per output tile and
// reuse it across many activation rows). A wavefront owns one 64-row weight tile and kQ 32-row
// blocks of activations, as 2 x kQ tiles of v_mfma_f32_32x32x16_f16 (16 fp32 accumulators per
// lane and tile). In the B operand lane l supplies weight row l % 32 of a 32-row subtile and
// channels 8 (l / 32) .. +7 of the 16-channel step, i.e. one subvector: step s of a group uses
// subvectors 2s (lanes 0-31) and 2s + 1 (lanes 32-63). A workgroup (4 waves, 4 weight tiles)
// shares a double-buffered activation slab [32 kQ rows][128 channels] in LDS, filled by
// buffer-to-LDS loads one group ahead, so every weight is decoded once per 32 kQ activation rows.
constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
// kQ 32-row blocks of activations per workgroup (4 or 8): rows and slab bytes. Slab rows are
// 256 bytes unpadded; 16-byte chunk c of row R sits at chunk slot c ^ (R % 16), so the 16 rows a
// quarter-wave reads in one operand load hit 16 different slots (all 64 banks).
template <int kQ> struct PfShape {
  static constexpr int kRows = 32 * kQ;
  static constexpr int kSlab = kRows * kGroupCols * 2;
  static constexpr int kLoads = kRows * kGroupCols * 2 / 1024 / kPfWaves;  // 1 KiB loads per wave
};

typedef float float16_t __attribute__((ext_vector_type(16)));

struct PrefillArgs {
  const uint8_t* packed;
  const uint16_t* codebook;
  const uint16_t* Xp;   // activations in permuted order, [M][ldx], 16-byte aligned rows
  uint16_t* Y;
  float* partial;       // split-K partial sums, see the split store below (S > 1)
  int64_t ldy;
  int64_t ldx;          // elements between activation rows (a multiple of 8)
  int32_t d_out, d_in, M, L;
  int32_t rt, ng;
  int32_t S, gs;        // column splits (blockIdx.z) and groups per split
};

__host__ __device__ inline uint32_t prefill_slab_offset(int L) {
  return (1u << L) * 256u + 256u;  // after the sign-applied codeword table and 256 spare bytes
}

// One lane's packed words of one row in one group: payload dwords P0..P7, then X and G.
struct RowWords {
  u32x4 a, b;
  u32x2 side;
};

// First half of a subvector decode: the two sign-applied codeword halves and the radius. The
// table reads are only issued here; decode_finish consumes them a pipeline step later.
struct Fetched {
  u32x2 lo, hi;
  float r;
};

// Lanes of the first half-wave (rot = 0, hb = 0) take subvector a = 2s of pair s, the others
// (rot = 14, hb = 1) subvector b = 2s + 1, whose index, low sign nibble and radius code the
// rotation by 14 brings to a's positions. The table keys come straight from the packed word as in
// the batch-one kernel: the low sign nibble sits next to z, the high one is rotated into place
// from X (a) or from P (b).
template <int L>
__device__ __forceinline__ Fetched decode_fetch(const RowWords& w, int s, uint32_t rot, uint32_t hb,
                                                const uint8_t* cb) {
  using TK = TKeys<L>;
  constexpr uint32_t kV = (1u << (10 - L)) - 1u;
  const uint32_t P = s < 4 ? w.a[s & 3] : w.b[s & 3];
  const uint32_t X = w.side[0], G = w.side[1];
  const uint32_t Pr = rotr32(P, rot);
  const uint32_t klo = Pr & TK::kKeyMask;
  const uint32_t src = hb ? P : X;
  const uint32_t sh = hb ? (uint32_t)(28 - L) : ((4u * (uint32_t)s + 29u - (uint32_t)L) & 31u);
  const uint32_t khi = (rotr32(src, sh) & TK::kSignMask) | (klo & ~TK::kSignMask);
  const uint32_t q = (Pr >> (7 + L)) & kV;
  Fetched o;
  o.r = fmaf((float)q, h2f(G >> 16), h2f(G));
  o.lo = *reinterpret_cast<const u32x2*>(cb + klo);
  o.hi = *reinterpret_cast<const u32x2*>(cb + TK::kTHi + khi);
  return o;
}

__device__ __forceinline__ half8_t decode_finish(const Fetched& d) {
  return __builtin_bit_cast(
      half8_t, make_uint4(scale_pair_mix(d.lo[0], d.r), scale_pair_mix(d.lo[1], d.r),
                          scale_pair_mix(d.hi[0], d.r), scale_pair_mix(d.hi[1], d.r)));
}

template <int L, int kQ>
__device__ void prefill_body(const PrefillArgs& A, uint8_t* smem) {
  constexpr uint32_t kK = 1u << L;
  constexpr int kPfRows = PfShape<kQ>::kRows;
  constexpr int kPfSlab = PfShape<kQ>::kSlab;
  constexpr int kPfLoads = PfShape<kQ>::kLoads;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;                    // k half of the 16-channel step
  const int r0 = lane & 31;                   // rows r0 and 32 + r0 of the tile
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). Without splits,
  // renumber them so that each XCD takes a contiguous run of (tile quad, row block) in
  // tile-quad-fastest order: the workgroups that read one activation slab then share an L2
  // (measured 1-6 % faster). With splits the plain order is kept: on 2560x9728 at M = 128
  // (19 splits) the renumbered grid ran 33 us against 24 us.
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;  // tile quad, row block, split
  if (gridDim.z == 1) {
    const int n = gridDim.x * gridDim.y * gridDim.z;
    const int lid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int xcd = lid & 7, k = lid >> 3, base = n >> 3, rem = n & 7;
    const int id = xcd < rem ? xcd * (base + 1) + k : rem * (base + 1) + (xcd - rem) * base + k;
    bx = id % gridDim.x;
    by = (id / gridDim.x) % gridDim.y;
    bz = id / (gridDim.x * gridDim.y);
  }
  const int rt = bx * kPfWaves + wave;
  const bool tile_ok = rt < A.rt;
  const int m0 = by * kPfRows;
  const int mrows = min(A.M - m0, kPfRows);
  const int g0 = bz * A.gs;                  // first column group of this split
  const int ng = min(A.ng - g0, A.gs);       // groups of this split
  uint8_t* cb = smem;
  uint8_t* slab0 = smem + prefill_slab_offset(L);

  const __amdgpu_buffer_rsrc_t cb_rs = view(A.codebook, kK * 16u);
  // the views start at the split's first group; words and activations of groups past the
  // split's last are never addressed (offsets point outside both views)
  const __amdgpu_buffer_rsrc_t w_rs =
      view(A.packed + ((int64_t)rt * A.ng + g0) * kBlockBytes,
           tile_ok ? (uint32_t)(ng * kBlockBytes) : 0u);
  const __amdgpu_buffer_rsrc_t x_rs =
      view(A.Xp + m0 * A.ldx + g0 * kGroupCols,
           (uint32_t)(((int64_t)(mrows - 1) * A.ldx + A.d_in - g0 * kGroupCols) * 2));
  // per-lane byte offsets, fixed for the whole loop; the group adds a uniform amount
  const uint32_t wa0 = kPlaneA + r0 * 16, wb0 = kPlaneB + r0 * 16, ws0 = kSidePlane + r0 * 8;
  // Buffer-to-LDS loads: lane l of a 1 KiB load j writes slot l % 16 of slab row 4 j + l / 16,
  // so it fetches chunk (l % 16) ^ ((4 j + l / 16) % 16) of that row; the chunk depends on j % 4.
  const uint32_t row_bytes = (uint32_t)A.ldx * 2u;
  uint32_t xl[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    xl[t] = (uint32_t)(lane >> 4) * row_bytes +
            (((uint32_t)(lane & 15) ^ ((4u * t + (uint32_t)(lane >> 4)) & 15u)) << 4);
  // operand loads: row q 32 + r0, chunk 2 s + h at slot (2 s) ^ (h ^ r0 % 16)
  const uint32_t a_row = (uint32_t)r0 * 256u;
  const uint32_t a_hm = ((uint32_t)h ^ (uint32_t)(r0 & 15)) << 4;

  const u32x4 cw = __builtin_amdgcn_raw_buffer_load_b128(cb_rs, tid * 16, 0, 0);
  // Packed words run two groups ahead through a three-deep register ring (group g computes from
  // slot g % 3; no slot is copied, so no wait covers a later group). Activations run one group
  // ahead, loaded straight into the other slab buffer.
  RowWords wr[3][2];
#define SAGE_PF_WORDS(slot, grp)                                                              \
  {                                                                                          \
    const uint32_t wg_ = (grp) < ng ? (uint32_t)(grp) * kBlockBytes : kNowhere;              \
    _Pragma("unroll") for (int t = 0; t < 2; ++t) {                                          \
      wr[slot][t].a = __builtin_amdgcn_raw_buffer_load_b128(w_rs, wg_ + wa0 + t * 512, 0, 2); \
      wr[slot][t].b = __builtin_amdgcn_raw_buffer_load_b128(w_rs, wg_ + wb0 + t * 512, 0, 2); \
      wr[slot][t].side = __builtin_amdgcn_raw_buffer_load_b64(w_rs, wg_ + ws0 + t * 256, 0, 2); \
    }                                                                                        \
  }
#define SAGE_PF_X(grp)                                                                       \
  {                                                                                          \
    const uint32_t xg_ = (grp) < ng ? (uint32_t)(grp) * (kGroupCols * 2) : kNowhere;         \
    uint8_t* dst_ = slab0 + ((grp) & 1) * kPfSlab + wave * (kPfLoads * 1024);                \
    _Pragma("unroll") for (int i = 0; i < kPfLoads; ++i) {                                   \
      const uint32_t row_ = (uint32_t)(4 * (wave * kPfLoads + i));                           \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                              \
          x_rs, (__attribute__((address_space(3))) void*)(dst_ + i * 1024), 16,              \
          xg_ + row_ * row_bytes + xl[i & 3], 0, 0, 0);                                      \
    }                                                                                        \
  }
  SAGE_PF_X(0)
  SAGE_PF_WORDS(0, 0)
  SAGE_PF_WORDS(1, 1)
  // the sign-applied codeword table: thread z < K writes the 32 halves of codeword z
  if (tid < (int)kK) {
#pragma unroll
    for (int hs = 0; hs < 32; ++hs) {
      const uint32_t hh = (uint32_t)hs >> 4, sg = (uint32_t)hs & 15u;
      const uint32_t c01 = hh ? cw[2] : cw[0];
      const uint32_t c23 = hh ? cw[3] : cw[1];
      const uint32_t m01 = ((sg & 1u) << 15) | ((sg & 2u) << 30);
      const uint32_t m23 = ((sg & 4u) << 13) | ((sg & 8u) << 28);
      *reinterpret_cast<u32x2*>(cb + ((uint32_t)hs * kK + (uint32_t)tid) * 8u) =
          u32x2{c01 ^ m01, c23 ^ m23};
    }
  }
  // the first slab has landed once only the two word groups are outstanding
  asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  __syncthreads();

  float16_t acc[2][kQ];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][q][v] = 0.0f;
  const uint32_t rot = h ? 14u : 0u;
  const uint32_t hb = (uint32_t)h;

  // One group, software-pipelined over its 8 steps: while the MFMAs of step s run, the operand
  // loads of step s + 1 and the table reads of step s + 2 are in flight and step s + 1's
  // decode finishes on the vector ALU. Activations of g + 1 go to the other slab buffer and the
  // words of g + 2 into ring slot (k + 2) % 3 at the start; at the end every wave waits for its
  // slab loads (all but the 6 word loads just issued) and meets the others at the barrier.
#define SAGE_PF_GROUP(k)                                                                      \
  {                                                                                           \
    const int gg = g + (k);                                                                   \
    SAGE_PF_X(gg + 1)                                                                         \
    SAGE_PF_WORDS(((k) + 2) % 3, gg + 2)                                                      \
    const uint8_t* abuf = slab0 + (gg & 1) * kPfSlab + a_row;                                 \
    Fetched fd[2][2];                                                                         \
    half8_t bv[2][2];                                                                         \
    half8_t av[2][kQ];                                                                        \
    _Pragma("unroll") for (int t = 0; t < 2; ++t) {                                           \
      fd[0][t] = decode_fetch<L>(wr[k][t], 0, rot, hb, cb);                                \
      fd[1][t] = decode_fetch<L>(wr[k][t], 1, rot, hb, cb);                                \
    }                                                                                         \
    _Pragma("unroll") for (int q = 0; q < kQ; ++q)                                            \
      av[0][q] = *reinterpret_cast<const half8_t*>(abuf + q * 8192 + (a_hm ^ 0u));            \
    _Pragma("unroll") for (int t = 0; t < 2; ++t) bv[0][t] = decode_finish(fd[0][t]);         \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    _Pragma("unroll") for (int s = 0; s < 8; ++s) {                                           \
      if (s + 1 < 8) {                                                                        \
        _Pragma("unroll") for (int q = 0; q < kQ; ++q)                                        \
          av[(s + 1) & 1][q] = *reinterpret_cast<const half8_t*>(                             \
              abuf + q * 8192 + (a_hm ^ (uint32_t)(32 * (s + 1))));                           \
      }                                                                                       \
      if (s + 2 < 8) {                                                                        \
        _Pragma("unroll") for (int t = 0; t < 2; ++t)                                         \
          fd[s & 1][t] = decode_fetch<L>(wr[k][t], s + 2, rot, hb, cb);                    \
      }                                                                                       \
      _Pragma("unroll") for (int q = 0; q < kQ; ++q)                                          \
        _Pragma("unroll") for (int t = 0; t < 2; ++t)                                         \
          acc[t][q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[s & 1][q], bv[s & 1][t],      \
                                                             acc[t][q], 0, 0, 0);             \
      if (s + 1 < 8) {                                                                        \
        _Pragma("unroll") for (int t = 0; t < 2; ++t)                                         \
          bv[(s + 1) & 1][t] = decode_finish(fd[(s + 1) & 1][t]);                             \
      }                                                                                       \
      __builtin_amdgcn_sched_barrier(0);                                                      \
    }                                                                                         \
    asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");                             \
  }
  // the group count is rounded up to a multiple of three: groups past the last read zeros
  // (out-of-range loads) and add nothing, which keeps the loop free of exits that would
  // multiply the register ring
  for (int g = 0; g < ng; g += 3) {
    SAGE_PF_GROUP(0)
    SAGE_PF_GROUP(1)
    SAGE_PF_GROUP(2)
  }
#undef SAGE_PF_GROUP
#undef SAGE_PF_X
#undef SAGE_PF_WORDS

  // D layout: lane holds weight row l % 32 of each subtile and activation rows
  // 8 (v / 4) + 4 (l / 32) + v % 4 of each 32-row block.
  if (!tile_ok) return;
  if (A.S > 1) {
    // one split's fp32 sums, stored as the accumulators lie: wave tile (split, block, rt) owns
    // 2 kQ 16 x 64 floats, element (t, q, v) of lane l at ((t kQ + q) 16 + v) 64 + l; a second
    // kernel adds the splits in order
    constexpr int kTileFloats = 2 * kQ * 16 * 64;
    float* base = A.partial +
                  (((int64_t)bz * gridDim.y + by) * A.rt + rt) * kTileFloats;
    const __amdgpu_buffer_rsrc_t p_rs = view(base, kTileFloats * 4u);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < kQ; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // copy the element out first: a bit cast taken straight from a vector element reads
          // the vector's first element (clang, ext_vector_type)
          const float f = acc[t][q][v];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, f), p_rs,
                                                (uint32_t)lane * 4u,
                                                ((t * kQ + q) * 16 + v) * 256, 0);
        }
    return;
  }
  const __amdgpu_buffer_rsrc_t y_rs =
      view(A.Y + (int64_t)m0 * A.ldy, (uint32_t)((int64_t)mrows * A.ldy * 2));
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = rt * kTileRows + t * 32 + r0;
    if (n >= A.d_out) continue;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = q * 32 + 8 * (v / 4) + 4 * h + (v % 4);
        // rows past mrows fall outside y_rs and are dropped
        __builtin_amdgcn_raw_buffer_store_b16(f2h(acc[t][q][v]), y_rs,
                                              (uint32_t)((m * (int)A.ldy + n) * 2), 0, 0);
      }
  }
}

// One kernel per codebook size: with a switch over L inside one kernel the compiler hoists the
// first activation loads above the switch and spills them. Both variants hold more than 256
// registers per lane (one wave per SIMD); the software pipeline inside the wave hides latency.
template <int L, int kQ>
__global__ void __launch_bounds__(kPfThreads) prefill_kernel(PrefillArgs A) {
  extern __shared__ __align__(16) uint8_t smem[];
  prefill_body<L, kQ>(A, smem);
}

typedef void (*PrefillFn)(PrefillArgs);

// kq = 8 exists for L <= 6 only: larger codebooks leave no room for two 256-row slabs
PrefillFn prefill_fn(int L, int kq) {
  if (kq == 8) {
    switch (L) {
      case 4: return prefill_kernel<4, 8>;
      case 5: return prefill_kernel<5, 8>;
      default: return prefill_kernel<6, 8>;
    }
  }
  if (kq == 2) {
    switch (L) {
      case 4: return prefill_kernel<4, 2>;
      case 5: return prefill_kernel<5, 2>;
      case 6: return prefill_kernel<6, 2>;
      case 7: return prefill_kernel<7, 2>;
      default: return prefill_kernel<8, 2>;
    }
  }
  switch (L) {
    case 4: return prefill_kernel<4, 4>;
    case 5: return prefill_kernel<5, 4>;
    case 6: return prefill_kernel<6, 4>;
    case 7: return prefill_kernel<7, 4>;
    default: return prefill_kernel<8, 4>;
  }
}

// Split sums of the prefill kernel, four outputs per thread: thread j reads elements 4j .. 4j + 3
// of every split's plane (laid out as the kernel's accumulators, 64 x rows floats per wave tile
// and block; the four are lanes l .. l + 3 of one accumulator, i.e. four consecutive outputs of
// one row) and writes Y[m][n] = fp16(partial[0] + ... + partial[S-1]), added in split order.
__global__ void __launch_bounds__(256) prefill_reduce_kernel(const float* __restrict__ partial,
                                                             int S, int64_t plane, int rows,
                                                             int rt, int M, int d_out,
                                                             uint16_t* __restrict__ Y, int64_t ldy) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= plane) return;
  const int tile = 64 * rows;                 // floats of one wave tile and activation block
  const int64_t c = i / tile;
  const int e = (int)(i - c * tile);
  const int lane = e & 63;
  const int v = (e >> 6) & 15;
  const int tq = e >> 10;                     // t kQ + q
  const int kq = rows / 32;
  const int t = tq / kq, q = tq - t * kq;
  const int r = (int)(c % rt);
  const int b = (int)(c / rt);
  const int n = r * kTileRows + t * 32 + (lane & 31);
  const int m = b * rows + q * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
  if (m >= M || n >= d_out) return;
  const float4* p4 = reinterpret_cast<const float4*>(partial + i);
  const int64_t step = plane / 4;
  float4 sum = p4[0];
  int sp = 1;
  for (; sp + 8 <= S; sp += 8) {
    // eight splits' loads in flight, added in split order
    float4 a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = p4[(sp + k) * step];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sum.x += a[k].x;
      sum.y += a[k].y;
      sum.z += a[k].z;
      sum.w += a[k].w;
    }
  }
  for (; sp < S; ++sp) {
    const float4 a0 = p4[sp * step];
    sum.x += a0.x; sum.y += a0.y; sum.z += a0.z; sum.w += a0.w;
  }
  uint16_t* y = Y + (int64_t)m * ldy + n;
  y[0] = f2h(sum.x);
  if (n + 1 < d_out) y[1] = f2h(sum.y);
  if (n + 2 < d_out) y[2] = f2h(sum.z);
  if (n + 3 < d_out) y[3] = f2h(sum.w);
}

// Launch shape of the prefill kernel: kq 32-row activation blocks per workgroup, S column splits
// of gs groups. kq = 0 means the small-batch kernel runs instead.
struct PfPlan {
  int kq = 0;
  int S = 1;
  int gs = 0;
};

size_t prefill_lds(int L, int kq) {
  return prefill_slab_offset(L) +
         2 * (size_t)(kq == 8 ? PfShape<8>::kSlab : (kq == 4 ? PfShape<4>::kSlab : PfShape<2>::kSlab));
}

// From kPrefillMinRows rows on (measured on 9728x2560 and 2560x9728, M = 128 ... 1024, every
// kq and split count):
//  - kq = 8 (each decoded subvector feeds 8 MFMAs, one workgroup per compute unit) when more than
//    128 rows come, two 256-row slabs fit beside the codebook and its grid covers at least half
//    the compute units; it never gained from splits.
//  - else kq = 4, with the column groups split until the grid reaches one workgroup per compute
//    unit (at least two groups per split). Wider grids lost: the splits' fp32 sums cost 8 bytes
//    per output and split.
//  - Below 256 rows the small-batch kernel wins unless the split is deep (grid of 128-row blocks
//    at most an eighth of the compute units).
//  - From 65 to 127 rows the same holds for kq = 2 (64-row blocks): 2560x9728 at M = 96 ran
//    32 us split 12 ways against 39 us in the small-batch kernel; at M = 32 and 64, and on
//    9728x2560, the small-batch kernel was faster.
PfPlan prefill_plan(int L, int d_out, int d_in, int M) {
  PfPlan P;
  const int64_t cus = device_cu_count();
  const int ng = d_in / kGroupCols;
  const int64_t wx = ceil_div(ceil_div(d_out, kTileRows), kPfWaves);
  if (M < kPrefillMinRows) {
    const int64_t wgs2 = wx * ceil_div(M, PfShape<2>::kRows);
    if (M <= PfShape<2>::kRows || 8 * wgs2 > cus) return P;
    int64_t S = cus / wgs2;
    if (S > ng / 2) S = ng / 2;
    if (S < 1) S = 1;
    P.kq = 2;
    P.gs = ceil_div(ng, (int)S);
    P.S = ceil_div(ng, P.gs);
    return P;
  }
  const int64_t wgs8 = wx * ceil_div(M, PfShape<8>::kRows);
  if (M > PfShape<4>::kRows && prefill_lds(L, 8) <= 160 * 1024 && 2 * wgs8 >= cus) {
    P.kq = 8;
    P.gs = ng;
    return P;
  }
  const int64_t wgs = wx * ceil_div(M, PfShape<4>::kRows);
  if (M < 256 && 8 * wgs > cus) return P;
  P.kq = 4;
  int64_t S = cus / wgs;
  if (S > ng / 2) S = ng / 2;
  if (S < 1) S = 1;
  P.gs = ceil_div(ng, (int)S);
  P.S = ceil_div(ng, P.gs);
  return P;
}

// floats of one split's partial sums: every wave tile of every activation block
int64_t prefill_plane(const PfPlan& P, int d_out, int M) {
  const int rows = 32 * P.kq;
  return (int64_t)ceil_div(M, rows) * rows * ceil_div(d_out, kTileRows) * kTileRows;
}

size_t prefill_partial_bytes(const PfPlan& P, int d_out, int M) {
  if (P.S <= 1) return 0;
  return ((size_t)P.S * prefill_plane(P, d_out, M) * 4 + 255) / 256 * 256;
}

int tiles_for(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

constexpr size_t kLdsLimit = 160 * 1024;

// LDS of the small-batch kernel: codebook, then the X tile or the part-sum exchange (T tiles,
// 4 / T parts), whichever is larger.
size_t lds_for(int L, int nt, int gs, int T) {
  const size_t xtile = (size_t)nt * 16 * ((size_t)gs * kGroupCols + 8) * 2;
  const size_t red = (size_t)(4 / T - 1) * T * 4 * nt * 64 * 16;
  return gemm_xs_offset(L) + (xtile > red ? xtile : red);
}

// Workgroup shape and groups per split (a workgroup fills a compute unit, so a launch should fit
// in one workgroup per compute unit):
//   1. 17 rows or more: 1 x 4 with streamed activations (below);
//   2. 8 to 16 activation rows (read as whole vectors, not gathered): 1 x 4 with every column
//      group in one split when that fits (no split-K at all; with fewer rows the per-thread
//      gather of twenty groups costs more than the split-K pass it saves);
//   3. else 2 x 2 with the fewest groups per split that fit, within the LDS budget.
void plan(GemmArgs& A, int M) {
  A.rt = ceil_div(A.d_out, kTileRows);
  A.ng = A.d_in / kGroupCols;
  A.mrows_chunk = 16 * tiles_for(M);
  A.mchunks = ceil_div(M, A.mrows_chunk);
  const int nt = tiles_for(M);
  const int64_t cus = device_cu_count();
  A.stream = 0;
  // 17 or more rows (X always in stored order from 8 rows on): one 64-row tile x 4 column parts
  // with the activations streamed through LDS a group at a time, so a workgroup can take every
  // column group (at most 20) of its tile; splits only where the row tiles alone leave most compute
  // units idle, at least one group per part
  if (nt >= 2 && M >= kPermuteMinRows && stream_lds(A.L, nt) <= kLdsLimit) {
    A.stream = 1;
    A.tiles = 1;
    A.rpairs = A.rt;
    const int64_t tiles = (int64_t)A.mchunks * A.rt;
    int64_t S = std::max<int64_t>(1, cus / tiles);
    S = std::max<int64_t>(S, ceil_div(A.ng, gshape_max_gs(1)));
    S = std::min<int64_t>(S, std::max(1, A.ng / 4));
    A.gs = ceil_div(A.ng, (int)S);
    A.S = ceil_div(A.ng, A.gs);
    return;
  }
  if (nt == 1 && M >= kPermuteMinRows && A.ng <= gshape_max_gs(1) && (int64_t)A.mchunks * A.rt <= cus &&
      lds_for(A.L, nt, A.ng, 1) <= kLdsLimit) {
    A.tiles = 1;
    A.rpairs = A.rt;
    A.S = 1;
    A.gs = A.ng;
    return;
  }
  A.tiles = 2;
  A.rpairs = ceil_div(A.rt, 2);
  int best = 1;
  for (int gs = 1; gs <= gshape_max_gs(2) && gs <= A.ng; ++gs) {
    if (lds_for(A.L, nt, gs, 2) > kLdsLimit) break;
    best = gs;
    if ((int64_t)A.mchunks * A.rpairs * ceil_div(A.ng, gs) <= cus) break;
  }
  A.S = ceil_div(A.ng, best);
  A.gs = ceil_div(A.ng, A.S);
}

size_t permuted_bytes(int M, int d_in) {
  return M >= kPermuteMinRows ? ((size_t)M * d_in * 2 + 255) / 256 * 256 : 0;
}

size_t workspace_for(const GemmArgs& A) {
  const size_t xp = permuted_bytes(A.M, A.d_in);
  const PfPlan pf = prefill_plan(A.L, A.d_out, A.d_in, A.M);
  if (pf.kq) return xp + prefill_partial_bytes(pf, A.d_out, A.M);
  if (A.S == 1) return xp;
  const size_t part = (size_t)A.mchunks * A.S * A.mrows_chunk * A.rt * kTileRows * 4;
  const size_t cnt = (size_t)A.mchunks * A.rpairs * 4;
  return xp + (part + cnt + 255) / 256 * 256;
}

}  // namespace
}  // namespace sage

namespace sage {
namespace {

// The no-allocation entry point's workspace: a fixed device array, one copy per device the library
// runs on, held until the process ends. Host code never passes `scratch` itself (on the host the
// name is a stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t(SAGE_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of the current device's scratch array (resolved on first use per device).
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return SAGE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return SAGE_ERR_ARG;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return SAGE_ERR_HIP;
    }
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return SAGE_OK;
}

// Zero n words (the split-K arrival counters; a kernel, not hipMemsetAsync, so the call can be
// captured into a graph).
__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Both small-batch entry points. With from_scratch the workspace is the device's scratch array
// (ws and ws_bytes unused) and the arrival counters are zeroed before the product runs; otherwise
// it is the caller's zero-ready workspace.
int gemm_small_run(const sage_matrix_t* m, const uint16_t* X, int M, int ldx, uint16_t* Y, int ldy,
                   void* ws, size_t ws_bytes, bool from_scratch, sage_stream_t stream) {
  int st = check_matrix(m);
  if (st != SAGE_OK) return st;
  if (X == nullptr || Y == nullptr) return SAGE_ERR_NULL;
  if (M < 1 || ldx < m->d_in || ldy < m->d_out) return SAGE_ERR_SHAPE;
  if (!aligned(X, 4) || !aligned(Y, 2) || (ldx & 1)) return SAGE_ERR_ALIGN;
  if (M == 1) return sage_gemv(m, X, Y, nullptr, 0, stream);  // no workspace
  GemmArgs A{};
  A.packed = static_cast<const uint8_t*>(m->packed);
  A.codebook = m->codebook;
  A.pi = m->pi;
  A.X = X;
  A.Y = Y;
  A.ldx = ldx;
  A.ldy = ldy;
  A.d_out = m->d_out;
  A.d_in = m->d_in;
  A.M = M;
  A.L = m->log2K;
  plan(A, M);
  const size_t need = workspace_for(A);
  const size_t xp_bytes = permuted_bytes(M, A.d_in);
  if (from_scratch) {
    if (need > kScratchBytes) return SAGE_ERR_SCRATCH;
    if (need) {
      st = scratch_address(&ws);
      if (st != SAGE_OK) return st;
    }
  } else if (need) {
    if (ws == nullptr || ws_bytes < need) return SAGE_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return SAGE_ERR_ALIGN;
  }
  char* wsb = static_cast<char*>(ws);
  const PfPlan pf = prefill_plan(A.L, A.d_out, A.d_in, M);
  hipStream_t hs = (hipStream_t)stream;
  if (A.S > 1 && !pf.kq) {
    A.partial = reinterpret_cast<float*>(wsb + xp_bytes);
    A.counters = reinterpret_cast<uint32_t*>(
        wsb + xp_bytes + (size_t)A.mchunks * A.S * A.mrows_chunk * A.rt * kTileRows * 4);
    if (from_scratch) {
      // the array keeps whatever the device's previous call left there
      const int n = A.mchunks * A.rpairs;
      hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, hs,
                         A.counters, n);
    }
  }
  // Activations already in stored column order (pi = NULL) with 16-byte aligned rows are read in
  // place (a producer that writes its output permuted saves the reorder launch).
  const bool direct = m->pi == nullptr && aligned(X, 16) && (ldx % 8) == 0;
  const uint16_t* Xs = X;
  int64_t xs_ld = ldx;
  if (xp_bytes || direct) {
    // reorder the activations once, then every workgroup reads contiguous 16-byte chunks
    uint16_t* Xp = reinterpret_cast<uint16_t*>(wsb);
    const PermPlan pp = permute_plan(A.d_in, M, aligned(X, 16) && (ldx % 8) == 0);
    if (direct) {
      // nothing to reorder
    } else if (pp.rows > 0) {
      const dim3 grid((unsigned)ceil_div(M, pp.rows), (unsigned)pp.ranges);
      const size_t lds = (size_t)pp.rows * A.d_in * 2;
      const int64_t lx = ldx;
      switch (pp.rows) {
        case 8: hipLaunchKernelGGL(permute_rows_kernel<8>, grid, dim3(256), lds, hs, X, lx, m->pi, A.d_in, M, pp.units, Xp); break;
        case 4: hipLaunchKernelGGL(permute_rows_kernel<4>, grid, dim3(256), lds, hs, X, lx, m->pi, A.d_in, M, pp.units, Xp); break;
        case 2: hipLaunchKernelGGL(permute_rows_kernel<2>, grid, dim3(256), lds, hs, X, lx, m->pi, A.d_in, M, pp.units, Xp); break;
        default: hipLaunchKernelGGL(permute_rows_kernel<1>, grid, dim3(256), lds, hs, X, lx, m->pi, A.d_in, M, pp.units, Xp); break;
      }
    } else {
      hipLaunchKernelGGL(permute_gather_kernel,
                         dim3((unsigned)ceil_div(A.d_in, 256), (unsigned)std::min(M, 65535)),
                         dim3(256), 0, hs, X, (int64_t)ldx, m->pi, A.d_in, M, Xp);
    }
    if (!direct) {
      Xs = Xp;
      xs_ld = A.d_in;
    }
    if (pf.kq) {
      PrefillArgs P{};
      P.packed = A.packed;
      P.codebook = A.codebook;
      P.Xp = Xs;
      P.ldx = xs_ld;
      P.Y = Y;
      P.ldy = ldy;
      P.d_out = A.d_out;
      P.d_in = A.d_in;
      P.M = M;
      P.L = A.L;
      P.rt = A.rt;
      P.ng = A.ng;
      P.S = pf.S;
      P.gs = pf.gs;
      if (pf.S > 1) P.partial = reinterpret_cast<float*>(wsb + xp_bytes);
      const PrefillFn fn = prefill_fn(A.L, pf.kq);
      static bool attr_set[3][9] = {};
      const int kqi = pf.kq == 8 ? 2 : (pf.kq == 4 ? 1 : 0);
      if (!attr_set[kqi][A.L]) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr_set[kqi][A.L] = true;
      }
      const dim3 grid((unsigned)ceil_div(A.rt, kPfWaves), (unsigned)ceil_div(M, 32 * pf.kq),
                      (unsigned)pf.S);
      hipLaunchKernelGGL(fn, grid, dim3(kPfThreads), prefill_lds(A.L, pf.kq), hs, P);
      if (pf.S > 1) {
        const int64_t plane = prefill_plane(pf, A.d_out, M);
        hipLaunchKernelGGL(prefill_reduce_kernel, dim3((unsigned)((plane / 4 + 255) / 256)), dim3(256),
                           0, hs, P.partial, pf.S, plane, 32 * pf.kq, A.rt, M, A.d_out, Y,
                           (int64_t)ldy);
      }
      return hip_status();
    }
    A.X = Xs;
    A.ldx = xs_ld;
    A.pi = nullptr;
    A.vec_x = 1;
  } else {
    A.vec_x = 0;  // fewer than kPermuteMinRows rows, gathered through pi by the kernel
  }
  const int nt = tiles_for(M);
  const size_t lds = A.stream ? stream_lds(A.L, nt) : lds_for(A.L, nt, A.gs, A.tiles);
  const unsigned grid = (unsigned)(A.mchunks * A.rpairs * A.S);
  // Each instantiation gets its LDS limit raised once (slot = variant, split).
  static bool attr_set[8][9] = {};
  auto launch = [&](GemmFn kern, int slot) {
    if (!attr_set[slot][A.L]) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      attr_set[slot][A.L] = true;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kGThreads), lds, hs, A);
  };
  if (A.stream) {  // nt == 2 or 4, 1 x 4 with streamed activations
    if (nt == 2) launch(gemm_fn<2, true, 1, true>(A.L), 2);
    else launch(gemm_fn<4, true, 1, true>(A.L), 3);
  } else if (A.tiles == 1) {  // nt == 1, whole-vector rows
    launch(gemm_fn<1, true, 1>(A.L), 1);
  } else {
    if (!A.vec_x) launch(gemm_fn<1, false, 2>(A.L), 4);  // fewer than kPermuteMinRows rows: nt == 1
    else if (nt == 1) launch(gemm_fn<1, true, 2>(A.L), 5);
    else if (nt == 2) launch(gemm_fn<2, true, 2>(A.L), 6);
    else launch(gemm_fn<4, true, 2>(A.L), 7);
  }
  return hip_status();
}


}  // namespace
}  // namespace sage

using namespace sage;

extern "C" {

int sage_gemm_small_workspace_bytes(const sage_matrix_t* m, int M, size_t* bytes) {
  if (bytes == nullptr) return SAGE_ERR_NULL;
  int st = check_matrix(m);
  if (st != SAGE_OK) return st;
  if (M < 1) return SAGE_ERR_SHAPE;
  if (M == 1) return sage_gemv_workspace_bytes(m, bytes);  // one row: the batch-one kernel
  GemmArgs A{};
  A.d_out = m->d_out;
  A.d_in = m->d_in;
  A.M = M;
  A.L = m->log2K;
  plan(A, M);
  *bytes = workspace_for(A);
  return SAGE_OK;
}

int sage_gemm_small(const sage_matrix_t* m, const uint16_t* X, int M, int ldx, uint16_t* Y,
                    int ldy, void* ws, size_t ws_bytes, sage_stream_t stream) {
  return gemm_small_run(m, X, M, ldx, Y, ldy, ws, ws_bytes, false, stream);
}

int sage_gemm_small_noalloc(const sage_matrix_t* m, const uint16_t* X, int M, int ldx, uint16_t* Y,
                            int ldy, sage_stream_t stream) {
  return gemm_small_run(m, X, M, ldx, Y, ldy, nullptr, 0, true, stream);
}

}  // extern "C"
