// Batch-one decode-and-multiply for SAGE-packed weights on gfx950 (SAGE paper §3.5 and App. A.1).
//
// Work decomposition. Lane l of a wavefront owns output row 64 rt + l of one row tile. A workgroup
// has 16 wavefronts: 4 consecutive row tiles x 4 column parts. The workgroup owns a range of
// column groups (split-K over workgroups when the matrix alone does not fill the GPU, App. A.1 /
// §3.5); its columns are cut into half-groups (8 subvectors) and each column part takes a
// contiguous run of them. The four parts of a row tile add their sums in LDS. Every lane of a
// wave works on the same input columns at the same time, so the activations are uniform across
// the wave and no cross-lane reduction is needed. Sixteen waves per compute unit keep four waves
// on every SIMD, which hides the LDS latency of the decode loop.
//
// Per workgroup set-up, in LDS:
//   * the codebook, replicated 16 times with replica r at byte offset 16 r of each 256-byte row,
//     so lane l reads replica (l mod 16): random codeword gathers become bank-conflict free;
//   * the whole activation vector (when it fits), then the permuted activations x[pi[p]] of the
//     workgroup's columns, gathered once from LDS (§3.2 / §3.5);
//   * for every subvector position, a table of the 16 sign patterns of each 4-wide activation
//     half: entry n holds (x0..x3) and (x4..x7) with element i negated when bit i of n is set.
// A subvector is then: two conflict-free 8-byte table reads selected by the low and high sign
// nibbles, one 16-byte codeword read, four fp16 dot2 steps with fp32 accumulation, and the radius
// mu + q*delta applied once to the 8-term dot product (App. A.1 applies the radius after the dot
// for the same reason: one multiply instead of eight).
//
// Memory access. Every global load is a buffer load through a range-checked descriptor and is
// issued unconditionally (loads past the range return zeros without touching memory), so each
// wait before a use covers exactly the loads issued before it; the packed weights of a wave are
// all in flight before the LDS set-up starts.
//
// Split-K partials go to a caller workspace (coherent stores, no cache-wide fences); the last
// workgroup of a row-quad (atomic counter) sums them in split order, writes y in fp16 and resets
// the counter to zero.
#include <algorithm>

#include "sage_internal.hpp"
#include "sage_gemv.hpp"

namespace sage {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Range-checked buffer view: loads at offsets past `bytes` return zeros without a memory access.
__device__ inline __amdgpu_buffer_rsrc_t view(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
constexpr int kNonTemporal = 2;         // streamed once: no reuse expected in the caches
constexpr uint32_t kNowhere = 1u << 30;  // an offset past every range

// First step of a dot chain, accumulator 0 (VOP3P form, so no register needs zeroing first).
__device__ inline float dot2_z(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

// Sign pattern n applied to four fp16 values held as two packed dwords.
__device__ inline uint2 apply_nibble(uint32_t p01, uint32_t p23, uint32_t n) {
  const uint32_t m01 = ((n & 1u) << 15) | ((n & 2u) << 30);
  const uint32_t m23 = ((n & 4u) << 13) | ((n & 8u) << 28);
  return make_uint2(p01 ^ m01, p23 ^ m23);
}

// (a & m) | c in one VALU op with m in an SGPR and c in a VGPR (register-only inline asm).
__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}

// Compile-time constants and LDS layout of one split (L = log2 K).
template <int L>
struct SplitC {
  static constexpr uint32_t kK = 1u << L;
  static constexpr uint32_t kZMask = (kK - 1u) << 8;                      // F at bit 8
  static constexpr uint32_t kQMask = ((1u << (10 - L)) - 1u) << (8 + L);  // q at bit 8 + L
  // OR-ing this exponent onto q at bit 8+L gives the float 2^(15-L) + q exactly.
  static constexpr uint32_t kExpo = (127u + 15u - (uint32_t)L) << 23;
  static constexpr float kBias = (float)(1u << (15 - L));
  // LDS: codebook replicas, then the signed-activation tables, then the region that lds_tail()
  // describes.
  static constexpr uint32_t kCbOff = 0u;
  static constexpr uint32_t kXtOff = kK * 256u;
};

// Start of the LDS tail (gathered columns, part sums, flag, whole x) for split L and gs groups.
__host__ __device__ inline uint32_t lds_tail(int L, int gs) {
  return (1u << L) * 256u + (uint32_t)gs * kSubPerGroup * 256u;
}
// Offsets inside the tail for workgroup shape T (row tiles): gathered columns fp16 [max gs * 128]
// (only when x is not staged whole), part sums f32 [parts - 1][T][64] (chunked shape: [16
// waves][64]), flag, whole x fp16 [d_in] when staged.
constexpr uint32_t kTailXp = 0;
__host__ __device__ constexpr uint32_t tail_red(int T, bool whole) {
  return whole ? 0u : shape_max_gs(T) * kGroupCols * 2;
}
__host__ __device__ constexpr uint32_t red_bytes(int T) {
  return T == 0 ? kWaves * 64 * 4 : (kWaves / T - 1) * T * 64 * 4;
}
__host__ __device__ constexpr uint32_t tail_flag(int T, bool whole) {
  return tail_red(T, whole) + red_bytes(T);
}
__host__ __device__ constexpr uint32_t tail_x(int T, bool whole) {
  return (tail_flag(T, whole) + 16 + 255) / 256 * 256;
}

struct Resolved {
  const uint8_t* packed;
  const uint16_t* codebook;
  const int32_t* pi;
  int L;
};

// One half-group of one lane: four payload dwords (one plane), then the side dwords X and G.
struct UnitRegs {
  uint32_t p[4];
  uint32_t x, g;
};

__device__ inline void load_unit(UnitRegs& r, __amdgpu_buffer_rsrc_t rs, uint32_t main_off,
                                 uint32_t side_off) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, main_off, 0, kNonTemporal);
  const u32x2 s = __builtin_amdgcn_raw_buffer_load_b64(rs, side_off, 0, kNonTemporal);
  r.p[0] = a[0]; r.p[1] = a[1]; r.p[2] = a[2]; r.p[3] = a[3];
  r.x = s[0];
  r.g = s[1];
}

// LDS reads at absolute LDS byte addresses. The kernel declares no static LDS, so its dynamic LDS
// starts at address 0 and compile-time offsets become ds_read immediates.
typedef __attribute__((address_space(3))) const u32x2 lds_u2;
typedef __attribute__((address_space(3))) const u32x4 lds_u4;
__device__ inline uint2 lds8(uint32_t addr) {
  const u32x2 v = *(lds_u2*)(size_t)addr;
  return make_uint2(v.x, v.y);
}
__device__ inline uint4 lds16(uint32_t addr) {
  const u32x4 v = *(lds_u4*)(size_t)addr;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One subvector: two signed-activation half reads, one codeword read, 4 dot2, radius, accumulate.
// lo and hi already hold the table base and the nibble offset; off is the step's offset.
template <int L>
__device__ __forceinline__ float subvec(int off, uint32_t lo, uint32_t hi, uint32_t cz,
                                        uint32_t qbits, float dl, float mu_b, float acc) {
  const uint2 x0 = lds8(lo + (uint32_t)off);
  const uint2 x1 = lds8(hi + (uint32_t)(off + 8));
  const uint4 c = lds16(cz + SplitC<L>::kCbOff);
  float t = dot2_z(c.x, x0.x);
  t = dot2(c.y, x0.y, t);
  t = dot2(c.z, x1.x, t);
  t = dot2(c.w, x1.y, t);
  const float r = fmaf(__uint_as_float(qbits), dl, mu_b);
  return fmaf(r, t, acc);
}

// The 8 subvectors of one half-group: payload dwords P_{4h+ii} (ii = 0..3), pairs a = 2ii and
// b = 2ii + 1 of the half. tb is the LDS address of the half's first table.
template <int L>
__device__ __forceinline__ float half_dot(const UnitRegs& U, uint32_t h, uint32_t tb,
                                          uint32_t laneoff, uint32_t expo, float acc) {
  using C = SplitC<L>;
  const float mu = h2f(U.g);
  const float dl = h2f(U.g >> 16);
  const float mu_b = fmaf(-C::kBias, dl, mu);  // radius = (2^(15-L) + q) * delta + mu_b
  const uint32_t xa = U.x >> (16u * h);        // high sign nibbles of this half's b subvectors
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const uint32_t P = U.p[ii];
    // subvector a: nibbles at bits 4..7 and 28..31, field at bit 8
    acc = subvec<L>((2 * ii) * 256, and_or(P, 0xF0u, tb), and_or(P >> 24, 0xF0u, tb),
                                    and_or(P, C::kZMask, laneoff), and_or(P, C::kQMask, expo), dl,
                                    mu_b, acc);
    // subvector b: low nibble at bits 0..3 of P, high nibble in slot ii of xa, field at bit 18
    const uint32_t xs = ii == 0 ? (xa << 4) : ii == 1 ? xa : ii == 2 ? (xa >> 4) : (xa >> 8);
    const uint32_t Pb = P >> 10;
    acc = subvec<L>((2 * ii + 1) * 256, and_or(P << 4, 0xF0u, tb), and_or(xs, 0xF0u, tb),
                                        and_or(Pb, C::kZMask, laneoff),
                                        and_or(Pb, C::kQMask, expo), dl, mu_b, acc);
  }
  return acc;
}

// A producer row group is complete: its fp32 rows are acknowledged, then one signal.
__device__ inline void signal_row_group(const Job& J, int tid) {
  wait_stores();
  __syncthreads();
  if (tid == 0) counter_add(J.sync);
}

// Input of a consumer piece (second stage of a fused SwiGLU MLP): waits until every producer row
// group has signalled, then writes h = fp16(silu(fp16(g)) * fp16(u)) for all d_in entries to xw.
// The wait is bounded; a wait that runs out is counted in sync[2] and the launch completes.
constexpr int kSpinLimit = 1 << 17;
__device__ inline void mlp_input(const Job& J, uint16_t* xw, int tid) {
  if (tid == 0) {
    uint32_t n = load_coherent_u32(J.sync);
    for (int it = 0; n < (uint32_t)J.signal_total && it < kSpinLimit; ++it) {
      __builtin_amdgcn_s_sleep(8);
      n = load_coherent_u32(J.sync);
    }
    if (n < (uint32_t)J.signal_total) counter_add(J.sync + 2);
  }
  __syncthreads();
  constexpr int kH = kWholeXMax / 4 / kThreads;  // 4-float chunks per thread
  const uint32_t bytes = (uint32_t)J.d_in * 4u;
  const __amdgpu_buffer_rsrc_t g_rs = coherent_rsrc(J.src_gate, bytes);
  const __amdgpu_buffer_rsrc_t u_rs = coherent_rsrc(J.src_up, bytes);
  u32x4 g[kH], u[kH];
#pragma unroll
  for (int i = 0; i < kH; ++i) {
    const uint32_t off = (uint32_t)(tid + i * kThreads) * 16u;
    g[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(g_rs, off, 0, 0x10));
    u[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(u_rs, off, 0, 0x10));
  }
  const bool copy_out = J.h_out != nullptr && blockIdx.x == 0;
#pragma unroll
  for (int i = 0; i < kH; ++i) {
    const int e = tid + i * kThreads;
    if (e * 4 >= J.d_in) continue;
    uint16_t hv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float g16 = (float)(_Float16)__uint_as_float(g[i][q]);
      const float u16 = (float)(_Float16)__uint_as_float(u[i][q]);
      hv[q] = f2h(g16 / (1.0f + __expf(-g16)) * u16);
    }
    const uint2 packed = make_uint2(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16));
    *reinterpret_cast<uint2*>(xw + e * 4) = packed;
    if (copy_out) *reinterpret_cast<uint2*>(J.h_out + e * 4) = packed;
  }
  if (tid == 0) {
    if (counter_add(J.sync + 1) == (uint32_t)(J.consumer_wgs - 1)) {
      counter_reset(J.sync);
      counter_reset(J.sync + 1);
    }
  }
}

template <int L, int kT, bool kWholeX, bool kFused, int kMU, bool kStream>
__device__ __forceinline__ void gemv_body(const Resolved& R, const Job& J, const ChunkMap& CM,
                                          int inst, int rq, int split, uint8_t* smem) {
  using C = SplitC<L>;
  constexpr int kTiles = WgShape<kT>::kTiles;
  constexpr int kParts = WgShape<kT>::kParts;
  // half-group steps a wave can take in this launch (the loads of a wave stop there: a load
  // instruction costs address-unit time even when no lane is in range)
  constexpr int kMaxUnits = kMU;
  static_assert(kMU <= WgShape<kT>::kMaxUnits, "more steps than the shape allows");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: addresses in SGPRs
  const int lane = tid & 63;
  // chunked shape: this wave's entries of the work map, read first (their latency then overlaps
  // that of the piece's fields)
  uint32_t cm_lo = 0, cm_hi = 0, cm_red[8] = {};
  int wmax = 0, presum = 0;
  if constexpr (kT == 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      cm_red[q] = CM.red[q];
      asm volatile("" ::"s"(cm_red[q]));  // scalar loads, issued now
    }
    cm_lo = *reinterpret_cast<const uint32_t*>(&CM.lane_group[wave * 4]);
    cm_hi = *reinterpret_cast<const uint32_t*>(&CM.lane_group[wave * 4 + 2]);
    const uint32_t wi = CM.wave[wave];
    wmax = (int)(wi & 255u);
    presum = (int)(wi >> 8);
    asm volatile("" ::"s"(cm_lo), "s"(cm_hi), "s"(wi));  // issue these loads now
  }
  const int tile = wave % kTiles;
  const int part = wave / kTiles;
  const int g0 = split * J.gs;
  const int ngl = min(J.ng - g0, J.gs);
  const int rt = rq * kTiles + tile;  // row tile inside the piece
  const bool tile_ok = rt < J.rt;
  // Half-groups of this wave (<= kMaxUnits): the first units % kParts parts take one more. The
  // waves of one SIMD hold parts that are kParts / 4 apart, so every SIMD gets the same share.
  const int units = 2 * ngl;
  const int ubase = units / kParts;
  const int uextra = units - ubase * kParts;
  const int u0 = part * ubase + min(part, uextra);
  const int nu = ubase + (part < uextra ? 1 : 0);
  // Chunked shape: this lane group's chunk and half-group range (us, un), and the wave's steps.
  int ck = 0, us = 0, un = 0;
  if constexpr (kT == 0) {
    const int lg = lane >> 4;
    const uint32_t e = ((lg & 2) ? cm_hi : cm_lo) >> ((lg & 1) * 16);
    ck = (int)(e & 15u);
    un = (int)((e >> 4) & 15u);
    us = (int)((e >> 8) & 255u);
  }
  const int c0 = g0 * kGroupCols;
  const int cols = ngl * kGroupCols;
  const uint32_t tail = lds_tail(L, J.gs);
  uint16_t* xp = reinterpret_cast<uint16_t*>(smem + tail + kTailXp);
  float* red = reinterpret_cast<float*>(smem + tail + tail_red(kT, kWholeX));
  uint32_t* flag = reinterpret_cast<uint32_t*>(smem + tail + tail_flag(kT, kWholeX));

  // 1. Loads, in the order their data is needed.
  const __amdgpu_buffer_rsrc_t cb_rs = view(R.codebook, C::kK * 16u);
  const __amdgpu_buffer_rsrc_t pi_rs = view(R.pi ? R.pi + c0 : nullptr, R.pi ? cols * 4u : 0u);
  const bool consumer = kFused && J.src_gate != nullptr;  // input built in LDS from a first stage
  const __amdgpu_buffer_rsrc_t x_rs =
      view(consumer ? nullptr : J.x + (int64_t)inst * J.x_stride, consumer ? 0u : (uint32_t)J.d_in * 2u);
  const uint8_t* blk0 =
      kT == 0 ? R.packed : R.packed + ((int64_t)(J.tile0 + rt) * J.ng + g0) * kBlockBytes;
  const uint32_t w_bytes =
      kT == 0 ? (uint32_t)((J.d_out + kTileRows - 1) / kTileRows * J.ng * kBlockBytes)
              : (tile_ok ? (uint32_t)(ngl * kBlockBytes) : 0u);
  const __amdgpu_buffer_rsrc_t w_rs = view(blk0, w_bytes);

  // Waves whose lanes would all read past a small array skip the load (wave-uniform branches):
  // a load instruction takes the same address-unit time whether or not its lanes are in range.
  // With x staged whole its loads go first, so the staging waits for nothing else.
  constexpr int kChunks = kWholeXMax / 8 / kThreads;  // 16-byte chunks of x per thread
  u32x4 xc[kChunks];
  if constexpr (kWholeX) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      xc[i] = u32x4{0u, 0u, 0u, 0u};
      if ((wave * 64 + i * kThreads) * 8 < J.d_in)
        xc[i] = __builtin_amdgcn_raw_buffer_load_b128(x_rs, (tid + i * kThreads) * 16, 0, 0);
    }
  }
  u32x4 cw = {0u, 0u, 0u, 0u};
  if (wave * 64 < (int)C::kK) cw = __builtin_amdgcn_raw_buffer_load_b128(cb_rs, tid * 16, 0, 0);
  // columns of the workgroup per thread: one for 4 x 4 (8 groups), up to three for the others
  constexpr int kCpt = (WgShape<kT>::kMaxGS * kGroupCols + kThreads - 1) / kThreads;
  // Whole x staged: the tables of subvector position s are written by tps threads, which read
  // the eight pi entries of s. Otherwise thread t gathers columns t + 1024 k from memory.
  const int steps = ngl * kSubPerGroup;  // subvector positions of the workgroup
  const int tps = steps * 2 <= kThreads ? 2 : 1;  // more would repeat the pi loads
  const int tshift = tps - 1;
  const int my_step = tid >> tshift;
  uint32_t src[kCpt];
  u32x4 ps[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  if constexpr (kWholeX) {
    if (((wave * 64) >> tshift) < steps) {
      ps[0] = __builtin_amdgcn_raw_buffer_load_b128(pi_rs, my_step * 32, 0, 0);
      ps[1] = __builtin_amdgcn_raw_buffer_load_b128(pi_rs, my_step * 32 + 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kCpt; ++k) {
      src[k] = 0u;
      if (wave * 64 + k * kThreads < cols)
        src[k] = __builtin_amdgcn_raw_buffer_load_b32(pi_rs, (tid + k * kThreads) * 4, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order: the counters wait in order
  const uint32_t last = (uint32_t)J.d_in - 1u;  // an out-of-range pi entry is clamped
  // identity when pi is absent, as a lane mask rather than a branch
  uint32_t use_pi = R.pi ? ~0u : 0u;
  asm volatile("" : "+v"(use_pi));
  UnitRegs U[kMaxUnits];
  uint16_t xv[kCpt] = {};
  if constexpr (!kWholeX) {
    // wide inputs: the gathered activations straight from memory, after pi
#pragma unroll
    for (int k = 0; k < kCpt; ++k) {
      const uint32_t c = (uint32_t)(c0 + tid + k * kThreads);
      const uint32_t col = (min(src[k], last) & use_pi) | (c & ~use_pi);
      xv[k] = __builtin_amdgcn_raw_buffer_load_b16(x_rs, col * 2u, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // chunked shape: the packed half-groups of this lane group for workgroup block rqb (lane l:
  // row 16 * chunk + l % 16, i.e. row (chunk % 4) * 16 + l % 16 of tile chunk / 4)
  auto load_block = [&](UnitRegs (&Ux)[kMaxUnits], int rqb) {
    const int gc = J.chunk0 + rqb * J.cq + ck;
    const bool cok = ck < J.cq && gc < J.chunk0 + J.nchunk;
    const uint32_t rin = (uint32_t)((gc & 3) * kChunkRows + (lane & 15));
    const uint32_t tbase = (uint32_t)((gc >> 2) * J.ng + g0) * kBlockBytes;
#pragma unroll
    for (int k = 0; k < kMaxUnits; ++k) {
      const int u = us + k;
      const uint32_t blk = tbase + (uint32_t)(u >> 1) * kBlockBytes;
      const bool ok = cok && k < un;
      load_unit(Ux[k], w_rs, ok ? blk + ((u & 1) ? kPlaneB : kPlaneA) + rin * 16 : kNowhere,
                ok ? blk + kSidePlane + rin * 8 : kNowhere);
    }
  };
  if constexpr (kT == 0) {
    load_block(U, rq);
  } else {
#pragma unroll
    for (int k = 0; k < kMaxUnits; ++k) {
      const int u = u0 + k;
      const uint32_t blk = (uint32_t)(u >> 1) * kBlockBytes;
      const bool ok = k < nu;
      load_unit(U[k], w_rs, ok ? blk + ((u & 1) ? kPlaneB : kPlaneA) + lane * 16 : kNowhere,
                ok ? blk + kSidePlane + lane * 8 : kNowhere);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. LDS set-up: replicated codebook, gathered activations, signed-activation tables.
  if (tid < (int)C::kK) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      *reinterpret_cast<u32x4*>(smem + C::kCbOff + tid * 256 + r * 16) = cw;
  }
  if constexpr (kWholeX) {
    uint16_t* xw = reinterpret_cast<uint16_t*>(smem + tail + tail_x(kT, true));
    if (kFused && consumer) {
      mlp_input(J, xw, tid);
    } else {
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
        if (tid + i * kThreads < J.d_in / 8)
          *reinterpret_cast<u32x4*>(xw + (tid + i * kThreads) * 8) = xc[i];
    }
    __syncthreads();
    // the threads of position s gather its eight activations through pi, then write 16 / tps of
    // its 16 table entries each (no second pass through a gathered copy, one barrier less)
    if (my_step < steps) {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t pv = ps[i >> 2][i & 3];
        const uint32_t col =
            (min(pv, last) & use_pi) | ((uint32_t)(c0 + my_step * 8 + i) & ~use_pi);
        h[i] = xw[col];
      }
      const uint32_t p01 = h[0] | (h[1] << 16), p23 = h[2] | (h[3] << 16);
      const uint32_t p45 = h[4] | (h[5] << 16), p67 = h[6] | (h[7] << 16);
      // thread q of a position writes entries q * np + (i + s) mod np: the eight lanes of one
      // 128-byte write cycle then land in eight different 16-byte slots (all banks)
      const int np = 16 >> tshift, q = tid & (tps - 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < np) {
          const uint32_t n = (uint32_t)(q * np + ((i + my_step) & (np - 1)));
          const uint2 lo = apply_nibble(p01, p23, n);
          const uint2 hi = apply_nibble(p45, p67, n);
          *reinterpret_cast<uint4*>(smem + C::kXtOff + my_step * 256 + n * 16) =
              make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kCpt; ++k)
      if (tid + k * kThreads < cols) xp[tid + k * kThreads] = xv[k];
    __syncthreads();
    for (int e = tid; e < ngl * kSubPerGroup * 16; e += kThreads) {
      const int step = e >> 4;
      const uint32_t n = (uint32_t)(e & 15);
      const uint4 v = *reinterpret_cast<const uint4*>(xp + step * 8);
      const uint2 lo = apply_nibble(v.x, v.y, n);
      const uint2 hi = apply_nibble(v.z, v.w, n);
      *reinterpret_cast<uint4*>(smem + C::kXtOff + step * 256 + n * 16) =
          make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
  __syncthreads();

  // 3. Decode and multiply this wave's half-groups. The four waves of a SIMD share its issue
  // slots, which go to the oldest wave first; a wave's priority is its remaining work (3 down to
  // 0), so the waves advance together and the SIMD stays busy until the last one ends.
  const uint32_t laneoff = (uint32_t)(lane & 15) * 16u;
  const uint32_t expo = C::kExpo;
  if constexpr (kT == 0) {
    auto decode_block = [&](const UnitRegs (&Ux)[kMaxUnits]) {
      float a = 0.0f;
      __builtin_amdgcn_s_setprio(3);
#pragma unroll
      for (int k = 0; k < kMaxUnits; ++k) {
        if (k < wmax) {
          // lane groups past their range keep their sum (their unit, clamped into the split,
          // addresses valid tables; its zero-filled payload is discarded)
          const uint32_t u = (uint32_t)min(us + k, units - 1);
          const uint32_t tb = C::kXtOff + (u >> 1) * (kSubPerGroup * 256) + (u & 1) * (8 * 256);
          const float a2 = half_dot<L>(Ux[k], u & 1, tb, laneoff, expo, a);
          a = k < un ? a2 : a;
          const int left = wmax - 1 - k;
          if (left == 2) __builtin_amdgcn_s_setprio(2);
          else if (left == 1) __builtin_amdgcn_s_setprio(1);
          else if (left == 0) __builtin_amdgcn_s_setprio(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      return a;
    };
    // The lane groups of a chunk add up in a fixed order, main waves first, then the
    // remaining-chunk lane groups; thread t sums row t % 16 of chunk t / 16 of block rqb.
    uint32_t rm = cm_red[0];  // contributors of this thread's chunk
#pragma unroll
    for (int q = 1; q < 8; ++q) rm = (tid >> 4) == q ? cm_red[q] : rm;
    auto reduce_store = [&](float a, int rqb) {
      if (presum >= 2) a += __shfl_xor(a, 16);
      if (presum >= 1) a += __shfl_xor(a, 32);
      red[wave * 64 + lane] = a;
      __syncthreads();
      if (tid < J.cq * kChunkRows) {
        const int c = tid >> 4, r = tid & 15;
        const int first = (int)(rm & 63u), step = (int)((rm >> 6) & 63u), count = (int)(rm >> 12);
        // sixteen LDS reads in flight at a time (zero past the last contributor), added as a
        // fixed pairwise tree
        float sum = 0.0f;
        for (int i0 = 0; i0 < count; i0 += 16) {
          float v[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float t = red[min(first + (i0 + i) * step, 63) * 16 + r];
            v[i] = i0 + i < count ? t : 0.0f;
          }
#pragma unroll
          for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
            for (int i = 0; i < w; ++i) v[i] = v[2 * i] + v[2 * i + 1];
          sum += v[0];
        }
        const int gc = J.chunk0 + rqb * J.cq + c;
        const int row = gc * kChunkRows + r;
        if (gc < J.chunk0 + J.nchunk && row < J.d_out) {
          uint16_t* yv = J.y + (int64_t)inst * J.y_stride;
          yv[row] = f2h(sum);
        }
      }
    };
    if constexpr (!kStream) {
      reduce_store(decode_block(U), rq);
    } else {
      // Persistent workgroups (launches of several rounds): the tables are built once, then the
      // workgroup takes blocks rq, rq + G, rq + 2G, ... (G workgroups in the launch) with the
      // next block's weights loading into the other register set while this one decodes.
      const int G = J.wg_per_inst;
      UnitRegs V[kMaxUnits];
      for (int b = rq; b < J.rq; b += 2 * G) {
        load_block(V, b + G);
        reduce_store(decode_block(U), b);
        __syncthreads();  // the part sums of the next block reuse the LDS
        if (b + G >= J.rq) break;
        load_block(U, b + 2 * G);
        reduce_store(decode_block(V), b + G);
        __syncthreads();
      }
    }
    return;
  }
  float acc = 0.0f;
  __builtin_amdgcn_s_setprio(3);
  const int nloop = nu;
#pragma unroll
  for (int k = 0; k < kMaxUnits; ++k) {
    if (k < nloop) {
      const uint32_t u = (uint32_t)(u0 + k);
      const uint32_t tb = C::kXtOff + (u >> 1) * (kSubPerGroup * 256) + (u & 1) * (8 * 256);
      acc = half_dot<L>(U[k], u & 1, tb, laneoff, expo, acc);
      const int left = nloop - 1 - k;
      if (left == 2) __builtin_amdgcn_s_setprio(2);
      else if (left == 1) __builtin_amdgcn_s_setprio(1);
      else if (left == 0) __builtin_amdgcn_s_setprio(0);
    }
  }
  __builtin_amdgcn_s_setprio(0);

  // 4. Column parts of a row tile add up in LDS (in part order).
  if (part > 0) red[((part - 1) * kTiles + tile) * 64 + lane] = acc;
  __syncthreads();
  if (part == 0) {
#pragma unroll
    for (int p = 1; p < kParts; ++p) acc += red[((p - 1) * kTiles + tile) * 64 + lane];
  }

  // 5. Output: direct, or split-K partials reduced by the last workgroup of the row quad.
  const int row_local = rt * kTileRows + lane;
  const int row = J.tile0 * kTileRows + row_local;
  const bool row_ok = part == 0 && tile_ok && row < J.d_out;
  uint16_t* y = J.y != nullptr ? J.y + (int64_t)inst * J.y_stride : nullptr;
  if (J.S == 1) {
    if (row_ok) {
      if (y != nullptr) y[row] = f2h(acc);
      if (kFused && J.out32 != nullptr) store_coherent(J.out32 + row, acc);
    }
    if (kFused && J.out32 != nullptr) signal_row_group(J, tid);
    return;
  }
  float* pbuf = J.partial + (int64_t)inst * J.partial_stride;
  const int64_t rows_pad = (int64_t)J.rt * kTileRows;
  if (row_ok) store_coherent(pbuf + (int64_t)split * rows_pad + row_local, acc);
  wait_stores();
  __syncthreads();
  uint32_t* counter = J.counters + (int64_t)inst * J.counters_stride + rq;
  if (tid == 0) *flag = (counter_add(counter) == (uint32_t)(J.S - 1)) ? 1u : 0u;
  __syncthreads();
  if (*flag == 0u) return;
  if (row_ok) {
    // all partials of this row, 32 at a time in flight, summed in split order
    const __amdgpu_buffer_rsrc_t rs =
        coherent_rsrc(pbuf, (uint32_t)(J.S * rows_pad * (int64_t)sizeof(float)));
    float s = 0.0f;
    for (int sp0 = 0; sp0 < J.S; sp0 += 32) {
      float v[32];
#pragma unroll
      for (int q = 0; q < 32; ++q)
        v[q] = load_coherent_at(rs, (uint32_t)(((sp0 + q) * rows_pad + row_local) * sizeof(float)));
#pragma unroll
      for (int q = 0; q < 32; ++q)
        if (sp0 + q < J.S) s += v[q];
    }
    if (y != nullptr) y[row] = f2h(s);
    if (kFused && J.out32 != nullptr) store_coherent(J.out32 + row, s);
  }
  if (tid == 0) counter_reset(counter);
  if (kFused && J.out32 != nullptr) signal_row_group(J, tid);
}

template <int kT, bool kWholeX, bool kFused, int kMU, bool kStream = false>
__global__ void __launch_bounds__(kThreads) gemv_kernel(JobTable T) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Job& J = T.jobs[blockIdx.y];
  // Touch every 64-byte line of the piece (and of the chunk map) at once, so the argument reads
  // that follow (several depend on one another through branches) hit the scalar cache instead of
  // waiting for one memory round trip each.
  {
    const uint32_t* jw = reinterpret_cast<const uint32_t*>(&J);
    constexpr int kLast = (int)(sizeof(Job) / 4) - 1;
    const uint32_t a0 = jw[0], a1 = jw[16], a2 = jw[32], a3 = jw[48 < kLast ? 48 : kLast],
                   a4 = jw[kLast];
    asm volatile("" ::"s"(a0), "s"(a1), "s"(a2), "s"(a3), "s"(a4));
    if constexpr (kT == 0) {
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(&T.cmap);
      constexpr int kCLast = (int)(sizeof(ChunkMap) / 4) - 1;
      const uint32_t c0 = cw[0], c1 = cw[16], c2 = cw[32], c3 = cw[kCLast];
      asm volatile("" ::"s"(c0), "s"(c1), "s"(c2), "s"(c3));
    }
  }
  int local = blockIdx.x;
  if (local >= J.wg_per_inst * J.inst) return;  // the grid is as wide as the widest piece
  const int inst = local / J.wg_per_inst;
  local -= inst * J.wg_per_inst;
  const int rq = local / J.S;
  const int split = local - rq * J.S;
  Resolved R;
  if (J.table != nullptr) {
    const uint32_t e = min((uint32_t)gview(J.ids)[inst], (uint32_t)J.n_experts - 1u);
    const sage_matrix_t* M = J.table + (int64_t)e * J.tstride + J.toff;
    R.packed = static_cast<const uint8_t*>(M->packed);
    R.codebook = M->codebook;
    R.pi = M->pi;
    R.L = M->log2K;
  } else {
    R.packed = J.packed;
    R.codebook = J.codebook;
    R.pi = J.pi;
    R.L = J.log2K;
  }
  switch (R.L) {
    case 4: gemv_body<4, kT, kWholeX, kFused, kMU, kStream>(R, J, T.cmap, inst, rq, split, smem); break;
    case 5: gemv_body<5, kT, kWholeX, kFused, kMU, kStream>(R, J, T.cmap, inst, rq, split, smem); break;
    case 6: gemv_body<6, kT, kWholeX, kFused, kMU, kStream>(R, J, T.cmap, inst, rq, split, smem); break;
    case 7: gemv_body<7, kT, kWholeX, kFused, kMU, kStream>(R, J, T.cmap, inst, rq, split, smem); break;
    default: gemv_body<8, kT, kWholeX, kFused, kMU, kStream>(R, J, T.cmap, inst, rq, split, smem); break;
  }
}

// ------------------------------------------------------------------------------------------------
// Host planning

// One product of a launch before it is cut into pieces.
struct Product {
  int d_out, d_in, inst;
};

struct Plan {
  int tiles;              // workgroup shape: row tiles per workgroup (4, 2 or 1; 0 = chunked)
  int cq, cwm;            // chunked shape: chunks per workgroup, waves on whole quads
  bool stream;            // chunked shape with persistent workgroups (several blocks each)
  int gs;                 // groups per split (before balancing per product)
  int n;                  // pieces
  Job pieces[kMaxJobs];   // planning fields filled: d_out, d_in, tile0, rt, rq, ng, S, gs, inst
  int src[kMaxJobs];      // product index of each piece
  int grid_x;
};

int64_t launch_wgs(const Product* p, int n, int gs, int T) {
  int64_t wgs = 0;
  for (int i = 0; i < n; ++i) {
    const int ng = p[i].d_in / kGroupCols;
    const int g = gs < ng ? gs : ng;
    wgs += (int64_t)p[i].inst * ceil_div(ceil_div(p[i].d_out, kTileRows), T) * ceil_div(ng, g);
  }
  return wgs;
}

size_t lds_bytes(int maxL, int gs, int whole_d_in, int T) {
  size_t need = 0;
  for (int L = 4; L <= maxL; ++L) {
    const size_t b = lds_tail(L, gs) + tail_x(T, whole_d_in > 0);
    if (b > need) need = b;
  }
  return need + (size_t)whole_d_in * 2;
}

// Groups per split: the fewest that keep the launch within one workgroup per compute unit (a
// workgroup fills a compute unit), so every launch runs in a single round with the least work
// per workgroup; the largest allowed when even that does not fit.
int plan_gs(const Product* p, int n, int T) {
  const int64_t cus = device_cu_count();
  for (int gs = 1; gs <= shape_max_gs(T); ++gs)
    if (launch_wgs(p, n, gs, T) <= cus) return gs;
  return shape_max_gs(T);
}

// Issue-slot cost of a workgroup: the largest number of half-group steps one SIMD runs (wave w
// sits on SIMD w % 4 and a wave steps as long as its longest lane group).
int shape_cost(int T, int units) {
  const int parts = kWaves / T;
  const int base = units / parts, extra = units % parts;
  int worst = 0;
  for (int s = 0; s < 4; ++s) {
    int sum = 0;
    for (int w = s; w < kWaves; w += 4) {
      const int part = w / T;
      sum += base + (part < extra ? 1 : 0);
    }
    worst = std::max(worst, sum);
  }
  return worst;
}

// Work map of the chunked shape with Q chunks, cwm main waves and `units` half-groups per lane
// (ChunkMap in sage_gemv.hpp). Main waves take the whole quads of chunks: wave w works on quad
// w % (Q / 4), lane group g on chunk 4 (w % (Q / 4)) + g, all four on the same half-group range
// (so they read the same table rows); the quad's ranges split the half-groups evenly. The other
// waves take the Q % 4 remaining chunks: lane group h (counted from the first such wave) works
// on remaining chunk h % (Q % 4) with its own range. Returns the issue-slot cost (largest sum of
// wave steps on one SIMD, wave w on SIMD w % 4), or -1 when a lane group would get more than
// kMaxChunkUnits half-groups.
int chunk_map(int Q, int cwm, int units, ChunkMap& M) {
  const int nq = Q >> 2, nb = Q & 3;
  M = ChunkMap{};
  for (int w = 0; w < kWaves; ++w) {
    int longest = 0;
    for (int g = 0; g < 4; ++g) {
      int ck, us, un;
      if (w < cwm) {
        const int a = w % nq, ri = w / nq;
        const int nr = (cwm - a + nq - 1) / nq;
        ck = 4 * a + g;
        us = ri * (units / nr) + std::min(ri, units % nr);
        un = units / nr + (ri < units % nr ? 1 : 0);
      } else {
        const int nr = 4 * (kWaves - cwm) / nb;
        const int h = (w - cwm) * 4 + g, ri = h / nb;
        ck = 4 * nq + h % nb;
        const bool valid = h < nr * nb;
        us = valid ? ri * (units / nr) + std::min(ri, units % nr) : 0;
        un = valid ? units / nr + (ri < units % nr ? 1 : 0) : 0;
      }
      if (un > kMaxChunkUnits) return -1;
      M.lane_group[w * 4 + g] = (uint16_t)(ck | (un << 4) | (us << 8));
      longest = std::max(longest, un);
    }
    const int presum = w < cwm ? 0 : (nb == 1 ? 2 : (nb == 2 ? 1 : 0));
    M.wave[w] = (uint32_t)longest | ((uint32_t)presum << 8);
  }
  for (int c = 0; c < Q; ++c) {
    int first, step, count;
    if (c < 4 * nq) {
      first = (c >> 2) * 4 + (c & 3);
      step = 4 * nq;
      count = (cwm - (c >> 2) + nq - 1) / nq;
    } else if (nb <= 2) {  // summed inside each wave first: lane group c - 4 nq of every wave
      first = 4 * cwm + (c - 4 * nq);
      step = 4;
      count = kWaves - cwm;
    } else {
      first = 4 * cwm + (c - 4 * nq);
      step = nb;
      count = 4 * (kWaves - cwm) / nb;
    }
    M.red[c] = (uint32_t)first | ((uint32_t)step << 6) | ((uint32_t)count << 12);
  }
  int worst = 0;
  for (int s = 0; s < 4; ++s) {
    int sum = 0;
    for (int w = s; w < kWaves; w += 4) sum += (int)(M.wave[w] & 255u);
    worst = std::max(worst, sum);
  }
  return worst;
}

// Best chunked workgroup for one split of `units` half-groups: Q chunks per workgroup (the launch
// within one workgroup per compute unit) and the number of main waves with the lowest cost.
// Returns the cost, or -1 when no Q fits.
int plan_chunks(const Product* p, int n, int units, int& best_q, int& best_wm) {
  const int64_t cus = device_cu_count();
  int best = -1;
  for (int Q = 1; Q <= 8; ++Q) {
    int64_t wgs = 0;
    for (int i = 0; i < n; ++i) wgs += (int64_t)p[i].inst * ceil_div(ceil_div(p[i].d_out, kChunkRows), Q);
    if (wgs > cus) continue;
    const int nq = Q >> 2, nb = Q & 3;
    // main waves: all of them without remaining chunks, none without quads, else at least one
    // per quad and at least one wave left for the remaining chunks
    const int lo = nb == 0 ? kWaves : nq, hi = nb == 0 ? kWaves : (nq == 0 ? 0 : kWaves - 1);
    for (int wm = hi; wm >= lo; --wm) {  // ties: more main waves (one table row per wave)
      ChunkMap M;
      const int c = chunk_map(Q, wm, units, M);
      if (c >= 0 && (best < 0 || c < best)) {
        best = c;
        best_q = Q;
        best_wm = wm;
      }
    }
  }
  return best;
}

// Workgroup shape and groups per split of a batch-one launch (every shape within the LDS: the
// codebook of the largest split in the launch, the tables of its groups, the staged x), measured
// on the decoder layer:
//   1. one split per product when a shape with more parts per tile fits it in one workgroup per
//      compute unit: 1 x 16 first (q|k|v: 7.56 us against 7.57 us), then 2 x 8 (gate|up: 10.1 us
//      against 10.5 us), or the chunked shape (below);
//   2. else the chunked shape in one split, when its tables fit;
//   3. else 1 x 16 with the fewest groups per split that keep one round (down: 9.3 us against
//      10.0 us: a tile's 16 parts leave 6 splits instead of 19);
//   4. else the general 4 x 4 shape.
// The LDS check covers both input paths (x staged whole or gathered from memory), so the plan
// does not depend on the pointers.
void plan_shape(const Product* p, int n, int maxL, bool shapes, Plan& P) {
  P.tiles = 4;
  P.cq = 0;
  P.cwm = 0;
  P.stream = false;
  P.gs = plan_gs(p, n, 4);
  if (!shapes) return;
  const int64_t cus = device_cu_count();
  int max_ng = 0, max_din = 0;
  for (int i = 0; i < n; ++i) {
    max_ng = std::max(max_ng, p[i].d_in / kGroupCols);
    max_din = std::max(max_din, p[i].d_in);
  }
  const int whole = max_din <= kWholeXMax ? max_din : 0;
  // LDS of either input path (whether x is staged whole depends on the pointers at launch)
  auto lds_ok = [&](int gs, int T) {
    return std::max(lds_bytes(maxL, gs, whole, T), lds_bytes(maxL, gs, 0, T)) <= 160 * 1024;
  };
  auto fits = [&](int gs, int T) {
    return gs <= shape_max_gs(T) && launch_wgs(p, n, gs, T) <= cus && lds_ok(gs, T);
  };
  bool same_ng = true;
  for (int i = 0; i < n; ++i) same_ng = same_ng && p[i].d_in / kGroupCols == max_ng;
  for (int T : {1, 2}) {
    if (fits(max_ng, T)) {
      P.tiles = T;
      P.gs = max_ng;
      // The chunked shape (one split as well) when the tile shape leaves a SIMD 16 or more
      // half-group steps and the chunks cut that down: gate|up goes from 20 steps on 152 compute
      // units to 13 on 244 (11.3 -> 10.6 us). With fewer steps the extra workgroups cost more
      // than they save: each stages x and builds the tables of every column, and their weight
      // streams delay the input reads (q|k|v: 10 steps on 96 units, 7.3 us; 5 on 192, 7.6 us).
      int q = 0, wm = 0;
      const int c = same_ng && max_ng <= shape_max_gs(0) && lds_ok(max_ng, 0)
                        ? plan_chunks(p, n, 2 * max_ng, q, wm)
                        : -1;
      const int tc = shape_cost(T, 2 * max_ng);
      if (c >= 0 && tc >= 16 && c < tc) {
        P.tiles = 0;
        P.cq = q;
        P.cwm = wm;
      }
      return;
    }
  }
  // No tile shape takes a whole row in one split: the chunked shape still does when its tables
  // fit (up to 32 groups), which saves the split-K hand-off (o: 160 workgroups of one chunk
  // instead of 240 split ones).
  {
    int q = 0, wm = 0;
    if (same_ng && max_ng <= shape_max_gs(0) && lds_ok(max_ng, 0) &&
        plan_chunks(p, n, 2 * max_ng, q, wm) >= 0) {
      P.tiles = 0;
      P.gs = max_ng;
      P.cq = q;
      P.cwm = wm;
      return;
    }
  }
  for (int gs = 1; gs <= shape_max_gs(1); ++gs) {
    if (fits(gs, 1)) {
      P.tiles = 1;
      P.gs = gs;
      return;
    }
  }
  // More rows than one round of workgroups can hold even with splits (an LM-head-sized product):
  // one product gets persistent chunked workgroups (one per compute unit, the tables built once,
  // the next block's weights loading while one decodes) with the most chunks a block can take
  // at two half-group steps per wave (2560-wide rows: 3 chunks, 120 of 128 lane-group steps
  // used; 2 chunks used 80); several products get rounds of the chunked shape with its largest
  // workgroups (8 chunks), no split-K either way.
  if (same_ng && max_ng <= shape_max_gs(0) && lds_ok(max_ng, 0)) {
    ChunkMap M;
    int sq = 0, swm = 0;
    if (n == 1 && p[0].inst == 1) {
      for (int Q = 8; Q >= 2 && sq == 0; --Q) {
        const int nq = Q >> 2, nb = Q & 3;
        const int lo = nb == 0 ? kWaves : nq, hi = nb == 0 ? kWaves : (nq == 0 ? 0 : kWaves - 1);
        for (int wm = hi; wm >= lo && sq == 0; --wm) {
          if (chunk_map(Q, wm, 2 * max_ng, M) < 0) continue;
          int longest = 0;
          for (int w = 0; w < kWaves; ++w) longest = std::max(longest, (int)(M.wave[w] & 255u));
          if (longest <= kStreamSteps) {
            sq = Q;
            swm = wm;
          }
        }
      }
    }
    if (sq > 0) {
      P.tiles = 0;
      P.gs = max_ng;
      P.cq = sq;
      P.cwm = swm;
      P.stream = true;
    } else if (chunk_map(8, kWaves, 2 * max_ng, M) >= 0) {
      P.tiles = 0;
      P.gs = max_ng;
      P.cq = 8;
      P.cwm = kWaves;
    }
  }
}

// Cuts the products into pieces of whole tile blocks (P.tiles row tiles) with similar workgroup
// counts, so the 2-D grid (pieces x workgroups of the widest piece) wastes few workgroups.
void plan_pieces(const Product* p, int n, int maxL, bool shapes, Plan& P) {
  plan_shape(p, n, maxL, shapes, P);
  const bool chunked = P.tiles == 0;
  const int kTiles = chunked ? 1 : P.tiles;
  int S[kMaxJobs], gs[kMaxJobs], rq[kMaxJobs];
  int64_t count[kMaxJobs];
  int64_t smallest = INT64_MAX;
  for (int i = 0; i < n; ++i) {
    const int ng = p[i].d_in / kGroupCols;
    const int g = P.gs < ng ? P.gs : ng;
    S[i] = ceil_div(ng, g);
    gs[i] = ceil_div(ng, S[i]);
    rq[i] = chunked ? ceil_div(ceil_div(p[i].d_out, kChunkRows), P.cq)
                    : ceil_div(ceil_div(p[i].d_out, kTileRows), kTiles);
    count[i] = (int64_t)p[i].inst * rq[i] * S[i];
    if (count[i] < smallest) smallest = count[i];
  }
  int64_t target = smallest;
  int cuts[kMaxJobs];
  for (;;) {
    int total = 0;
    for (int i = 0; i < n; ++i) {
      int64_t c = (count[i] + target - 1) / target;
      if (c > rq[i]) c = rq[i];
      cuts[i] = (int)c;
      total += cuts[i];
    }
    if (total <= kMaxJobs) break;
    target *= 2;
  }
  P.n = 0;
  P.grid_x = 0;
  for (int i = 0; i < n; ++i) {
    const int rt_all = ceil_div(p[i].d_out, kTileRows);
    const int rq_per = ceil_div(rq[i], cuts[i]);
    for (int q0 = 0; q0 < rq[i]; q0 += rq_per) {
      Job& J = P.pieces[P.n];
      J = Job{};
      J.d_out = p[i].d_out;
      J.d_in = p[i].d_in;
      J.ng = p[i].d_in / kGroupCols;
      if (chunked) {
        const int nch = ceil_div(p[i].d_out, kChunkRows);
        J.chunk0 = q0 * P.cq;
        J.nchunk = std::min(nch - J.chunk0, rq_per * P.cq);
        J.rq = ceil_div(J.nchunk, P.cq);
        J.cq = P.cq;
        J.tile0 = 0;
        J.rt = rt_all;
      } else {
        J.tile0 = q0 * kTiles;
        J.rt = rt_all - J.tile0 < rq_per * kTiles ? rt_all - J.tile0 : rq_per * kTiles;
        J.rq = ceil_div(J.rt, kTiles);
      }
      J.S = S[i];
      J.gs = gs[i];
      J.inst = p[i].inst;
      J.wg_per_inst = J.rq * J.S;
      if (P.stream) J.wg_per_inst = (int)std::min<int64_t>(J.rq, device_cu_count());
      J.partial_stride = J.S > 1 ? (int64_t)J.S * J.rt * kTileRows : 0;
      J.counters_stride = J.S > 1 ? J.rq : 0;
      if (J.wg_per_inst * J.inst > P.grid_x) P.grid_x = J.wg_per_inst * J.inst;
      P.src[P.n] = i;
      ++P.n;
    }
  }
}

size_t piece_workspace_bytes(const Job& J) {
  if (J.S == 1) return 0;
  const size_t per = (size_t)J.partial_stride * 4 + (size_t)J.counters_stride * 4;
  return ((size_t)J.inst * per + 255) / 256 * 256;
}

size_t plan_workspace(const Plan& P) {
  size_t need = 0;
  for (int i = 0; i < P.n; ++i) need += piece_workspace_bytes(P.pieces[i]);
  return need;
}

// Kernel variants: shape, whole-x staging, fused stages, and the most half-group steps a wave
// takes (its loads stop there). The chunked shape comes with 3 to 5 steps, 1 x 16 with 1 to 3,
// 2 x 8 and 4 x 4 with their maximum.
typedef void (*GemvFn)(JobTable);
const GemvFn kGemvFns[] = {
    gemv_kernel<0, true, false, 3>,  gemv_kernel<0, true, false, 4>,  gemv_kernel<0, true, false, 5>,
    gemv_kernel<0, false, false, 3>, gemv_kernel<0, false, false, 4>, gemv_kernel<0, false, false, 5>,
    gemv_kernel<1, true, false, 1>,  gemv_kernel<1, true, false, 2>,  gemv_kernel<1, true, false, 3>,
    gemv_kernel<1, false, false, 1>, gemv_kernel<1, false, false, 2>, gemv_kernel<1, false, false, 3>,
    gemv_kernel<2, true, false, 5>,  gemv_kernel<2, false, false, 5>, gemv_kernel<4, true, false, 4>,
    gemv_kernel<4, false, false, 4>, gemv_kernel<4, true, true, 4>,
    gemv_kernel<0, true, false, kStreamSteps, true>, gemv_kernel<0, false, false, kStreamSteps, true>};

GemvFn gemv_fn(int tiles, bool whole, bool fused, int mu, bool stream) {
  if (fused) return tiles == 4 && whole && mu <= 4 ? kGemvFns[16] : nullptr;
  if (stream) return tiles == 0 && mu <= kStreamSteps ? kGemvFns[whole ? 17 : 18] : nullptr;
  const int w = whole ? 0 : 1;
  switch (tiles) {
    case 0: return mu <= 5 ? kGemvFns[w * 3 + std::max(mu, 3) - 3] : nullptr;
    case 1: return mu <= 3 ? kGemvFns[6 + w * 3 + mu - 1] : nullptr;
    case 2: return mu <= 5 ? kGemvFns[12 + w] : nullptr;
    default: return mu <= 4 ? kGemvFns[14 + w] : nullptr;
  }
}

// Fills the piece fields the plan leaves open (matrix, vectors, workspace) and launches.
int launch(Plan& P, const Job* proto, bool whole, int maxL, void* ws, size_t ws_bytes,
           hipStream_t stream) {
  JobTable T{};
  size_t need = 0;
  int gs_max = 1, d_in_max = 0;
  for (int i = 0; i < P.n; ++i) {
    Job& J = T.jobs[i];
    const Job& plan = P.pieces[i];
    const Job& src = proto[P.src[i]];
    J = src;
    J.d_out = plan.d_out;
    J.d_in = plan.d_in;
    J.ng = plan.ng;
    J.tile0 = plan.tile0;
    J.rt = plan.rt;
    J.rq = plan.rq;
    J.cq = plan.cq;
    J.chunk0 = plan.chunk0;
    J.nchunk = plan.nchunk;
    J.S = plan.S;
    J.gs = plan.gs;
    J.inst = plan.inst;
    J.wg_per_inst = plan.wg_per_inst;
    J.partial_stride = plan.partial_stride;
    J.counters_stride = plan.counters_stride;
    const size_t bytes = piece_workspace_bytes(J);
    if (bytes) {
      if (ws == nullptr) return SAGE_ERR_WORKSPACE;
      char* base = static_cast<char*>(ws) + need;
      J.partial = reinterpret_cast<float*>(base);
      J.counters = reinterpret_cast<uint32_t*>(base + (size_t)J.inst * J.partial_stride * 4);
    } else {
      J.partial = nullptr;
      J.counters = nullptr;
    }
    need += bytes;
    if (J.gs > gs_max) gs_max = J.gs;
    if (J.d_in > d_in_max) d_in_max = J.d_in;
  }
  if (need > ws_bytes) return SAGE_ERR_WORKSPACE;
  if (need && !aligned(ws, 256)) return SAGE_ERR_ALIGN;
  if (P.grid_x == 0) return SAGE_OK;
  // fused stages: producers signal once per row group; consumers wait for all of them
  int signals = 0, consumers = 0, first_consumer = -1;
  for (int i = 0; i < P.n; ++i) {
    const Job& J = T.jobs[i];
    if (J.out32 != nullptr) signals += J.rq * J.inst;
    if (J.src_gate != nullptr) {
      consumers += J.wg_per_inst * J.inst;
      if (first_consumer < 0) first_consumer = i;
    }
  }
  for (int i = 0; i < P.n; ++i) {
    Job& J = T.jobs[i];
    J.signal_total = signals;
    J.consumer_wgs = consumers;
    if (i != first_consumer) J.h_out = nullptr;
  }
  if (P.tiles == 0 && chunk_map(P.cq, P.cwm, 2 * T.jobs[0].ng, T.cmap) < 0) return SAGE_ERR_ARG;
  const bool fused = signals > 0;
  if (fused && !whole) return SAGE_ERR_ARG;  // the fused block stages its input whole
  if (fused && P.tiles != 4) return SAGE_ERR_ARG;  // the fused block is built for the 4 x 4 shape
  // half-group steps a wave takes at most in this launch
  int mu = 1;
  if (P.tiles == 0) {
    for (int w = 0; w < kWaves; ++w) mu = std::max(mu, (int)(T.cmap.wave[w] & 255u));
  } else {
    for (int i = 0; i < P.n; ++i) mu = std::max(mu, ceil_div(2 * T.jobs[i].gs, kWaves / P.tiles));
  }
  const GemvFn fn = gemv_fn(P.tiles, whole, fused, mu, P.stream);
  if (fn == nullptr) return SAGE_ERR_ARG;
  static bool attr_done = false;
  if (!attr_done) {
    for (const GemvFn k : kGemvFns)
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
        return SAGE_ERR_HIP;
    attr_done = true;
  }
  const size_t lds = lds_bytes(maxL, gs_max, whole ? d_in_max : 0, P.tiles);
  hipLaunchKernelGGL(fn, dim3((unsigned)P.grid_x, (unsigned)P.n), dim3(kThreads), lds, stream, T);
  return hip_status();
}

// Whole-x staging needs 16-byte aligned inputs no wider than kWholeXMax.
bool whole_x_ok(const uint16_t* x, int64_t x_stride, int d_in) {
  return d_in <= kWholeXMax && aligned(x, 16) && (x_stride % 8) == 0;
}

}  // namespace
}  // namespace sage

using namespace sage;

namespace {

// shapes: whether the launch may use the shapes other than 4 x 4 (the fused SwiGLU launch keeps
// 4 x 4)
int multi_plan(const sage_matrix_t* mats, int n, bool shapes, Plan& P) {
  Product p[kMaxJobs];
  int maxL = 4;
  for (int i = 0; i < n; ++i) {
    p[i] = Product{mats[i].d_out, mats[i].d_in, 1};
    maxL = std::max(maxL, mats[i].log2K);
  }
  plan_pieces(p, n, maxL, shapes, P);
  return SAGE_OK;
}

int moe_plan(const sage_matrix_t* shapes, int n_mats, int n_sel, Plan& P) {
  Product p[kMaxJobs];
  for (int j = 0; j < n_mats; ++j) p[j] = Product{shapes[j].d_out, shapes[j].d_in, n_sel};
  plan_pieces(p, n_mats, 8, true, P);
  return SAGE_OK;
}

}  // namespace

extern "C" {

int sage_gemv_workspace_bytes(const sage_matrix_t* m, size_t* bytes) {
  return sage_gemv_multi_workspace_bytes(m, 1, bytes);
}

int sage_gemv(const sage_matrix_t* m, const uint16_t* x, uint16_t* y, void* ws, size_t ws_bytes,
              sage_stream_t stream) {
  const uint16_t* xs[1] = {x};
  uint16_t* ys[1] = {y};
  return sage_gemv_multi(m, xs, ys, 1, ws, ws_bytes, stream);
}

int sage_gemv_multi_workspace_bytes(const sage_matrix_t* mats, int n, size_t* bytes) {
  if (bytes == nullptr || mats == nullptr) return SAGE_ERR_NULL;
  if (n < 1 || n > kMaxJobs) return SAGE_ERR_ARG;
  for (int i = 0; i < n; ++i) {
    int st = check_matrix(&mats[i]);
    if (st != SAGE_OK) return st;
  }
  Plan P;
  multi_plan(mats, n, true, P);
  *bytes = plan_workspace(P);
  return SAGE_OK;
}

int sage_gemv_multi(const sage_matrix_t* mats, const uint16_t* const* xs, uint16_t* const* ys,
                    int n, void* ws, size_t ws_bytes, sage_stream_t stream) {
  if (mats == nullptr || xs == nullptr || ys == nullptr) return SAGE_ERR_NULL;
  if (n < 1 || n > kMaxJobs) return SAGE_ERR_ARG;
  for (int i = 0; i < n; ++i) {
    int st = check_matrix(&mats[i]);
    if (st != SAGE_OK) return st;
    if (xs[i] == nullptr || ys[i] == nullptr) return SAGE_ERR_NULL;
    if (!aligned(xs[i], 4) || !aligned(ys[i], 2)) return SAGE_ERR_ALIGN;
  }
  Plan P;
  multi_plan(mats, n, true, P);
  Job proto[kMaxJobs];
  int maxL = 4;
  bool whole = true;
  for (int i = 0; i < n; ++i) {
    Job& J = proto[i];
    J = Job{};
    J.packed = static_cast<const uint8_t*>(mats[i].packed);
    J.codebook = mats[i].codebook;
    J.pi = mats[i].pi;
    J.log2K = mats[i].log2K;
    J.x = xs[i];
    J.y = ys[i];
    if (mats[i].log2K > maxL) maxL = mats[i].log2K;
    whole = whole && whole_x_ok(xs[i], 0, mats[i].d_in);
  }
  return launch(P, proto, whole, maxL, ws, ws_bytes, (hipStream_t)stream);
}

static int mlp_check(const sage_matrix_t* gate, const sage_matrix_t* up,
                     const sage_matrix_t* down) {
  if (gate == nullptr || up == nullptr || down == nullptr) return SAGE_ERR_NULL;
  int st = check_matrix(gate);
  if (st == SAGE_OK) st = check_matrix(up);
  if (st == SAGE_OK) st = check_matrix(down);
  if (st != SAGE_OK) return st;
  if (gate->d_out != up->d_out || gate->d_in != up->d_in || down->d_in != gate->d_out)
    return SAGE_ERR_SHAPE;
  if (gate->d_in > kWholeXMax || down->d_in > kWholeXMax) return SAGE_ERR_SHAPE;
  return SAGE_OK;
}

// Workspace of the fused MLP: split-K partials of all pieces, then gate and up rows in fp32,
// then the three synchronisation words.
static size_t mlp_extra_bytes(int inter) { return ((size_t)inter * 8 + 255) / 256 * 256 + 256; }

int sage_mlp_workspace_bytes(const sage_matrix_t* gate, const sage_matrix_t* up,
                             const sage_matrix_t* down, size_t* bytes) {
  if (bytes == nullptr) return SAGE_ERR_NULL;
  int st = mlp_check(gate, up, down);
  if (st != SAGE_OK) return st;
  const sage_matrix_t mats[3] = {*gate, *up, *down};
  Plan P;
  multi_plan(mats, 3, false, P);
  *bytes = plan_workspace(P) + mlp_extra_bytes(gate->d_out);
  return SAGE_OK;
}

int sage_mlp(const sage_matrix_t* gate, const sage_matrix_t* up, const sage_matrix_t* down,
             const uint16_t* x, uint16_t* y, uint16_t* h, void* ws, size_t ws_bytes,
             sage_stream_t stream) {
  int st = mlp_check(gate, up, down);
  if (st != SAGE_OK) return st;
  if (x == nullptr || y == nullptr || ws == nullptr) return SAGE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 2) || !aligned(h, 8) || !aligned(ws, 256))
    return SAGE_ERR_ALIGN;
  const sage_matrix_t mats[3] = {*gate, *up, *down};
  Plan P;
  multi_plan(mats, 3, false, P);
  const size_t parts_bytes = plan_workspace(P);
  if (ws_bytes < parts_bytes + mlp_extra_bytes(gate->d_out)) return SAGE_ERR_WORKSPACE;
  char* extra = static_cast<char*>(ws) + parts_bytes;
  float* g32 = reinterpret_cast<float*>(extra);
  float* u32 = g32 + gate->d_out;
  uint32_t* sync = reinterpret_cast<uint32_t*>(extra + mlp_extra_bytes(gate->d_out) - 256);
  Job proto[3];
  int maxL = 4;
  for (int i = 0; i < 3; ++i) {
    Job& J = proto[i];
    J = Job{};
    J.packed = static_cast<const uint8_t*>(mats[i].packed);
    J.codebook = mats[i].codebook;
    J.pi = mats[i].pi;
    J.log2K = mats[i].log2K;
    J.sync = sync;
    maxL = std::max(maxL, mats[i].log2K);
  }
  proto[0].x = x;
  proto[0].out32 = g32;
  proto[1].x = x;
  proto[1].out32 = u32;
  proto[2].src_gate = g32;
  proto[2].src_up = u32;
  proto[2].y = y;
  proto[2].h_out = h;
  return launch(P, proto, true, maxL, ws, ws_bytes, (hipStream_t)stream);
}

int sage_moe_gemv_workspace_bytes(const sage_matrix_t* shapes, int n_mats, int n_sel,
                                  size_t* bytes) {
  if (bytes == nullptr || shapes == nullptr) return SAGE_ERR_NULL;
  if (n_mats < 1 || n_mats > kMaxJobs || n_sel < 1) return SAGE_ERR_ARG;
  for (int j = 0; j < n_mats; ++j) {
    int st = check_shape(shapes[j].d_out, shapes[j].d_in);
    if (st != SAGE_OK) return st;
  }
  Plan P;
  moe_plan(shapes, n_mats, n_sel, P);
  *bytes = plan_workspace(P);
  return SAGE_OK;
}

int sage_moe_gemv(const sage_matrix_t* experts_dev, int n_experts, const sage_matrix_t* shapes,
                  int n_mats, const int32_t* ids_dev, int n_sel, const uint16_t* const* xs,
                  const int64_t* x_strides, uint16_t* const* ys, const int64_t* y_strides,
                  void* ws, size_t ws_bytes, sage_stream_t stream) {
  if (experts_dev == nullptr || shapes == nullptr || ids_dev == nullptr || xs == nullptr ||
      ys == nullptr || x_strides == nullptr || y_strides == nullptr)
    return SAGE_ERR_NULL;
  if (n_experts < 1 || n_mats < 1 || n_mats > kMaxJobs || n_sel < 1 || n_sel > n_experts)
    return SAGE_ERR_ARG;
  if (!aligned(experts_dev, 8) || !aligned(ids_dev, 4)) return SAGE_ERR_ALIGN;
  for (int j = 0; j < n_mats; ++j) {
    int st = check_shape(shapes[j].d_out, shapes[j].d_in);
    if (st != SAGE_OK) return st;
    if (xs[j] == nullptr || ys[j] == nullptr) return SAGE_ERR_NULL;
    if (!aligned(xs[j], 4) || !aligned(ys[j], 2)) return SAGE_ERR_ALIGN;
    if (x_strides[j] < 0 || (x_strides[j] & 1) || y_strides[j] < 0) return SAGE_ERR_ARG;
    if (n_sel > 1 && y_strides[j] < shapes[j].d_out) return SAGE_ERR_ARG;
  }
  Plan P;
  moe_plan(shapes, n_mats, n_sel, P);
  Job proto[kMaxJobs];
  bool whole = true;
  for (int j = 0; j < n_mats; ++j) {
    Job& J = proto[j];
    J = Job{};
    J.table = experts_dev;
    J.ids = ids_dev;
    J.n_experts = n_experts;
    J.tstride = n_mats;
    J.toff = j;
    J.x = xs[j];
    J.x_stride = x_strides[j];
    J.y = ys[j];
    J.y_stride = y_strides[j];
    whole = whole && whole_x_ok(xs[j], x_strides[j], shapes[j].d_in);
  }
  return launch(P, proto, whole, 8, ws, ws_bytes, (hipStream_t)stream);
}

}  // extern "C"
