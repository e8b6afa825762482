// Batch-one decode-and-multiply for SAGE-packed weights on gfx950 (SAGE paper §3.5 and App. A.1).
//
// Work decomposition. Lane l of a wavefront owns output row 64*rt + l of one row tile; the four
// wavefronts of a workgroup own four consecutive row tiles and share one range of column groups
// (split-K over workgroups when the matrix alone does not fill the GPU, App. A.1 / §3.5). Because
// every lane of a wave works on the same input columns at the same time, the activations are
// uniform across the wave and no cross-lane reduction is needed.
//
// Per workgroup set-up, in LDS:
//   * the codebook, replicated 16 times with replica r at byte offset 16 r of each 256-byte row,
//     so lane l reads replica (l mod 16): random codeword gathers become bank-conflict free;
//   * the permuted activations x[pi[p]] of the workgroup's columns (gathered once, §3.2/§3.5);
//   * for every subvector position, a table of the 16 sign patterns of each 4-wide activation
//     half: entry n holds (x0..x3) and (x4..x7) with element i negated when bit i of n is set.
// A subvector is then: two conflict-free 8-byte table reads selected by the low and high sign
// nibbles, one 16-byte codeword read, four fp16 dot2 steps with fp32 accumulation, and the radius
// mu + q*delta applied once to the 8-term dot product (App. A.1 applies the radius after the dot
// for the same reason: one multiply instead of eight).
//
// Split-K partials go to a caller workspace (coherent stores, no cache-wide fences); the last
// workgroup of a row-tile group (atomic counter) sums them in split order, writes y in fp16 and
// resets the counter to zero.
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
constexpr int kNonTemporal = 2;  // streamed once: no reuse expected in the caches

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
// ((a >> 8) & m) in one VALU op (SDWA byte select; the compiler only forms the 16/24-bit cases).
__device__ inline uint32_t and_byte1(uint32_t a, uint32_t m) {
  uint32_t r;
  asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 "
      "src1_sel:DWORD"
      : "=v"(r)
      : "v"(a), "s"(m));
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
  // LDS: codebook replicas and signed-activation tables at compile-time offsets, so that every
  // table offset folds into the ds_read immediate. K = 256 needs the tables first.
  static constexpr int kCbOff = (L == 8) ? 32768 : 0;
  static constexpr int kXtOff = (L == 8) ? 0 : (int)(kK * 256);
};

struct Resolved {
  const uint8_t* packed;
  const uint16_t* codebook;
  const int32_t* pi;
  int L;
};

template <int L>
__device__ inline int xp_offset(int gs) {
  return (L == 8) ? 32768 + 65536 : SplitC<L>::kXtOff + gs * kSubPerGroup * 256;
}

struct GroupRegs {
  uint32_t p[8];
  uint32_t x, g;
};

// One group of one lane: main words of subvectors 0-7 and 8-15, then aux fields and the grid.
__device__ inline void load_group(GroupRegs& r, __amdgpu_buffer_rsrc_t rs, uint32_t blk_off,
                                  int lane) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, blk_off + kPlaneA + lane * 16, 0, kNonTemporal);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, blk_off + kPlaneB + lane * 16, 0, kNonTemporal);
  const u32x2 s = __builtin_amdgcn_raw_buffer_load_b64(rs, blk_off + kSidePlane + lane * 8, 0, kNonTemporal);
  r.p[0] = a[0]; r.p[1] = a[1]; r.p[2] = a[2]; r.p[3] = a[3];
  r.p[4] = b[0]; r.p[5] = b[1]; r.p[6] = b[2]; r.p[7] = b[3];
  r.x = s[0];
  r.g = s[1];
}

// LDS reads at absolute LDS byte addresses. The kernel declares no static LDS, so its dynamic LDS
// starts at address 0 and table offsets become ds_read immediates.
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
template <int L>
__device__ __forceinline__ float subvec(int xt_off, uint32_t lo, uint32_t hi, uint32_t cz,
                                        uint32_t qbits, float dl, float mu_b, float acc) {
  const uint2 x0 = lds8(lo + (uint32_t)xt_off);
  const uint2 x1 = lds8(hi + (uint32_t)(xt_off + 8));
  const uint4 c = lds16(cz + (uint32_t)SplitC<L>::kCbOff);
  float t = dot2_z(c.x, x0.x);
  t = dot2(c.y, x0.y, t);
  t = dot2(c.z, x1.x, t);
  t = dot2(c.w, x1.y, t);
  const float r = fmaf(__uint_as_float(qbits), dl, mu_b);
  return fmaf(r, t, acc);
}

// All 16 subvectors of one group; k is the group's slot in this workgroup (compile-time).
template <int L, int k>
__device__ __forceinline__ float group_dot(const GroupRegs& R, uint32_t laneoff, uint32_t expo,
                                           float acc) {
  using C = SplitC<L>;
  const float mu = h2f(R.g);
  const float dl = h2f(R.g >> 16);
  const float mu_b = fmaf(-C::kBias, dl, mu);  // radius = (2^(15-L) + q) * delta + mu_b
  const uint32_t x4 = R.x << 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t P = R.p[i];
    const int off_a = C::kXtOff + k * kSubPerGroup * 256 + (2 * i) * 256;
    // subvector a = 2i: nibbles at bits 4..7 and 28..31, field at bit 8
    acc = subvec<L>(off_a, P & 0xF0u, (P >> 24) & 0xF0u, and_or(P, C::kZMask, laneoff),
                    and_or(P, C::kQMask, expo), dl, mu_b, acc);
    // subvector b = 2i+1: nibble at bits 0..3 of P and slot i of X, field at bit 18
    uint32_t hi_b;
    if (i & 1) {
      const int byte = (i - 1) >> 1;
      hi_b = byte == 0 ? (R.x & 0xF0u)
           : byte == 1 ? and_byte1(R.x, 0xF0u)
           : byte == 2 ? ((R.x >> 16) & 0xF0u) : ((R.x >> 24) & 0xF0u);
    } else {
      const int byte = i >> 1;
      hi_b = byte == 0 ? (x4 & 0xF0u)
           : byte == 1 ? and_byte1(x4, 0xF0u)
           : byte == 2 ? ((x4 >> 16) & 0xF0u) : ((x4 >> 24) & 0xF0u);
    }
    const uint32_t Pb = P >> 10;
    acc = subvec<L>(off_a + 256, (P << 4) & 0xF0u, hi_b, and_or(Pb, C::kZMask, laneoff),
                    and_or(Pb, C::kQMask, expo), dl, mu_b, acc);
  }
  return acc;
}

template <int L, int W, bool kWholeX>
__device__ __forceinline__ void gemv_body(const Resolved& R, const Job& J, int inst, int wgrow,
                                          int split, uint8_t* smem) {
  constexpr int kThreads = W * 64;
  using C = SplitC<L>;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: addresses in SGPRs
  const int lane = tid & 63;
  const int g0 = split * J.gs;
  const int ngl = min(J.ng - g0, J.gs);
  const int rt = wgrow * W + wave;
  const bool tile_ok = rt < J.rt;

  // 1. Loads, in the order their data is needed. Every load is unconditional: a range-checked
  //    view returns zeros past the split's last group (or for a wave past the last row tile), so
  //    the wait before each use covers exactly the loads issued before it.
  constexpr int kColsPerThread = kMaxGroupsPerSplit * kGroupCols / kThreads;
  const int c0 = g0 * kGroupCols;
  const int cols = ngl * kGroupCols;
  const __amdgpu_buffer_rsrc_t cb_rs = view(R.codebook, C::kK * 16u);
  const __amdgpu_buffer_rsrc_t pi_rs = view(R.pi ? R.pi + c0 : nullptr, R.pi ? cols * 4u : 0u);
  const __amdgpu_buffer_rsrc_t x_rs =
      view(J.x + (int64_t)inst * J.x_stride, (uint32_t)J.d_in * 2u);
  const uint8_t* blk0 = R.packed + ((int64_t)rt * J.ng + g0) * kBlockBytes;
  const __amdgpu_buffer_rsrc_t w_rs = view(blk0, tile_ok ? (uint32_t)(ngl * kBlockBytes) : 0u);

  const u32x4 cw = __builtin_amdgcn_raw_buffer_load_b128(cb_rs, tid * 16, 0, 0);
  uint32_t src[kColsPerThread];
#pragma unroll
  for (int i = 0; i < kColsPerThread; ++i)
    src[i] = __builtin_amdgcn_raw_buffer_load_b32(pi_rs, (tid + i * kThreads) * 4, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t last = (uint32_t)J.d_in - 1u;  // an out-of-range pi entry is clamped
  // identity when pi is absent, as a lane mask rather than a branch
  uint32_t use_pi = R.pi ? ~0u : 0u;
  asm volatile("" : "+v"(use_pi));
  uint16_t* xp = reinterpret_cast<uint16_t*>(smem + xp_offset<L>(J.gs));
  GroupRegs g[kMaxGroupsPerSplit];
  if constexpr (kWholeX) {
    // The whole activation vector is staged in LDS next to pi, so the gather x[pi[p]] is an LDS
    // read instead of a second dependent trip to memory.
    constexpr int kChunks = kWholeXMax / 8 / kThreads;  // 16-byte chunks per thread
    u32x4 xc[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      xc[i] = __builtin_amdgcn_raw_buffer_load_b128(x_rs, (tid + i * kThreads) * 16, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep the issue order: the counters wait in order
#pragma unroll
    for (int k = 0; k < kMaxGroupsPerSplit; ++k) load_group(g[k], w_rs, k * kBlockBytes, lane);
    __builtin_amdgcn_sched_barrier(0);
    uint16_t* xw = xp + kMaxGroupsPerSplit * kGroupCols;  // whole x after the gathered columns
    const int nchunks = J.d_in / 8;
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      if (tid + i * kThreads < nchunks)
        *reinterpret_cast<u32x4*>(xw + (tid + i * kThreads) * 8) = xc[i];
    if (tid < (int)C::kK) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        *reinterpret_cast<u32x4*>(smem + C::kCbOff + tid * 256 + r * 16) = cw;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kColsPerThread; ++i) {
      const int p = tid + i * kThreads;
      const uint32_t col = (min(src[i], last) & use_pi) | ((uint32_t)(c0 + p) & ~use_pi);
      if (p < cols) xp[p] = xw[col];
    }
  } else {
    // Wide inputs: pi first, then the gathered activations straight from memory.
#pragma unroll
    for (int k = 0; k < kMaxGroupsPerSplit / 2; ++k) load_group(g[k], w_rs, k * kBlockBytes, lane);
    __builtin_amdgcn_sched_barrier(0);
    uint16_t xv[kColsPerThread];
#pragma unroll
    for (int i = 0; i < kColsPerThread; ++i) {
      const uint32_t ident = (uint32_t)(c0 + tid + i * kThreads);
      const uint32_t col = (min(src[i], last) & use_pi) | (ident & ~use_pi);
      xv[i] = __builtin_amdgcn_raw_buffer_load_b16(x_rs, col * 2u, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = kMaxGroupsPerSplit / 2; k < kMaxGroupsPerSplit; ++k)
      load_group(g[k], w_rs, k * kBlockBytes, lane);
    __builtin_amdgcn_sched_barrier(0);
    if (tid < (int)C::kK) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        *reinterpret_cast<u32x4*>(smem + C::kCbOff + tid * 256 + r * 16) = cw;
    }
#pragma unroll
    for (int i = 0; i < kColsPerThread; ++i)
      if (tid + i * kThreads < cols) xp[tid + i * kThreads] = xv[i];
  }
  __syncthreads();
  // 2. Signed-activation tables of the workgroup's columns.
  for (int e = tid; e < ngl * kSubPerGroup * 16; e += kThreads) {
    const int step = e >> 4;
    const uint32_t n = (uint32_t)(e & 15);
    const uint4 v = *reinterpret_cast<const uint4*>(xp + step * 8);
    const uint2 lo = apply_nibble(v.x, v.y, n);
    const uint2 hi = apply_nibble(v.z, v.w, n);
    *reinterpret_cast<uint4*>(smem + C::kXtOff + step * 256 + n * 16) =
        make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  __syncthreads();

  // 3. Decode and multiply.
  float acc = 0.0f;
  const uint32_t laneoff = (uint32_t)(lane & 15) * 16u;
  const uint32_t expo = C::kExpo;
#define SAGE_GROUP(k) \
  if (k < ngl) acc = group_dot<L, k>(g[k], laneoff, expo, acc);
  SAGE_GROUP(0) SAGE_GROUP(1) SAGE_GROUP(2) SAGE_GROUP(3)
  SAGE_GROUP(4) SAGE_GROUP(5) SAGE_GROUP(6) SAGE_GROUP(7)
#undef SAGE_GROUP

  // 4. Output: direct, or split-K partials reduced by the last workgroup of the row-tile group.
  const int row = rt * kTileRows + lane;
  const bool row_ok = tile_ok && row < J.d_out;
  uint16_t* y = J.y + (int64_t)inst * J.y_stride;
  if (J.S == 1) {
    if (row_ok) y[row] = f2h(acc);
    return;
  }
  float* part = J.partial + (int64_t)inst * J.partial_stride;
  const int64_t rows_pad = (int64_t)J.rt * kTileRows;
  if (row_ok) store_coherent(part + (int64_t)split * rows_pad + row, acc);
  wait_stores();
  __syncthreads();
  uint32_t* flag = reinterpret_cast<uint32_t*>(smem);  // LDS no longer needed
  uint32_t* counter = J.counters + (int64_t)inst * J.counters_stride + wgrow;
  if (tid == 0) *flag = (counter_add(counter) == (uint32_t)(J.S - 1)) ? 1u : 0u;
  __syncthreads();
  if (*flag == 0u) return;
  if (row_ok) {
    // all partials of this row issued back to back, summed in split order
    const __amdgpu_buffer_rsrc_t rs =
        coherent_rsrc(part, (uint32_t)(J.S * rows_pad * (int64_t)sizeof(float)));
    float s = 0.0f;
#pragma unroll 16
    for (int sp = 0; sp < J.S; ++sp)
      s += load_coherent_at(rs, (uint32_t)((sp * rows_pad + row) * sizeof(float)));
    y[row] = f2h(s);
  }
  if (tid == 0) counter_reset(counter);
}

template <bool kWholeX>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 8)))
gemv_kernel(JobTable T) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int wg = blockIdx.x;
  int jid = 0;
#pragma unroll
  for (int i = 1; i < kMaxJobs; ++i) jid += (wg >= T.wg_begin[i]) ? 1 : 0;
  const Job& J = T.jobs[jid];
  int local = wg - J.wg_begin;
  const int inst = local / J.wg_per_inst;
  local -= inst * J.wg_per_inst;
  const int wgrow = local / J.S;
  const int split = local - wgrow * J.S;
  Resolved R;
  if (J.table != nullptr) {
    const uint32_t e = min((uint32_t)J.ids[inst], (uint32_t)J.n_experts - 1u);
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
    case 4: gemv_body<4, kWaves, kWholeX>(R, J, inst, wgrow, split, smem); break;
    case 5: gemv_body<5, kWaves, kWholeX>(R, J, inst, wgrow, split, smem); break;
    case 6: gemv_body<6, kWaves, kWholeX>(R, J, inst, wgrow, split, smem); break;
    case 7: gemv_body<7, kWaves, kWholeX>(R, J, inst, wgrow, split, smem); break;
    default: gemv_body<8, kWaves, kWholeX>(R, J, inst, wgrow, split, smem); break;
  }
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// Host planning

size_t lds_bytes(int maxL, int gs, int whole_d_in) {
  // the largest layout among the splits a launch may meet (see SplitC / xp_offset): codebook
  // replicas and tables, the gathered columns (room for the largest split), then whole x if staged
  size_t need = 0;
  for (int L = 4; L <= maxL; ++L) {
    const size_t b = (L == 8) ? (size_t)32768 + 65536
                              : ((size_t)1 << L) * 256 + (size_t)gs * kSubPerGroup * 256;
    if (b > need) need = b;
  }
  need += (size_t)kMaxGroupsPerSplit * kGroupCols * 2 + (size_t)whole_d_in * 2;
  return need;
}

// Launch plan shared by every job of one launch: column groups per split.
struct LaunchPlan {
  int gs;
};

LaunchPlan plan_launch(int64_t total_blocks) {
  // Four row tiles per workgroup, so two workgroups fit a compute unit at once and every launch
  // runs in a single round; groups per split grow until the launch would drop below one
  // workgroup per compute unit (more groups per split = fewer split-K partials to combine).
  const int64_t target = (int64_t)device_cu_count();
  for (int gs = kMaxGroupsPerSplit; gs > 1; --gs) {
    const int64_t wgs = (total_blocks + kWaves * gs - 1) / (kWaves * gs);
    if (wgs >= target) return LaunchPlan{gs};
  }
  return LaunchPlan{1};
}

void plan_job(Job& J, int d_out, int d_in, const LaunchPlan& P, int instances) {
  J.d_out = d_out;
  J.d_in = d_in;
  J.rt = ceil_div(d_out, kTileRows);
  J.ng = d_in / kGroupCols;
  J.wgr = ceil_div(J.rt, kWaves);
  J.gs = P.gs < J.ng ? P.gs : J.ng;
  J.S = ceil_div(J.ng, J.gs);
  J.gs = ceil_div(J.ng, J.S);
  J.wg_per_inst = J.wgr * J.S;
  J.inst = instances;
  J.partial_stride = J.S > 1 ? (int64_t)J.S * J.rt * kTileRows : 0;
  J.counters_stride = J.S > 1 ? J.wgr : 0;
}

size_t job_workspace_bytes(const Job& J) {
  if (J.S == 1) return 0;
  const size_t per = (size_t)J.partial_stride * 4 + (size_t)J.counters_stride * 4;
  return ((size_t)J.inst * per + 255) / 256 * 256;
}

int finish_and_launch(JobTable& T, void* ws, size_t ws_bytes, hipStream_t stream, int maxL) {
  size_t need = 0;
  int wg = 0;
  size_t lds = 0;
  // whole-x staging when every input of the launch fits
  bool whole = true;
  for (int i = 0; i < T.n; ++i) whole = whole && T.jobs[i].d_in <= kWholeXMax;
  for (int i = 0; i < T.n; ++i) {
    Job& J = T.jobs[i];
    const size_t bytes = job_workspace_bytes(J);
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
    J.wg_begin = wg;
    T.wg_begin[i] = wg;
    wg += J.wg_per_inst * J.inst;
    const size_t l = lds_bytes(maxL, J.gs, whole ? J.d_in : 0);
    if (l > lds) lds = l;
  }
  for (int i = T.n; i < kMaxJobs; ++i) T.wg_begin[i] = 0x7FFFFFFF;
  if (need > ws_bytes) return SAGE_ERR_WORKSPACE;
  if (need && !aligned(ws, 256)) return SAGE_ERR_ALIGN;
  T.total_wg = wg;
  if (wg == 0) return SAGE_OK;
  static bool attr_done = false;
  if (!attr_done) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return SAGE_ERR_HIP;
    attr_done = true;
  }
  if (whole)
    hipLaunchKernelGGL(gemv_kernel<true>, dim3(wg), dim3(kWaves * 64), lds, stream, T);
  else
    hipLaunchKernelGGL(gemv_kernel<false>, dim3(wg), dim3(kWaves * 64), lds, stream, T);
  return hip_status();
}

size_t plan_workspace(const Job* jobs, int n) {
  size_t need = 0;
  for (int i = 0; i < n; ++i) need += job_workspace_bytes(jobs[i]);
  return need;
}

}  // namespace sage

using namespace sage;

namespace {

void direct_job(Job& J, const sage_matrix_t* m, const LaunchPlan& P) {
  J = Job{};
  J.packed = static_cast<const uint8_t*>(m->packed);
  J.codebook = m->codebook;
  J.pi = m->pi;
  J.log2K = m->log2K;
  plan_job(J, m->d_out, m->d_in, P, 1);
}

LaunchPlan plan_for(const sage_matrix_t* mats, int n, int instances = 1) {
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i)
    blocks += (int64_t)instances * ceil_div(mats[i].d_out, kTileRows) * (mats[i].d_in / kGroupCols);
  return plan_launch(blocks);
}

}  // namespace

extern "C" {

int sage_gemv_workspace_bytes(const sage_matrix_t* m, size_t* bytes) {
  if (bytes == nullptr) return SAGE_ERR_NULL;
  int st = check_matrix(m);
  if (st != SAGE_OK) return st;
  Job J;
  direct_job(J, m, plan_for(m, 1));
  *bytes = job_workspace_bytes(J);
  return SAGE_OK;
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
  const LaunchPlan P = plan_for(mats, n);
  size_t need = 0;
  for (int i = 0; i < n; ++i) {
    Job J;
    direct_job(J, &mats[i], P);
    need += job_workspace_bytes(J);
  }
  *bytes = need;
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
  JobTable T{};
  T.n = n;
  const LaunchPlan P = plan_for(mats, n);
  int maxL = 4;
  for (int i = 0; i < n; ++i) {
    direct_job(T.jobs[i], &mats[i], P);
    T.jobs[i].x = xs[i];
    T.jobs[i].y = ys[i];
    if (mats[i].log2K > maxL) maxL = mats[i].log2K;
  }
  return finish_and_launch(T, ws, ws_bytes, (hipStream_t)stream, maxL);
}

int sage_moe_gemv_workspace_bytes(const sage_matrix_t* shapes, int n_mats, int n_sel,
                                  size_t* bytes) {
  if (bytes == nullptr || shapes == nullptr) return SAGE_ERR_NULL;
  if (n_mats < 1 || n_mats > kMaxJobs || n_sel < 1) return SAGE_ERR_ARG;
  for (int j = 0; j < n_mats; ++j) {
    int st = check_shape(shapes[j].d_out, shapes[j].d_in);
    if (st != SAGE_OK) return st;
  }
  const LaunchPlan P = plan_for(shapes, n_mats, n_sel);
  size_t need = 0;
  for (int j = 0; j < n_mats; ++j) {
    Job J{};
    plan_job(J, shapes[j].d_out, shapes[j].d_in, P, n_sel);
    need += job_workspace_bytes(J);
  }
  *bytes = need;
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
  const LaunchPlan P = plan_for(shapes, n_mats, n_sel);
  JobTable T{};
  T.n = n_mats;
  for (int j = 0; j < n_mats; ++j) {
    Job& J = T.jobs[j];
    J = Job{};
    J.table = experts_dev;
    J.ids = ids_dev;
    J.n_experts = n_experts;
    J.tstride = n_mats;
    J.toff = j;
    plan_job(J, shapes[j].d_out, shapes[j].d_in, P, n_sel);
    J.x = xs[j];
    J.x_stride = x_strides[j];
    J.y = ys[j];
    J.y_stride = y_strides[j];
  }
  return finish_and_launch(T, ws, ws_bytes, (hipStream_t)stream, 8);
}

}  // extern "C"
