// Internal definitions shared by the libsage translation units (not part of the C ABI).
//
// Packed layout (format version 3). Rows are grouped in tiles of 64 (one wavefront lane per row);
// columns in groups of 128 (16 subvectors of 8 weights: the radius-grid group of the SAGE paper,
// §3.1 / App. A.6). Each (row tile, column group) block is 2560 bytes and blocks are stored
// row-tile major: block(rt, g) at byte (rt * n_groups + g) * 2560. Inside a block:
//
//   bytes [   0, 1024)  plane A: lane l owns 16 bytes = payload dwords P0..P3 of row 64 rt + l
//   bytes [1024, 2048)  plane B: lane l owns 16 bytes = payload dwords P4..P7
//   bytes [2048, 2560)  side plane: lane l owns 8 bytes = dword X, then dword G = mu | delta << 16
//
// With L = log2(K), V = 10 - L, and for subvector j of the group its sign byte s_j (bit i <=>
// weight i negative), codeword index z_j and radius code q_j, payload dword P_i (i = 0..7) carries
// the pair a = 2i, b = 2i + 1:
//
//   bits [0, 3)        s_b bits 5..7          bits [17, 17+L)    z_b
//   bits [3, 3+L)      z_a                    bits [17+L, 21+L)  s_b bits 0..3
//   bits [3+L, 7+L)    s_a bits 0..3          bits [21+L, 31)    q_b
//   bits [7+L, 17)     q_a                    bit  31            s_b bit 4
//
// and X carries s_{2i} bits 4..7 at bits [4i, 4i+4). Every subvector costs 8 + L + V = 18 bits
// (§3.1 Eq. (3)) and every group 4 more bytes of fp16 grid: 2.5 bits per weight. The positions
// serve the batch-one decoder, whose LDS table of sign-applied codeword halves is indexed by
// (z | s_half << L) * 8 bytes: P & mask gives subvector a's first-half table address, the
// rotation of P by 14 brings b's index, sign nibble and radius code to a's positions, rotating P
// left by 4 + L brings b's second sign nibble (bits 31, 0, 1, 2) next to its index, and q sits at
// bits [7+L, 17) of P or of the rotated P, where OR-ing an exponent turns it into the float
// 2^(16-L) + q. Rows past d_out in the last tile are zero.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "../../include/sage.h"

namespace sage {

constexpr int kFormatVersion = 3;
constexpr int kTileRows = 64;                  // rows per tile = lanes per wavefront
constexpr int kGroupCols = 128;                // weights per radius-grid group
constexpr int kSubPerGroup = 16;               // subvectors per group
constexpr int kBlockBytes = 2560;              // 64 rows x 128 cols x 2.5 bits
constexpr int kPlaneA = 0;
constexpr int kPlaneB = 1024;
constexpr int kSidePlane = 2048;

// Payload dword of the pair (a, b) (format version 3). Field values must be in range.
__host__ __device__ inline uint32_t v3_pair(uint32_t sa, uint32_t za, uint32_t qa, uint32_t sb,
                                            uint32_t zb, uint32_t qb, int L) {
  return (sb >> 5) | (za << 3) | ((sa & 15u) << (3 + L)) | (qa << (7 + L)) | (zb << 17) |
         ((sb & 15u) << (17 + L)) | (qb << (21 + L)) | (((sb >> 4) & 1u) << 31);
}

// Fields of subvector j (0..15) of a group from its payload dwords P[0..7] and X.
__host__ __device__ inline void v3_fields(const uint32_t P[8], uint32_t X, int j, int L,
                                          uint32_t* s, uint32_t* z, uint32_t* q) {
  const uint32_t w = P[j >> 1];
  const uint32_t kmask = (1u << L) - 1u, vmask = (1u << (10 - L)) - 1u;
  if ((j & 1) == 0) {
    *z = (w >> 3) & kmask;
    *q = (w >> (7 + L)) & vmask;
    *s = ((w >> (3 + L)) & 15u) | (((X >> (4 * (j >> 1))) & 15u) << 4);
  } else {
    *z = (w >> 17) & kmask;
    *q = (w >> (21 + L)) & vmask;
    *s = ((w >> (17 + L)) & 15u) | ((w >> 31) << 4) | ((w & 7u) << 5);
  }
}

// The 8 payload dwords, X and G of one lane of a block.
__device__ inline void read_lane_block(const uint8_t* blk, int lane, uint32_t p[8], uint32_t* x,
                                       uint32_t* grid) {
  const uint4 a = *reinterpret_cast<const uint4*>(blk + kPlaneA + lane * 16);
  const uint4 b = *reinterpret_cast<const uint4*>(blk + kPlaneB + lane * 16);
  const uint2 s = *reinterpret_cast<const uint2*>(blk + kSidePlane + lane * 8);
  p[0] = a.x; p[1] = a.y; p[2] = a.z; p[3] = a.w;
  p[4] = b.x; p[5] = b.y; p[6] = b.z; p[7] = b.w;
  *x = s.x;
  *grid = s.y;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int check_split(int log2K, int V) {
  if (log2K < 4 || log2K > 8 || log2K + V != 10) return SAGE_ERR_SPLIT;
  return SAGE_OK;
}

inline int check_shape(int d_out, int d_in) {
  if (d_out < 1 || d_in < kGroupCols || d_in % kGroupCols != 0) return SAGE_ERR_SHAPE;
  // keep every byte offset inside 63 bits and every row index inside int32
  if ((int64_t)d_out * (int64_t)d_in > ((int64_t)1 << 40)) return SAGE_ERR_SHAPE;
  return SAGE_OK;
}

inline size_t packed_bytes(int d_out, int d_in) {
  return (size_t)ceil_div(d_out, kTileRows) * (size_t)(d_in / kGroupCols) * kBlockBytes;
}

int check_matrix(const sage_matrix_t* m);   // shape, split, pointers, alignment
int hip_status();                            // SAGE_ERR_HIP if the last launch failed
int device_cu_count();                       // compute units of the current device (cached)

// Range-checked buffer view: loads at offsets past `bytes` return zeros without a memory access.
__device__ inline __amdgpu_buffer_rsrc_t view(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
constexpr uint32_t kNowhere = 1u << 30;  // an offset past every range
constexpr int kNonTemporal = 2;          // streamed once: no reuse expected in the caches

// Global-memory view of a device pointer. Pointers read from memory (descriptor tables) are
// generic, and loads through them compile to flat instructions, which count against both the
// vector-memory and the LDS wait counters: every LDS wait would then also wait for the HBM stream.
// Loads through this view are global loads, counted by vmcnt alone.
template <typename T>
__device__ inline const __attribute__((address_space(1))) T* gview(const T* p) {
  return (const __attribute__((address_space(1))) T*)(p);
}

// Cross-workgroup hand-off of split-K partials without cache-wide fences. Partials are written with
// agent-scope relaxed atomic stores (coherent stores, sc1) and read back the same way; each wave
// waits for its stores to be acknowledged before the workgroup barrier that precedes the counter
// increment, so a workgroup that sees the final count also sees every partial.
__device__ inline void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Coherent (sc1) loads through a buffer descriptor: unlike atomic loads they can be batched.
__device__ inline __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ inline float load_coherent_at(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0x10 /* sc1 */));
}
__device__ inline uint32_t load_coherent_u32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t counter_add(uint32_t* c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void counter_reset(uint32_t* c) {
  __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fp16 <-> fp32 on bit patterns; the float -> half conversion rounds to nearest even.
__device__ inline float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}
__device__ inline uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// fp64 -> fp16 with a single round-to-nearest-even: round to fp32 "to odd" first (exact when the
// fp32 rounding was exact), then RNE to fp16. Rounding to odd with >= 2 extra bits of precision
// makes the second rounding equal to a direct correct rounding.
__device__ inline uint16_t f64_to_f16_rne(double d) {
  float f = (float)d;
  if ((double)f != d) {
    uint32_t u = __float_as_uint(f);
    if ((u & 1u) == 0u) u += (fabs((double)f) < fabs(d)) ? 1u : 0xFFFFFFFFu;
    f = __uint_as_float(u);
  }
  return f2h(f);
}

}  // namespace sage
