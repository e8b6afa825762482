// Batch-one decode-and-multiply for SAGE-packed weights on gfx950 (SAGE paper §3.5 and App. A.1):
// y = W_hat x with W_hat decoded on the fly from its 18-bit subvector codes (§3.1 Eq. (1)-(3)).
//
// Work decomposition. Rows are taken in chunks of 16 (a quarter of a packed row tile). A workgroup
// of 1024 threads (16 wavefronts, one workgroup per compute unit) owns whole rows: a run of chunks
// of one product, so no partial sum ever leaves the compute unit (no split-K hand-off between
// workgroups). Its 64 lane groups of 16 lanes split the workgroup's (chunk, half-group) units into
// contiguous, equally long ranges in chunk-major order; lane l of a group owns row l of the chunk
// it is working on. A range crosses at most one chunk boundary, so a lane keeps two sums. At the
// end the lane groups that worked on a chunk add their sums in LDS in lane-group order (a fixed
// order: results are reproducible bit for bit) and one rounding to fp16 gives y.
//
// Decode. The workgroup builds, once, a table of sign-applied codeword halves in LDS:
// T[h][s][z] (h = first or second half of the 8-wide codeword, s = 4 sign bits, z = codeword) holds
// the four fp16 values c_z[4h..4h+3] with element i negated when bit i of s is set. The table
// depends only on the codebook (256 K bytes), not on the input, so nothing is rebuilt per input
// position. A subvector then costs two 8-byte table reads, addressed straight from bit fields of
// the packed word (the packed layout puts z and each sign nibble next to each other), four fp16
// dot2 steps with fp32 accumulation against the input, and the radius mu + q*delta applied once
// to the 8-term dot product (App. A.1: one multiply instead of eight). The input is staged in LDS
// in stored (permuted) column order: copied as is when the matrix's pi is NULL (the producer wrote
// it permuted, §3.5 compiled decoding), else gathered through pi once per workgroup (§3.5 eager
// decoding: the gather fused into the product).
//
// Memory access. Every global load is a buffer load through a range-checked view: loads past the
// range return zeros without a memory access, so loads are issued unconditionally (units a lane
// group does not own decode as zeros: their grid is zero, so they add exactly 0). The codebook and
// input loads go out first, then the packed units of every lane group; four units per lane group
// stay in flight while it decodes.
#include <algorithm>
#include <mutex>
#include <vector>

#include "sage_internal.hpp"

namespace sage {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 1024;
constexpr int kLaneGroups = 64;
constexpr int kChunkRows = 16;
constexpr int kMaxChunks = 64;     // chunks per workgroup (a lane-group range stays within 2)
constexpr int kRing = 4;           // half-group units in flight per lane group
constexpr int kMaxProducts = 16;
constexpr int kMaxWgs = 768;
constexpr int kMaxDin = 32768;     // widest input staged whole in LDS (stored order)
constexpr int kXIter = kMaxDin / 8 / kThreads;   // 8-wide input pieces per thread, at most
constexpr uint32_t kMaxLds = 160u * 1024u;
constexpr uint32_t kPartBytes = 2 * kLaneGroups * kChunkRows * 4;

// LDS layout of a workgroup: T [256 K bytes], then the input in stored order [2 d_in bytes, whole
// KiB], then (gathering only) the input in original order [as many] and pi [4 d_in bytes, whole
// KiB], then the lane-group sums. A launch fits when the total is at most 160 KiB.
__host__ __device__ inline uint32_t x_bytes(int d_in) { return (2u * (uint32_t)d_in + 1023u) & ~1023u; }
__host__ __device__ inline uint32_t lds_x(int L) { return 256u << L; }
__host__ __device__ inline uint32_t lds_xs(int L, int d_in) { return lds_x(L) + x_bytes(d_in); }
__host__ __device__ inline uint32_t pi_bytes(int d_in) { return (4u * (uint32_t)d_in + 1023u) & ~1023u; }
__host__ __device__ inline uint32_t lds_pi(int L, int d_in) { return lds_xs(L, d_in) + x_bytes(d_in); }
__host__ __device__ inline uint32_t lds_part(int L, int d_in, bool gather) {
  return gather ? lds_pi(L, d_in) + pi_bytes(d_in) : lds_x(L) + x_bytes(d_in);
}
__host__ __device__ inline uint32_t lds_total(int L, int d_in, bool gather) {
  return lds_part(L, d_in, gather) + kPartBytes;
}

// One product of a launch.
struct Prod {
  const uint8_t* packed;
  const uint16_t* codebook;
  const int32_t* pi;
  const uint16_t* x;
  uint16_t* y;
  int32_t d_out, d_in, L, pad;
};

// Kernel argument of a planned launch: per workgroup, product (bits 0-3), chunks - 1 (bits 4-9)
// and first chunk (bits 10-31).
struct GemvArgs {
  Prod prod[kMaxProducts];
  uint32_t wg[kMaxWgs];
};
static_assert(sizeof(GemvArgs) <= 4096, "kernel argument block too large");

// Kernel argument of a routed-expert launch (descriptors read on the device).
constexpr int kMaxMats = 4;
struct MoeArgs {
  const sage_matrix_t* experts;   // [n_experts * n_mats]
  const int32_t* ids;             // [n_sel]
  const uint16_t* x[kMaxMats];
  uint16_t* y[kMaxMats];
  int64_t x_stride[kMaxMats];
  int64_t y_stride[kMaxMats];
  int32_t n_experts, n_sel, n_mats, wg_per_mat;
};

typedef __attribute__((address_space(3))) const u32x2 lds_u2;
typedef __attribute__((address_space(3))) const u32x4 lds_u4;
__device__ inline u32x2 lds8(uint32_t addr) { return *(lds_u2*)(size_t)addr; }
__device__ inline u32x4 lds16(uint32_t addr) { return *(lds_u4*)(size_t)addr; }
__device__ inline void lds_store8(uint32_t addr, u32x2 v) {
  *(__attribute__((address_space(3))) u32x2*)(size_t)addr = v;
}
__device__ inline void lds_store16(uint32_t addr, u32x4 v) {
  *(__attribute__((address_space(3))) u32x4*)(size_t)addr = v;
}

// First step of a dot chain, accumulator 0 (the VOP3P form takes the constant; the accumulating
// VOP2 form would need a register zeroed first).
__device__ inline float dot2_z(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}
__device__ inline uint32_t rotr(uint32_t v, uint32_t n) { return __builtin_amdgcn_alignbit(v, v, n); }
// (a & m) | c as one v_and_or_b32 with m in a scalar register.
__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}
// (a & m) | (b & ~m) as one v_bfi_b32 with m in a scalar register.
__device__ inline uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(a), "v"(b));
  return r;
}

// Constants of one split (L = log2 K).
template <int L>
struct Split {
  static constexpr uint32_t kK = 1u << L;
  static constexpr uint32_t kKeyMask = ((1u << (4 + L)) - 1u) << 3;   // z and a sign nibble
  static constexpr uint32_t kSignMask = 15u << (3 + L);                 // the sign nibble
  static constexpr uint32_t kQMask = ((1u << (10 - L)) - 1u) << (7 + L);
  // OR-ed onto q at bit 7 + L this exponent gives the float 2^(16-L) + q exactly.
  static constexpr uint32_t kExpo = (127u + 16u - (uint32_t)L) << 23;
  static constexpr float kBias = (float)(1u << (16 - L));
  static constexpr uint32_t kTHi = 128u << L;   // second-half table
};

struct Unit {
  u32x4 p;  // payload dwords of the half-group (one plane)
  u32x2 s;  // X, G
};

// Per lane-group work: units [u0, u0 + cnt) of the workgroup, chunk-major; the first kb of them
// lie in the lane group's first chunk cf (at half-groups hf, hf + 1, ...), the rest in chunk cf + 1.
struct LaneWork {
  int cnt, cf, hf, kb;
};

__device__ inline LaneWork lane_work(int lg, int nc, int nh) {
  const int U = nc * nh;
  const int base = U >> 6, rem = U & 63;
  LaneWork w;
  w.cnt = base + (lg < rem ? 1 : 0);
  const int u0 = lg * base + min(lg, rem);
  w.cf = u0 / nh;
  w.hf = u0 - w.cf * nh;
  w.kb = nh - w.hf;
  return w;
}
// Lane group holding unit u (inverse of the split above).
__device__ inline int lane_group_of(int u, int base, int rem) {
  if (base == 0) return u;
  const int big = (base + 1) * rem;
  return u < big ? u / (base + 1) : rem + (u - big) / base;
}

// Decode the 8 subvectors of one half-group unit and add them to acc.
template <int L>
__device__ __forceinline__ float decode_unit(const Unit& U, uint32_t half, uint32_t xa, float acc) {
  using S = Split<L>;
  const uint32_t G = U.s[1];
  const float mu = h2f(G);
  const float dl = h2f(G >> 16);
  const float mub = fmaf(-S::kBias, dl, mu);   // radius = (2^(16-L) + q) * delta + mub
  const uint32_t Xh = rotr(U.s[0], half << 4);  // this half's four high sign nibbles at bits 0..15
  const uint32_t expo = S::kExpo;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t P = U.p[m];
    const uint32_t R = rotr(P, 14);                              // b's fields at a's positions
    const uint32_t ka = P & S::kKeyMask;                         // T[0][s_a lo][z_a]
    const uint32_t kb = R & S::kKeyMask;                         // T[0][s_b lo][z_b]
    const uint32_t ha = bfi(S::kSignMask, rotr(Xh, (4 * m + 29 - L) & 31), ka);  // s_a hi
    const uint32_t hb = bfi(S::kSignMask, rotr(P, 28 - L), kb);                 // s_b hi
    const float qa = __uint_as_float(and_or(P, S::kQMask, expo));
    const float qb = __uint_as_float(and_or(R, S::kQMask, expo));
    {
      const u32x2 lo = lds8(ka);
      const u32x2 hi = lds8(ha + S::kTHi);
      const u32x4 xv = lds16(xa + 32u * m);
      float t = dot2_z(lo[0], xv[0]);
      t = dot2(lo[1], xv[1], t);
      t = dot2(hi[0], xv[2], t);
      t = dot2(hi[1], xv[3], t);
      acc = fmaf(fmaf(qa, dl, mub), t, acc);
    }
    {
      const u32x2 lo = lds8(kb);
      const u32x2 hi = lds8(hb + S::kTHi);
      const u32x4 xv = lds16(xa + 32u * m + 16u);
      float t = dot2_z(lo[0], xv[0]);
      t = dot2(lo[1], xv[1], t);
      t = dot2(hi[0], xv[2], t);
      t = dot2(hi[1], xv[3], t);
      acc = fmaf(fmaf(qb, dl, mub), t, acc);
    }
  }
  return acc;
}

// Sum of v over each aligned group of tau lanes (tau a power of two up to 64), left in the group's
// last lane, by a fixed sequence of cross-lane (DPP) additions: pairs, quads, eights (half-row
// mirror), rows (row mirror), then rows carried forward through row broadcasts.
template <int kCtrl, int kRowMask>
__device__ inline float dpp_add(float v) {
  const float t = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xF, false));
  return v + t;
}
__device__ inline float group_sum(float v, int tau) {
  if (tau >= 2) v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  if (tau >= 4) v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  if (tau >= 8) v = dpp_add<0x141, 0xF>(v);   // row_half_mirror
  if (tau >= 16) v = dpp_add<0x140, 0xF>(v);  // row_mirror
  if (tau >= 32) v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if (tau >= 64) v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// The whole workgroup: chunks [c0, c0 + nc) of one product. kGather: pi may be non-NULL.
template <int L, bool kGather>
__device__ __attribute__((always_inline)) void gemv_wg(const uint8_t* packed, const uint16_t* codebook, const int32_t* pi,
                        const uint16_t* x, uint16_t* y, int d_out, int d_in, int c0, int nc) {
  using S = Split<L>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lg = tid >> 4;
  const int l16 = tid & 15;
  const int nh = d_in >> 6;   // half-groups per row
  const int ng = d_in >> 7;   // groups per row
  const bool gather = kGather && pi != nullptr;
  const uint32_t XB = lds_x(L);
  const uint32_t XS = lds_xs(L, d_in);
  const uint32_t PB = lds_part(L, d_in, gather);

  // 1. Small loads first. Waves 0-3 each load the whole codebook into registers (lane l holds
  // codewords l, l + 64, ...): four requests per workgroup for data every workgroup shares. The
  // input (and pi) go straight into LDS, 1 KiB per wave and load.
  constexpr int kCwPerLane = (int)((S::kK + 63u) / 64u);
  u32x4 cw[kCwPerLane];
  if (wave < 4) {
    const __amdgpu_buffer_rsrc_t cb_rs = view(codebook, S::kK * 16u);
#pragma unroll
    for (int i = 0; i < kCwPerLane; ++i) {
      const uint32_t z = (uint32_t)(lane + 64 * i);
      cw[i] = __builtin_amdgcn_raw_buffer_load_b128(cb_rs, z < S::kK ? z * 16u : kNowhere, 0, 0);
    }
  }
  const int n8 = d_in >> 3;   // 16-byte input pieces
  {
    const __amdgpu_buffer_rsrc_t x_rs = view(x, (uint32_t)d_in * 2u);
    const int nkb = (2 * d_in + 1023) >> 10;   // 1 KiB pieces of the input
    const uint32_t dst = gather ? XS : XB;
    for (int b = wave; b < nkb; b += kThreads / 64)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          x_rs, (__attribute__((address_space(3))) void*)(size_t)(dst + (uint32_t)b * 1024u), 16,
          (uint32_t)b * 1024u + (uint32_t)(tid & 63) * 16u, 0, 0, 0);
    if (gather) {
      const __amdgpu_buffer_rsrc_t pi_rs = view(pi, (uint32_t)d_in * 4u);
      const uint32_t PI = lds_pi(L, d_in);
      const int npb = (4 * d_in + 1023) >> 10;
      for (int b = wave; b < npb; b += kThreads / 64)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            pi_rs, (__attribute__((address_space(3))) void*)(size_t)(PI + (uint32_t)b * 1024u), 16,
            (uint32_t)b * 1024u + (uint32_t)(tid & 63) * 16u, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. The lane group's packed units: the first kRing go out now.
  const LaneWork W = lane_work(lg, nc, nh);
  const int nu = nc * nh;
  const int cntw = __builtin_amdgcn_readfirstlane((nu >> 6) + ((nu & 63) > 4 * wave ? 1 : 0));
  const int tile0 = c0 >> 2;
  const int tiles = ((c0 + nc - 1) >> 2) - tile0 + 1;
  const __amdgpu_buffer_rsrc_t wv =
      view(packed + (size_t)tile0 * ng * kBlockBytes, (uint32_t)tiles * ng * kBlockBytes);
  // offsets of unit k of this lane: payload (16 bytes) and side (8 bytes)
  auto unit_off = [&](int k, uint32_t* po, uint32_t* so) {
    const bool seg1 = k >= W.kb;
    const int c = c0 + W.cf + (seg1 ? 1 : 0);
    const int hg = W.hf + k - (seg1 ? nh : 0);
    const uint32_t lit = (uint32_t)(((c & 3) << 4) | l16);
    const uint32_t blk = (uint32_t)(((c >> 2) - tile0) * ng + (hg >> 1)) * kBlockBytes;
    const bool ok = k < W.cnt;
    *po = ok ? blk + (uint32_t)(hg & 1) * 1024u + lit * 16u : kNowhere;
    *so = ok ? blk + (uint32_t)kSidePlane + lit * 8u : kNowhere;
  };
  Unit ring[kRing];
#pragma unroll
  for (int k = 0; k < kRing; ++k) {
    uint32_t po, so;
    unit_off(k, &po, &so);
    ring[k].p = __builtin_amdgcn_raw_buffer_load_b128(wv, po, 0, kNonTemporal);
    ring[k].s = __builtin_amdgcn_raw_buffer_load_b64(wv, so, 0, kNonTemporal);
  }

  // 3. LDS set-up: waves 0-3 write the sign-applied codeword table (wave w the (half, signs)
  // combinations w, w + 4, ..., for every codeword it holds), then (gathering) the input is
  // gathered into stored order.
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < kCwPerLane; ++i) {
      const uint32_t z = (uint32_t)(lane + 64 * i);
      if (z < S::kK) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t hs = (uint32_t)(wave + 4 * c);   // h * 16 + s
          const uint32_t h = hs >> 4, sg = hs & 15u;
          const uint32_t c01 = h ? cw[i][2] : cw[i][0];
          const uint32_t c23 = h ? cw[i][3] : cw[i][1];
          const uint32_t m01 = ((sg & 1u) << 15) | ((sg & 2u) << 30);
          const uint32_t m23 = ((sg & 4u) << 13) | ((sg & 8u) << 28);
          lds_store8((hs * S::kK + z) * 8u, u32x2{c01 ^ m01, c23 ^ m23});
        }
      }
    }
  }
  // every load but this wave's packed units has landed (the input pieces included)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kRing) : "memory");
  if constexpr (kGather) {
    if (gather) {
      __syncthreads();
      const uint32_t PI = lds_pi(L, d_in);
#pragma unroll
      for (int i = 0; i < kXIter; ++i) {
        const int e = tid + i * kThreads;
        if (i * kThreads < n8 && e < n8) {
          const u32x4 p0 = lds16(PI + (uint32_t)e * 32u);
          const u32x4 p1 = lds16(PI + (uint32_t)e * 32u + 16u);
          const uint32_t pe[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
          uint32_t o[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t i0 = min(pe[2 * k], (uint32_t)d_in - 1u);
            const uint32_t i1 = min(pe[2 * k + 1], (uint32_t)d_in - 1u);
            const uint32_t v0 =
                *(__attribute__((address_space(3))) const uint16_t*)(size_t)(XS + 2u * i0);
            const uint32_t v1 =
                *(__attribute__((address_space(3))) const uint16_t*)(size_t)(XS + 2u * i1);
            o[k] = v0 | (v1 << 16);
          }
          lds_store16(XB + (uint32_t)e * 16u, u32x4{o[0], o[1], o[2], o[3]});
        }
      }
    }
  }
  __syncthreads();

  // 4. Decode: kRing units in flight; unit k + kRing is requested once unit k is decoded.
  float acc = 0.0f, acc0 = 0.0f;
  for (int kk = 0; kk < cntw; kk += kRing) {
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      const int k = kk + d;
      if (k < cntw) {
        const bool seg1 = k >= W.kb;
        if (k == W.kb) {   // the range enters its second chunk
          acc0 = acc;
          acc = 0.0f;
        }
        const int hg = W.hf + k - (seg1 ? nh : 0);
        // input of the unit's 8 subvectors (units past the lane's range read position 0)
        const uint32_t xa = XB + (k < W.cnt ? (uint32_t)hg * 128u : 0u);
        acc = decode_unit<L>(ring[d], (uint32_t)hg & 1u, xa, acc);
        if (k + kRing < cntw) {
          uint32_t po, so;
          unit_off(k + kRing, &po, &so);
          ring[d].p = __builtin_amdgcn_raw_buffer_load_b128(wv, po, 0, kNonTemporal);
          ring[d].s = __builtin_amdgcn_raw_buffer_load_b64(wv, so, 0, kNonTemporal);
        }
      }
    }
  }

  // 5. Lane-group sums to LDS; then the lane groups that worked on a chunk (a contiguous run
  // lo..hi) are added for each of its rows: tau threads per row take every tau-th contributor in
  // order and a fixed cross-lane tree adds their sums (results reproducible bit for bit).
  const bool split = W.kb < W.cnt;   // the range covers two chunks
  {
    const uint32_t a = PB + (uint32_t)(lg * kChunkRows + l16) * 4u;
    *(__attribute__((address_space(3))) float*)(size_t)a = split ? acc0 : acc;
    *(__attribute__((address_space(3))) float*)(size_t)(a + kLaneGroups * kChunkRows * 4u) =
        split ? acc : 0.0f;
  }
  __syncthreads();
  {
    const int rows = nc * kChunkRows;
    // threads per row: 64 for one chunk, halving as chunks are added (a power of two dividing 64)
    const int tau = rows <= 16 ? 64 : rows <= 32 ? 32 : rows <= 64 ? 16 : rows <= 128 ? 8
                  : rows <= 256 ? 4 : rows <= 512 ? 2 : 1;
    const int r = tid / tau, k = tid & (tau - 1);
    float sum = 0.0f;
    if (r < rows) {
      const int cl = r >> 4, rr = r & 15;
      const int base = nu >> 6, rem = nu & 63;
      const int lo = lane_group_of(cl * nh, base, rem);
      const int hi = lane_group_of((cl + 1) * nh - 1, base, rem);
      // lo may have started in the previous chunk: its sum for this chunk is its second one
      const bool lo_second = lo * base + min(lo, rem) < cl * nh;
      for (int g = lo + k; g <= hi; g += tau) {
        const uint32_t seg = (g == lo && lo_second) ? 1u : 0u;
        sum += *(__attribute__((address_space(3))) const float*)(size_t)(
            PB + ((seg * kLaneGroups + (uint32_t)g) * kChunkRows + (uint32_t)rr) * 4u);
      }
    }
    sum = group_sum(sum, tau);
    if (r < rows && k == tau - 1) {
      const int row = (c0 + (r >> 4)) * kChunkRows + (r & 15);
      if (row < d_out) y[row] = f2h(sum);
    }
  }
}

template <typename F>
__device__ __forceinline__ void by_split(int L, F&& f) {
  switch (L) {
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 5: f(std::integral_constant<int, 5>{}); break;
    case 6: f(std::integral_constant<int, 6>{}); break;
    case 7: f(std::integral_constant<int, 7>{}); break;
    default: f(std::integral_constant<int, 8>{}); break;
  }
}

template <bool kGather>
__global__ void __launch_bounds__(kThreads) gemv_kernel(GemvArgs A) {
  const uint32_t e = A.wg[blockIdx.x];
  const Prod& P = A.prod[e & 15u];
  const int nc = (int)((e >> 4) & 63u) + 1;
  const int c0 = (int)(e >> 10);
  by_split(P.L, [&](auto Lc) {
    gemv_wg<decltype(Lc)::value, kGather>(P.packed, P.codebook, P.pi, P.x, P.y, P.d_out, P.d_in,
                                          c0, nc);
  });
}

// One pass of a routed-expert workgroup (a function of its own, so the kernel holds one copy).
__device__ __attribute__((noinline)) void moe_pass(const uint8_t* packed, const uint16_t* codebook,
                                                  const int32_t* pi, const uint16_t* x,
                                                  uint16_t* y, int d_out, int d_in, int L, int c0,
                                                  int nc) {
  by_split(L, [&](auto Lc) {
    gemv_wg<decltype(Lc)::value, true>(packed, codebook, pi, x, y, d_out, d_in, c0, nc);
  });
}

// Routed experts: workgroup w serves matrix j = (w / wg_per_mat) % n_mats of selected slot
// s = w / (wg_per_mat * n_mats), part w % wg_per_mat of its chunks. Descriptors with an invalid
// expert id, shape or split are skipped (their outputs are left unwritten).
__global__ void __launch_bounds__(kThreads) moe_kernel(MoeArgs A) {
  const int w = blockIdx.x;
  const int part = w % A.wg_per_mat;
  const int j = (w / A.wg_per_mat) % A.n_mats;
  const int s = w / (A.wg_per_mat * A.n_mats);
  // scalar loads (constant address space): the descriptor fields live in scalar registers
  typedef const __attribute__((address_space(4))) int32_t c_i32;
  typedef const __attribute__((address_space(4))) uint64_t c_u64;
  const int id = *(c_i32*)(A.ids + s);
  if (id < 0 || id >= A.n_experts) return;
  const sage_matrix_t* dsc = A.experts + (int64_t)id * A.n_mats + j;
  const int d_out = *(c_i32*)&dsc->d_out;
  const int d_in = *(c_i32*)&dsc->d_in;
  const int L = *(c_i32*)&dsc->log2K;
  const int V = *(c_i32*)&dsc->V;
  if (d_out < 1 || d_in < kGroupCols || (d_in & (kGroupCols - 1)) != 0 || L < 4 || L > 8 ||
      L + V != 10)
    return;
  const int32_t* pi = (const int32_t*)*(c_u64*)&dsc->pi;
  if (d_in > kMaxDin || lds_total(L, d_in, pi != nullptr) > kMaxLds) return;
  const uint8_t* packed = (const uint8_t*)*(c_u64*)&dsc->packed;
  const uint16_t* codebook = (const uint16_t*)*(c_u64*)&dsc->codebook;
  const int chunks = (d_out + kChunkRows - 1) / kChunkRows;
  const int q = (chunks + A.wg_per_mat - 1) / A.wg_per_mat;
  const int cbeg = part * q;
  const int cend = min(cbeg + q, chunks);
  const uint16_t* x = A.x[j] + (int64_t)s * A.x_stride[j];
  uint16_t* y = A.y[j] + (int64_t)s * A.y_stride[j];
  if (cend - cbeg <= kMaxChunks) {
    if (cend > cbeg) {
      by_split(L, [&](auto Lc) {
        gemv_wg<decltype(Lc)::value, true>(packed, codebook, pi, x, y, d_out, d_in, cbeg,
                                           cend - cbeg);
      });
    }
    return;
  }
  // a share of more than kMaxChunks chunks runs as several passes (matrices of more than
  // 1024 rows per workgroup of the launch)
  for (int c0 = cbeg; c0 < cend; c0 += kMaxChunks) {
    moe_pass(packed, codebook, pi, x, y, d_out, d_in, L, c0, min(kMaxChunks, cend - c0));
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// Planner: workgroups are shared out over the products in proportion to their units (largest
// remainders, so the launch stays within one workgroup per compute unit), then each product's
// chunks are split evenly over its workgroups.
// ------------------------------------------------------------------------------------------------

int check_product(const sage_matrix_t& m, const void* x, const void* y) {
  int st = check_matrix(&m);
  if (st != SAGE_OK) return st;
  if (x == nullptr || y == nullptr) return SAGE_ERR_NULL;
  if (!aligned(x, 4) || !aligned(y, 2)) return SAGE_ERR_ALIGN;
  if (m.d_in > kMaxDin || lds_total(m.log2K, m.d_in, m.pi != nullptr) > kMaxLds)
    return SAGE_ERR_SHAPE;
  return SAGE_OK;
}

struct Plan {
  GemvArgs args;
  int nwg = 0;
  size_t lds = 0;
  bool gather = false;
};

int plan(const sage_matrix_t* mats, const uint16_t* const* xs, uint16_t* const* ys, int n,
         Plan* P) {
  if (n < 1 || n > kMaxProducts) return SAGE_ERR_ARG;
  const int cus = device_cu_count();
  std::vector<int64_t> chunks(n), units(n);
  int64_t total_units = 0, total_chunks = 0;
  for (int i = 0; i < n; ++i) {
    int st = check_product(mats[i], xs[i], ys[i]);
    if (st != SAGE_OK) return st;
    chunks[i] = ceil_div(mats[i].d_out, kChunkRows);
    units[i] = chunks[i] * (mats[i].d_in / 64);
    total_units += units[i];
    total_chunks += chunks[i];
  }
  // workgroups: one per compute unit, no more than there are chunks, and at least enough that no
  // workgroup has more than kMaxChunks chunks
  int64_t G = std::min<int64_t>(cus, total_chunks);
  std::vector<int64_t> g(n);
  std::vector<std::pair<double, int>> rema;
  int64_t given = 0;
  for (int i = 0; i < n; ++i) {
    const double share = (double)G * (double)units[i] / (double)total_units;
    g[i] = std::max<int64_t>(1, (int64_t)share);
    given += g[i];
    rema.push_back({share - (double)(int64_t)share, i});
  }
  std::sort(rema.begin(), rema.end(), [](auto a, auto b) { return a.first > b.first; });
  for (size_t k = 0; given < G && k < rema.size(); ++k, ++given) g[rema[k].second]++;
  int64_t nwg = 0;
  for (int i = 0; i < n; ++i) {
    g[i] = std::min(g[i], chunks[i]);
    g[i] = std::max(g[i], (chunks[i] + kMaxChunks - 1) / kMaxChunks);
    nwg += g[i];
  }
  if (nwg > kMaxWgs) return SAGE_ERR_SHAPE;
  P->nwg = (int)nwg;
  P->lds = 0;
  P->gather = false;
  int w = 0;
  for (int i = 0; i < n; ++i) {
    const sage_matrix_t& m = mats[i];
    Prod& d = P->args.prod[i];
    d.packed = (const uint8_t*)m.packed;
    d.codebook = m.codebook;
    d.pi = m.pi;
    d.x = xs[i];
    d.y = ys[i];
    d.d_out = m.d_out;
    d.d_in = m.d_in;
    d.L = m.log2K;
    d.pad = 0;
    P->lds = std::max<size_t>(P->lds, lds_total(m.log2K, m.d_in, m.pi != nullptr));
    P->gather = P->gather || m.pi != nullptr;
    const int64_t q = chunks[i] / g[i], r = chunks[i] % g[i];
    int64_t c = 0;
    for (int64_t k = 0; k < g[i]; ++k) {
      const int64_t nc = q + (k < r ? 1 : 0);
      P->args.wg[w++] = (uint32_t)i | ((uint32_t)(nc - 1) << 4) | ((uint32_t)c << 10);
      c += nc;
    }
  }
  return SAGE_OK;
}

int launch(const Plan& P, sage_stream_t stream) {
  if (P.gather)
    hipLaunchKernelGGL(gemv_kernel<true>, dim3(P.nwg), dim3(kThreads), P.lds, (hipStream_t)stream,
                       P.args);
  else
    hipLaunchKernelGGL(gemv_kernel<false>, dim3(P.nwg), dim3(kThreads), P.lds, (hipStream_t)stream,
                       P.args);
  return hip_status();
}

// Allow the kernels up to 160 KiB of dynamic LDS, once per device.
void lds_limit_set() {
  static std::mutex mu;
  static bool done[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    (void)hipFuncSetAttribute((const void*)gemv_kernel<false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)hipFuncSetAttribute((const void*)gemv_kernel<true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)hipFuncSetAttribute((const void*)moe_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    done[dev] = true;
  }
}

int moe_launch(const sage_matrix_t* experts_dev, int n_experts, int n_mats, const int32_t* ids_dev,
               int n_sel, const uint16_t* const* xs, const int64_t* x_strides,
               uint16_t* const* ys, const int64_t* y_strides, sage_stream_t stream) {
  if (experts_dev == nullptr || ids_dev == nullptr || xs == nullptr || ys == nullptr)
    return SAGE_ERR_NULL;
  if (n_experts < 1 || n_sel < 1 || n_mats < 1 || n_mats > kMaxMats) return SAGE_ERR_ARG;
  if (!aligned(experts_dev, 8) || !aligned(ids_dev, 4)) return SAGE_ERR_ALIGN;
  MoeArgs A{};
  A.experts = experts_dev;
  A.ids = ids_dev;
  for (int j = 0; j < n_mats; ++j) {
    if (xs[j] == nullptr || ys[j] == nullptr) return SAGE_ERR_NULL;
    if (!aligned(xs[j], 4) || !aligned(ys[j], 2)) return SAGE_ERR_ALIGN;
    if (x_strides[j] < 0 || (x_strides[j] & 1) != 0 || y_strides[j] < 0) return SAGE_ERR_ARG;
    if (n_sel > 1 && y_strides[j] == 0) return SAGE_ERR_ARG;
    A.x[j] = xs[j];
    A.y[j] = ys[j];
    A.x_stride[j] = x_strides[j];
    A.y_stride[j] = y_strides[j];
  }
  A.n_experts = n_experts;
  A.n_sel = n_sel;
  A.n_mats = n_mats;
  // every selected matrix gets the same share of the compute units; a matrix larger than that
  // share's kMaxChunks chunks per workgroup is cut at that many
  const int cus = device_cu_count();
  A.wg_per_mat = std::max(1, cus / (n_sel * n_mats));
  const int64_t nwg = (int64_t)A.wg_per_mat * n_mats * n_sel;
  if (nwg > (1 << 20)) return SAGE_ERR_ARG;
  lds_limit_set();
  hipLaunchKernelGGL(moe_kernel, dim3((unsigned)nwg), dim3(kThreads), 160 * 1024,
                     (hipStream_t)stream, A);
  return hip_status();
}

}  // namespace
}  // namespace sage

using namespace sage;

extern "C" {

int sage_gemv_workspace_bytes(const sage_matrix_t* m, size_t* bytes) {
  if (bytes == nullptr) return SAGE_ERR_NULL;
  int st = check_matrix(m);
  if (st != SAGE_OK) return st;
  *bytes = 0;
  return SAGE_OK;
}

int sage_gemv(const sage_matrix_t* m, const uint16_t* x, uint16_t* y, void* ws, size_t ws_bytes,
              sage_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (m == nullptr) return SAGE_ERR_NULL;
  Plan P;
  int st = plan(m, &x, &y, 1, &P);
  if (st != SAGE_OK) return st;
  lds_limit_set();
  return launch(P, stream);
}

int sage_gemv_multi_workspace_bytes(const sage_matrix_t* mats, int n, size_t* bytes) {
  if (bytes == nullptr || mats == nullptr) return SAGE_ERR_NULL;
  if (n < 1 || n > kMaxProducts) return SAGE_ERR_ARG;
  for (int i = 0; i < n; ++i) {
    int st = check_matrix(&mats[i]);
    if (st != SAGE_OK) return st;
  }
  *bytes = 0;
  return SAGE_OK;
}

int sage_gemv_multi(const sage_matrix_t* mats, const uint16_t* const* xs, uint16_t* const* ys,
                    int n, void* ws, size_t ws_bytes, sage_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (mats == nullptr || xs == nullptr || ys == nullptr) return SAGE_ERR_NULL;
  Plan P;
  int st = plan(mats, xs, ys, n, &P);
  if (st != SAGE_OK) return st;
  lds_limit_set();
  return launch(P, stream);
}

int sage_moe_gemv(const sage_matrix_t* experts_dev, int n_experts, const int32_t* ids_dev,
                  int n_sel, const uint16_t* x, int64_t x_stride, uint16_t* y, int64_t y_stride,
                  sage_stream_t stream) {
  return moe_launch(experts_dev, n_experts, 1, ids_dev, n_sel, &x, &x_stride, &y, &y_stride,
                    stream);
}

int sage_moe_gemv_grouped(const sage_matrix_t* experts_dev, int n_experts, int n_mats,
                          const int32_t* ids_dev, int n_sel, const uint16_t* const* xs,
                          const int64_t* x_strides, uint16_t* const* ys, const int64_t* y_strides,
                          sage_stream_t stream) {
  if (x_strides == nullptr || y_strides == nullptr) return SAGE_ERR_NULL;
  return moe_launch(experts_dev, n_experts, n_mats, ids_dev, n_sel, xs, x_strides, ys, y_strides,
                    stream);
}

}  // extern "C"
