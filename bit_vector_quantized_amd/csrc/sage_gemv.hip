// Batch-one decode-and-multiply for SAGE-packed weights on gfx950 (SAGE paper §3.5 and App. A.1):
// y = W_hat x with W_hat decoded on the fly from its 18-bit subvector codes (§3.1 Eq. (1)-(3)).
//
// Work decomposition. Rows are taken in chunks of 16 (a quarter of a packed row tile). A workgroup
// of 1024 threads (16 wavefronts; one or two per compute unit) owns whole rows: a run of chunks
// of one product, so no partial sum ever leaves the compute unit (no split-K hand-off between
// workgroups). Its (chunk, 128-column group) units, chunk-major, are cut into 64 contiguous ranges
// whose lengths differ by at most one, one per lane group of 16 lanes; lane l of a group owns row l
// of the chunk it is working on. A range crosses at most one chunk boundary, so a lane keeps two sums.
// At the end the sums of the ranges covering a row's chunk are added in a fixed order (results are
// reproducible bit for bit) and one rounding to fp16 gives y.
//
// Decode. The workgroup builds, once, a table of sign-applied codeword halves in LDS:
// T[h][s][z] (h = first or second half of the 8-wide codeword, s = 4 sign bits, z = codeword) holds
// the four fp16 values c_z[4h..4h+3] with element i negated when bit i of s is set. The table
// depends only on the codebook (256 K bytes), not on the input, so nothing is rebuilt per input
// position. A subvector then costs two 8-byte table reads, addressed straight from bit fields of
// the packed word (the packed layout puts z and each sign nibble next to each other), four fp16
// dot2 steps with fp32 accumulation against the input, and the radius mu + q*delta applied once
// to the 8-term dot product (App. A.1: one multiply instead of eight). Lane j of a lane group reads
// the inputs of the unit's subvector j from LDS once, and every lane of the group takes them from
// lane j through a DPP row broadcast inside the dot steps. The input is staged in LDS
// in stored (permuted) column order: copied as is when the matrix's pi is NULL (the producer wrote
// it permuted, §3.5 compiled decoding), else gathered through pi once per workgroup (§3.5 eager
// decoding: the gather fused into the product).
//
// Memory access. Every global load is a buffer load through a range-checked view: loads past the
// range return zeros without a memory access, so loads are issued unconditionally. The codebook
// and input land first; then every lane group requests its units, two in flight while it decodes.
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
constexpr int kRing = 2;           // group units in flight per lane group
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

// One unit of work: a lane group's 16 rows (one chunk) by one 128-column group, i.e. each lane's
// three pieces of one packed block.
struct Unit {
  u32x4 a;  // payload dwords P0..P3 of the lane's row (plane A)
  u32x4 b;  // P4..P7 (plane B)
  u32x2 s;  // X, G
};

// floor(n / d) for 0 <= n < 2^16, given r = v_rcp_f32(d) for an integer 1 <= d < 2^16: n + 1/2 over
// d lies at least 1/(2d) from every integer, and the float product's error is below (n/d) 2^-21.
__device__ inline int div_small(int n, float r) { return (int)(((float)n + 0.5f) * r); }

// Per lane-group work. A workgroup's units (chunk, group), chunk-major, are split into 64
// contiguous ranges, range w for lane group w (so a wavefront's four ranges are neighbours and
// differ in length only where the longer ranges end). Range w is units [u0, u0 + cnt); its first
// kb units lie in chunk cf (groups gf, gf + 1, ...), the rest in chunk cf + 1.
struct LaneWork {
  int u0, cnt, cf, gf, kb;
};

__device__ inline LaneWork lane_work(int w, int nu, int ng, float rcp_ng) {
  const int base = nu >> 6, rem = nu & 63;
  LaneWork r;
  r.cnt = base + (w < rem ? 1 : 0);
  r.u0 = w * base + min(w, rem);
  r.cf = div_small(r.u0, rcp_ng);
  r.gf = r.u0 - r.cf * ng;
  r.kb = ng - r.gf;
  return r;
}
// Range holding unit u (inverse of the split above).
__device__ inline int range_of(int u, int base, int rem) {
  if (base == 0) return u;
  const int big = (base + 1) * rem;
  return u < big ? div_small(u, __builtin_amdgcn_rcpf((float)(base + 1)))
                 : rem + div_small(u - big, __builtin_amdgcn_rcpf((float)base));
}

// acc += r * (c . x) for one subvector: c its 8 sign-applied codeword values (lo, hi: four fp16
// pairs), x its 8 inputs, all four fp16 pairs of which lane J of the lane group holds, r its radius.
// The lane group is a DPP row of 16 lanes, and row_newbcast hands every lane of the row lane J's
// register as the dot's first operand: no LDS traffic for the input. The dot product starts from 0
// and accumulates in fp32; the radius multiply-add follows in the same block, so each subvector is
// added in order and its dot product does not stay live.
//
// Wait states the compiler cannot insert, the dot steps being inside the block: the leading s_nop
// gives the two a DPP read needs after a VALU write of its source (the inputs come from LDS reads,
// but the block does not rely on that); the s_nop 2 gives the three a VALU read needs after a
// v_dot2c write of the value (a dot step reading it as its own accumulator needs none). Row
// broadcasts run with every lane active: under a partial exec mask they gave wrong sums.
template <int J>
__device__ __forceinline__ float dot8_row(float acc, float r, u32x2 lo, u32x2 hi, u32x4 xv) {
  float t;
  asm("s_nop 1\n\t"
      "v_mov_b32 %1, 0\n\t"
      "v_dot2c_f32_f16_dpp %1, %7, %3 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %1, %8, %4 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %1, %9, %5 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %1, %10, %6 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 2\n\t"
      "v_fmac_f32 %0, %2, %1"
      : "+v"(acc), "=&v"(t)
      : "v"(r), "v"(lo[0]), "v"(lo[1]), "v"(hi[0]), "v"(hi[1]), "v"(xv[0]), "v"(xv[1]),
        "v"(xv[2]), "v"(xv[3]), "n"(J));
  return acc;
}

// Decode the 16 subvectors of one unit and add them to acc. xa: LDS address of the group's 128
// inputs; lane l of the lane group reads inputs 8l .. 8l + 7 (subvector l's).
template <int L>
__device__ __forceinline__ float decode_unit(const Unit& U, uint32_t xa, int l16, float acc) {
  using S = Split<L>;
  const u32x4 xv = lds16(xa + (uint32_t)l16 * 16u);
  const uint32_t X = U.s[0];
  const uint32_t G = U.s[1];
  const float mu = h2f(G);
  const float dl = h2f(G >> 16);
  const float mub = fmaf(-S::kBias, dl, mu);   // radius = (2^(16-L) + q) * delta + mub
  const uint32_t expo = S::kExpo;
  auto pair = [&](auto mc) {
    constexpr int m = decltype(mc)::value;
    const uint32_t P = m < 4 ? U.a[m & 3] : U.b[m & 3];
    const uint32_t R = rotr(P, 14);                              // b's fields at a's positions
    const uint32_t ka = P & S::kKeyMask;                         // T[0][s_a lo][z_a]
    const uint32_t kb = R & S::kKeyMask;                         // T[0][s_b lo][z_b]
    const uint32_t ha = bfi(S::kSignMask, rotr(X, (4 * m + 29 - L) & 31), ka);  // s_a hi
    const uint32_t hb = bfi(S::kSignMask, rotr(P, 28 - L), kb);                // s_b hi
    const float qa = __uint_as_float(and_or(P, S::kQMask, expo));
    const float qb = __uint_as_float(and_or(R, S::kQMask, expo));
    acc = dot8_row<2 * m>(acc, fmaf(qa, dl, mub), lds8(ka), lds8(ha + S::kTHi), xv);
    acc = dot8_row<2 * m + 1>(acc, fmaf(qb, dl, mub), lds8(kb), lds8(hb + S::kTHi), xv);
  };
  pair(std::integral_constant<int, 0>{});
  pair(std::integral_constant<int, 1>{});
  pair(std::integral_constant<int, 2>{});
  pair(std::integral_constant<int, 3>{});
  pair(std::integral_constant<int, 4>{});
  pair(std::integral_constant<int, 5>{});
  pair(std::integral_constant<int, 6>{});
  pair(std::integral_constant<int, 7>{});
  return acc;
}

// The whole workgroup: chunks [c0, c0 + nc) of one product. kGather: pi may be non-NULL. kEarly:
// the launch has at most one workgroup per compute unit (see the order of work below).
//
// Order of work. The codebook (in registers of waves 0-3) and the input (in LDS) are waited for
// first: a compute unit returns load data in request order across its waves, so small loads
// queued behind a packed stream would arrive only with it. With two workgroups per compute unit
// the table is also written before any packed unit is requested, so the first workgroup's stream
// does not overtake the second's small loads. With one (kEarly), each wave requests the units it
// steps through as soon as the small loads have landed, and the table build (and the gather)
// overlap their latency. Each wave then decodes its units as they land. Every VALU instruction outside the decode loop runs on all 16 wavefronts, so
// the per-thread set-up is kept short and done while the first loads are in flight.
template <int L, bool kGather, bool kEarly>
__device__ __attribute__((always_inline)) void gemv_wg(const uint8_t* packed, const uint16_t* codebook, const int32_t* pi,
                        const uint16_t* x, uint16_t* y, int d_out, int d_in, int c0, int nc) {
  using S = Split<L>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = tid & 15;
  const int rw = tid >> 4;   // this lane group, and its range
  const int ng = d_in >> 7;   // groups per row
  const int nu = nc * ng;     // units of the workgroup
  const bool gather = kGather && pi != nullptr;
  const uint32_t XB = lds_x(L);
  const uint32_t XS = lds_xs(L, d_in);
  const uint32_t PB = lds_part(L, d_in, gather);

  // 1. Small loads. Waves 0-3 each load the whole codebook into registers (lane l holds codewords
  // l, l + 64, ...): four requests per workgroup for data every workgroup shares. The input (and
  // pi) go straight into LDS, 1 KiB per wave and load.
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
          (uint32_t)b * 1024u + (uint32_t)lane * 16u, 0, 0, 0);
    if (gather) {
      const __amdgpu_buffer_rsrc_t pi_rs = view(pi, (uint32_t)d_in * 4u);
      const uint32_t PI = lds_pi(L, d_in);
      const int npb = (4 * d_in + 1023) >> 10;
      for (int b = wave; b < npb; b += kThreads / 64)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            pi_rs, (__attribute__((address_space(3))) void*)(size_t)(PI + (uint32_t)b * 1024u), 16,
            (uint32_t)b * 1024u + (uint32_t)lane * 16u, 0, 0, 0);
    }
  }

  // 2. While those are in flight: this lane group's range and the offsets of its units. Unit k
  // of the range is (chunk cf, group gf + k) for k < kb, then (chunk cf + 1, group k - kb); both
  // runs step 2560 bytes (one block) per unit, so unit k sits at base + 2560 k with the base of
  // its run (the second run's base shifted back by kb blocks).
  const LaneWork W = lane_work(rw, nu, ng, __builtin_amdgcn_rcpf((float)ng));
  // units this wave steps through: the longest range among its four lane groups (range 4 wave)
  const int cntw = __builtin_amdgcn_readfirstlane((nu >> 6) + (4 * wave < (nu & 63) ? 1 : 0));
  const int tile0 = c0 >> 2;
  const int tiles = ((c0 + nc - 1) >> 2) - tile0 + 1;
  const uint32_t tile_bytes = (uint32_t)ng * kBlockBytes;
  const __amdgpu_buffer_rsrc_t wv =
      view(packed + (size_t)tile0 * tile_bytes, (uint32_t)tiles * tile_bytes);
  uint32_t pa0, sa0, pa1, sa1, xa0, xa1;   // payload, side and input offsets of both runs
  {
    const int ca = c0 + W.cf, cb = ca + 1;
    const uint32_t la = (uint32_t)(((ca & 3) << 4) | l16), lb = (uint32_t)(((cb & 3) << 4) | l16);
    const uint32_t ta = __umul24((uint32_t)((ca >> 2) - tile0), tile_bytes) +
                        __umul24((uint32_t)W.gf, (uint32_t)kBlockBytes);
    const uint32_t tb = __umul24((uint32_t)((cb >> 2) - tile0), tile_bytes) -
                        __umul24((uint32_t)W.kb, (uint32_t)kBlockBytes);
    pa0 = ta + la * 16u;
    sa0 = ta + (uint32_t)kSidePlane + la * 8u;
    pa1 = tb + lb * 16u;
    sa1 = tb + (uint32_t)kSidePlane + lb * 8u;
    xa0 = XB + (uint32_t)W.gf * 256u;
    xa1 = XB - (uint32_t)W.kb * 256u;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Packed units: kRing per lane group in flight; unit k + kRing is requested once unit k is
  // decoded. A range shorter than its wave's longest steps one unit past its end. That unit is
  // read as zeros and decoded with every lane active (its zero grid adds exactly 0): the DPP row
  // broadcasts of the dot steps gave wrong sums when run under a partial exec mask, even with every
  // lane of the row active. Its inputs are those of the group after the range's last one in the
  // same chunk, or of group 0 when the range ends at its chunk's end (a range covers at most a
  // chunk's units, so never the end of a second chunk): always staged, finite inputs.
  auto request = [&](Unit& u, int k) {
    const uint32_t step = (uint32_t)k * (uint32_t)kBlockBytes;
    const bool second = k >= W.kb;
    const bool ok = k < W.cnt;
    const uint32_t po = ok ? (second ? pa1 : pa0) + step : kNowhere;
    const uint32_t so = ok ? (second ? sa1 : sa0) + step : kNowhere;
    u.a = __builtin_amdgcn_raw_buffer_load_b128(wv, po, 0, kNonTemporal);
    u.b = __builtin_amdgcn_raw_buffer_load_b128(wv, po + (uint32_t)kPlaneB, 0, kNonTemporal);
    u.s = __builtin_amdgcn_raw_buffer_load_b64(wv, so, 0, kNonTemporal);
  };
  Unit ring[kRing];
  if constexpr (kEarly) {
    // only units the wave steps through (the others are never decoded)
#pragma unroll
    for (int k = 0; k < kRing; ++k)
      if (k < cntw) request(ring[k], k);
  }

  // 3. LDS set-up: waves 0-3 write the sign-applied codeword table (wave w the (half, signs)
  // combinations w, w + 4, ..., for every codeword it holds); gathering, every thread puts input
  // pieces into stored order.
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
  if constexpr (kGather) {
    if (gather) {
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

  // Waves in their decode loop issue ahead of waves still in their set-up (the other workgroup of
  // the compute unit) and of waves ending theirs: the decode of landed data is the launch's critical
  // path (measured: layer step 21.07-21.11 -> 20.75-20.89 us, gate|up 6.90-6.91 -> 6.76-6.79 us;
  // keeping the raised priority through the end gave back most of it).
  __builtin_amdgcn_s_setprio(2);
  // 4. The packed units (requested here with two workgroups per compute unit), decoded as they
  // land.
  if constexpr (!kEarly) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) request(ring[k], k);
  }
  // only a range that really crosses into a second chunk switches sums
  const bool split = W.kb < W.cnt;
  float acc = 0.0f, acc0 = 0.0f;
  for (int kk = 0; kk < cntw; kk += kRing) {
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      const int k = kk + d;
      if (k < cntw) {
        if (split && k == W.kb) {   // the range enters its second chunk
          acc0 = acc;
          acc = 0.0f;
        }
        const uint32_t xa = (k >= W.kb ? xa1 : xa0) + (uint32_t)k * 256u;
        acc = decode_unit<L>(ring[d], xa, l16, acc);
        if (k + kRing < cntw) request(ring[d], k + kRing);
      }
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // 5. Range sums to LDS (slot 0: the range's first chunk, slot 1: its second). A row's sum is
  // over the ranges that cover its chunk, a contiguous run lo..hi (at most 64, and at most the
  // chunk's ng units). The end of a launch is a chain of dependent waits, so eight neighbouring
  // lanes take one row: lane p adds ranges lo + p, lo + p + 8, ... (N reads, all issued before the
  // first add), and the eight part sums meet in a fixed tree ((p0 + p1) + (p2 + p3)) + ((p4 + p5)
  // + (p6 + p7)) by DPP moves, which hands every lane of the eight the same bits: a fixed order,
  // so results are reproducible bit for bit.
  {
    const uint32_t a = PB + (uint32_t)(rw * kChunkRows + l16) * 4u;
    *(__attribute__((address_space(3))) float*)(size_t)a = split ? acc0 : acc;
    *(__attribute__((address_space(3))) float*)(size_t)(a + kLaneGroups * kChunkRows * 4u) =
        split ? acc : 0.0f;
  }
  __syncthreads();
  {
    typedef __attribute__((address_space(3))) const float lds_f;
    const int base = nu >> 6, rem = nu & 63;
    const int p = lane & 7;
    const int nrows = nc * kChunkRows;
    auto rows = [&](auto Nc) {
      constexpr int N = decltype(Nc)::value;   // 8 N ranges per row at most
      // wave w takes rows 8w .. 8w + 7, then 8w + 128 ...: a wave-uniform trip count, so only
      // the waves with rows run and each runs whole (the DPP moves read neighbouring lanes)
      for (int i0 = wave * 8; i0 < nrows; i0 += kThreads / 8) {
        const int i = i0 + (lane >> 3);
        const bool valid = i < nrows;
        const int cl = valid ? i >> 4 : 0, rr = i & 15;
        const int ub = cl * ng;   // the chunk's first unit
        const int lo = range_of(ub, base, rem);
        const int last = valid ? range_of(ub + ng - 1, base, rem) - lo : -1;   // hi - lo
        // lo may have started in the previous chunk: its sum for this chunk is its second one
        const bool seg = p == 0 && lo * base + min(lo, rem) < ub;
        // range lo + p + 8k sits at a0 + 512 k; past hi the reads stay inside both slots
        // (lo + p + 8k < 128) and are replaced by zeros
        const uint32_t a0 = PB + ((uint32_t)(lo + p) * kChunkRows + (uint32_t)rr) * 4u;
        float v[N];
        v[0] = *(lds_f*)(size_t)(a0 + (seg ? (uint32_t)(kLaneGroups * kChunkRows * 4) : 0u));
#pragma unroll
        for (int k = 1; k < N; ++k) v[k] = *(lds_f*)(size_t)(a0 + 512u * (uint32_t)k);
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < N; ++k) s += p + 8 * k <= last ? v[k] : 0.0f;
        s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
        s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, false));
        s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, s), 0x141, 0xF, 0xF, false));
        const int row = (c0 + cl) * kChunkRows + rr;
        if (valid && p == 0 && row < d_out) y[row] = f2h(s);
      }
    };
    // a covering range holds at least one of the chunk's ng units
    if (ng <= 32)
      rows(std::integral_constant<int, 4>{});
    else
      rows(std::integral_constant<int, 8>{});
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

// kL: the split (log2 K) of every product of the launch, compiled in; 0 when the products' splits
// differ and each workgroup selects its product's at run time. One split per kernel keeps the code a
// wave runs through about a third as long (fewer instruction-cache misses while the workgroups
// start; measured: every layer launch 0.05-0.14 us shorter).
template <bool kGather, bool kEarly, int kL>
__global__ void __launch_bounds__(kThreads) gemv_kernel(GemvArgs A) {
  const uint32_t e = A.wg[blockIdx.x];
  const Prod& P = A.prod[e & 15u];
  const int nc = (int)((e >> 4) & 63u) + 1;
  const int c0 = (int)(e >> 10);
  if constexpr (kL != 0) {
    gemv_wg<kL, kGather, kEarly>(P.packed, P.codebook, P.pi, P.x, P.y, P.d_out, P.d_in, c0, nc);
  } else {
    by_split(P.L, [&](auto Lc) {
      gemv_wg<decltype(Lc)::value, kGather, kEarly>(P.packed, P.codebook, P.pi, P.x, P.y, P.d_out,
                                                    P.d_in, c0, nc);
    });
  }
}

// One pass of a routed-expert workgroup (a function of its own, so the kernel holds one copy).
__device__ __attribute__((noinline)) void moe_pass(const uint8_t* packed, const uint16_t* codebook,
                                                  const int32_t* pi, const uint16_t* x,
                                                  uint16_t* y, int d_out, int d_in, int L, int c0,
                                                  int nc) {
  by_split(L, [&](auto Lc) {
    gemv_wg<decltype(Lc)::value, true, true>(packed, codebook, pi, x, y, d_out, d_in, c0, nc);
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
        gemv_wg<decltype(Lc)::value, true, true>(packed, codebook, pi, x, y, d_out, d_in, cbeg,
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
  bool early = false;   // at most one workgroup per compute unit: request at the first barrier
  int L = 0;            // the products' common split, or 0 when they differ
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
  // workgroups: two per compute unit when two fit in its LDS and every compute unit gets two (at
  // least twice as many chunks as units; four times as many when a product gathers its input, whose
  // gather pass then runs over at least two chunks per workgroup): eight wavefronts per SIMD then
  // hide the latency of the table reads better than four. Otherwise one, which requests its packed
  // units as soon as its small loads have landed (measured: q|k|v's 384 chunks 5.14 -> 4.90 us with
  // one; gate|up's 1216 chunks 7.38 us with two, 7.76 us with one; with pi gathered, gate|up
  // 7.47-7.50 us with two, 7.78-7.81 us with one, but one 9728x2560 matrix (608 chunks) 5.9-6.1 us
  // with two, 5.3 us with one). No more workgroups than there are chunks, and at least enough that
  // no workgroup has more than kMaxChunks chunks.
  uint32_t lds_max = 0;
  bool any_gather = false;
  for (int i = 0; i < n; ++i) {
    lds_max = std::max(lds_max, lds_total(mats[i].log2K, mats[i].d_in, mats[i].pi != nullptr));
    any_gather = any_gather || mats[i].pi != nullptr;
  }
  const int per_cu =
      lds_max <= kMaxLds / 2 && total_chunks >= (any_gather ? 4 : 2) * (int64_t)cus ? 2 : 1;
  int64_t G = std::min<int64_t>((int64_t)cus * per_cu, total_chunks);
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
  P->early = nwg <= cus;
  P->lds = 0;
  P->gather = false;
  P->L = mats[0].log2K;
  for (int i = 1; i < n; ++i)
    if (mats[i].log2K != P->L) P->L = 0;
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
  // Workgroups with the most chunks first: they are dispatched first, so their small loads go out
  // before the other workgroups' packed streams and they start decoding earliest (measured: gate|up
  // 7.15 -> 6.87-6.96 us with two workgroups per compute unit, q|k|v 4.67 -> 4.61 us with one).
  std::stable_sort(P->args.wg, P->args.wg + w,
                   [](uint32_t a, uint32_t b) { return ((a >> 4) & 63u) > ((b >> 4) & 63u); });
  return SAGE_OK;
}

typedef void (*GemvFn)(GemvArgs);

// The kernels of one (gather, early) pair: index 0 selects the split at run time, 1 + L - 4 has
// split L compiled in.
template <bool kGather, bool kEarly>
constexpr GemvFn kGemvBySplit[6] = {gemv_kernel<kGather, kEarly, 0>, gemv_kernel<kGather, kEarly, 4>,
                                    gemv_kernel<kGather, kEarly, 5>, gemv_kernel<kGather, kEarly, 6>,
                                    gemv_kernel<kGather, kEarly, 7>, gemv_kernel<kGather, kEarly, 8>};
constexpr const GemvFn* kGemvFns[4] = {kGemvBySplit<false, false>, kGemvBySplit<false, true>,
                                       kGemvBySplit<true, false>, kGemvBySplit<true, true>};

int launch(const Plan& P, sage_stream_t stream) {
  const GemvFn fn = kGemvFns[(P.gather ? 2 : 0) + (P.early ? 1 : 0)][P.L ? P.L - 3 : 0];
  hipLaunchKernelGGL(fn, dim3(P.nwg), dim3(kThreads), P.lds, (hipStream_t)stream, P.args);
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
    for (const GemvFn* fns : kGemvFns)
      for (int k = 0; k < 6; ++k)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fns[k]),
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
