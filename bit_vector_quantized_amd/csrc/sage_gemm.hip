// Small-batch product Y = X W_hat^T for SAGE-packed weights on gfx950 matrix cores (SAGE paper §3.5
// and App. A.1: each weight is decoded once per output tile and reused across the activation rows).
//
// A workgroup owns one 64-row tile of W (16 rows per wavefront), one range of column groups and one
// chunk of up to 64 activation rows. The wavefront computes D = A * B with
// v_mfma_f32_16x16x32_f16: B is 32 input channels x 16 weight rows, A is 16 activation rows x the
// same 32 channels. In the B operand a lane supplies 8 consecutive input channels of one weight row,
// which is exactly one subvector, so the lane decodes its subvector straight into the operand:
// w_i = r_hat * (+-c_z,i), r_hat = mu + q*delta computed in fp32, the product formed in fp16. The
// activations are gathered through pi into LDS once per workgroup (§3.2) and read as the A operand.
// Lanes 16u..16u+15 of MFMA step kk supply subvector 4u + kk of their row, so A reads the same
// channels; the channel order inside the 32-wide contraction is the same for A and B.
#include "sage_internal.hpp"

namespace sage {
namespace {

constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kMaxGS = 8;        // column groups per split

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const uint8_t* packed;
  const uint16_t* codebook;
  const int32_t* pi;
  const uint16_t* X;
  uint16_t* Y;
  float* partial;
  uint32_t* counters;
  int64_t ldx, ldy;
  int32_t d_out, d_in, M, L;
  int32_t rt, ng, S, gs, mchunks;
  int32_t mrows_chunk;  // activation rows per workgroup = 16 * tiles
  int32_t vec_x;        // X rows are 16-byte aligned and already in permuted order
};

constexpr int kPermuteMinRows = 8;  // from this many rows on, X is permuted once per call

// Sign masks of one nibble: bits 0/1 -> signs of the first fp16 pair, bits 2/3 -> second pair.
__device__ inline uint2 nibble_masks(uint32_t n) {
  return make_uint2(((n & 1u) << 15) | ((n & 2u) << 30), ((n & 4u) << 13) | ((n & 8u) << 28));
}

// X[:, pi] for M rows into a dense [M][d_in] buffer (the reorder the paper does once per
// projection before prefill, §3.5).
__global__ void __launch_bounds__(256) permute_rows_kernel(const uint16_t* __restrict__ X,
                                                           int64_t ldx,
                                                           const int32_t* __restrict__ pi,
                                                           int d_in, int M,
                                                           uint16_t* __restrict__ Xp) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)M * d_in) return;
  const int m = (int)(t / d_in);
  const int p = (int)(t - (int64_t)m * d_in);
  const int src = pi ? (int)min((uint32_t)pi[p], (uint32_t)d_in - 1u) : p;
  Xp[t] = X[(int64_t)m * ldx + src];
}

__device__ inline uint32_t mul_pair(uint32_t c, half2_t r) {
  const half2_t v = __builtin_bit_cast(half2_t, c) * r;
  return __builtin_bit_cast(uint32_t, v);
}

template <int L, int NT>
__device__ void gemm_body(const GemmArgs& A, int rt, int split, int mchunk, uint8_t* smem) {
  constexpr uint32_t kK = 1u << L;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 15;      // weight row inside the wave's 16
  const int u = lane >> 4;      // channel quadrant
  const int g0 = split * A.gs;
  const int ngl = min(A.ng - g0, A.gs);
  const int m0 = mchunk * A.mrows_chunk;
  const int mrows = min(A.M - m0, NT * 16);
  const int wrow_in_tile = wave * 16 + j;
  const int wrow = rt * kTileRows + wrow_in_tile;

  // LDS: codebook replicas [K][16][16 B], sign-mask table [16][8 B], then the X tile
  // [NT*16][gs*128 (+8 pad)] fp16.
  uint8_t* cb = smem;
  uint2* smask = reinterpret_cast<uint2*>(smem + kK * 256);
  const int xstride = A.gs * kGroupCols + 8;  // fp16 elements per activation row (padded)
  _Float16* xs = reinterpret_cast<_Float16*>(smem + kK * 256 + 128);
  {
    const uint4* cbg = reinterpret_cast<const uint4*>(A.codebook);
    for (int z = tid; z < (int)kK; z += kGemmThreads) {
      const uint4 cw = cbg[z];
#pragma unroll
      for (int r = 0; r < 16; ++r) *reinterpret_cast<uint4*>(cb + z * 256 + r * 16) = cw;
    }
    if (tid < 16) smask[tid] = nibble_masks((uint32_t)tid);
    const int cols = ngl * kGroupCols;
    const int c0 = g0 * kGroupCols;
    if (A.vec_x) {
      // 16-byte chunks of already-permuted rows, eight loads in flight per thread
      const int chunks = cols / 8;
      const int total = NT * 16 * chunks;
      for (int base = 0; base < total; base += 8 * kGemmThreads) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = base + u * kGemmThreads + tid;
          const int m = e / chunks;
          v[u] = make_uint4(0, 0, 0, 0);
          if (e < total && m < mrows)
            v[u] = *reinterpret_cast<const uint4*>(A.X + (int64_t)(m0 + m) * A.ldx + c0 +
                                                   (e - m * chunks) * 8);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = base + u * kGemmThreads + tid;
          const int m = e / chunks;
          if (e < total) *reinterpret_cast<uint4*>(xs + m * xstride + (e - m * chunks) * 8) = v[u];
        }
      }
    } else {
      for (int e = tid; e < NT * 16 * cols; e += kGemmThreads) {
        const int m = e / cols;
        const int p = e - m * cols;
        _Float16 v = (_Float16)0.0f;
        if (m < mrows) {
          const int col = c0 + p;
          const int src = A.pi ? (int)min((uint32_t)A.pi[col], (uint32_t)A.d_in - 1u) : col;
          v = __builtin_bit_cast(_Float16, A.X[(int64_t)(m0 + m) * A.ldx + src]);
        }
        xs[m * xstride + p] = v;
      }
    }
  }
  __syncthreads();

  float4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  const bool row_ok = wrow < A.d_out;  // padded rows decode to zero weights anyway
  const uint32_t laneoff = (uint32_t)(lane & 15) * 16u;
  for (int k = 0; k < ngl; ++k) {
    const uint8_t* blk = A.packed + ((int64_t)rt * A.ng + g0 + k) * kBlockBytes;
    const uint8_t* plane = blk + (u < 2 ? kPlaneA : kPlaneB);
    const uint2 pp = *reinterpret_cast<const uint2*>(plane + wrow_in_tile * 16 + (u & 1) * 8);
    const uint2 side = *reinterpret_cast<const uint2*>(blk + kSidePlane + wrow_in_tile * 8);
    const float mu = h2f(side.y);
    const float dl = h2f(side.y >> 16);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // subvector 4u + kk of the group: payload dword 2u + kk/2, half a (kk even) or b (kk odd)
      const uint32_t P = (kk < 2) ? pp.x : pp.y;
      const int pair = 2 * u + (kk >> 1);
      uint32_t s, f;
      if ((kk & 1) == 0) {
        s = ((P >> 4) & 15u) | ((P >> 28) << 4);
        f = (P >> 8) & 1023u;
      } else {
        s = (P & 15u) | (((side.x >> (4 * pair)) & 15u) << 4);
        f = (P >> 18) & 1023u;
      }
      const uint32_t z = f & (kK - 1u);
      const float r = fmaf((float)(f >> L), dl, mu);
      const _Float16 rh = (_Float16)r;
      const half2_t r2 = half2_t{rh, rh};
      const uint4 c = *reinterpret_cast<const uint4*>(cb + z * 256 + laneoff);
      const uint2 mlo = smask[s & 15u];
      const uint2 mhi = smask[s >> 4];
      uint32_t w[4];
      w[0] = mul_pair(c.x ^ mlo.x, r2);
      w[1] = mul_pair(c.y ^ mlo.y, r2);
      w[2] = mul_pair(c.z ^ mhi.x, r2);
      w[3] = mul_pair(c.w ^ mhi.y, r2);
      if (!row_ok) w[0] = w[1] = w[2] = w[3] = 0u;
      const half8_t b = __builtin_bit_cast(half8_t, make_uint4(w[0], w[1], w[2], w[3]));
      const int xcol = k * kGroupCols + (4 * u + kk) * 8;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const half8_t a = *reinterpret_cast<const half8_t*>(xs + (t * 16 + j) * xstride + xcol);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
      }
    }
  }

  // D layout: lane holds column j (weight row) and activation rows 4u .. 4u+3 of each 16-row tile.
  const int64_t rows_pad = (int64_t)A.rt * kTileRows;
  if (A.S == 1) {
    if (row_ok) {
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
  // split-K: partial[mchunk][split][m][rows_pad]
  float* part = A.partial + (int64_t)mchunk * A.S * A.mrows_chunk * rows_pad;
  if (row_ok) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = t * 16 + 4 * u + r;
        if (m < mrows)
          store_coherent(part + ((int64_t)split * A.mrows_chunk + m) * rows_pad + wrow, acc[t][r]);
      }
  }
  wait_stores();
  __syncthreads();
  uint32_t* flag = reinterpret_cast<uint32_t*>(smem);
  uint32_t* counter = A.counters + (int64_t)mchunk * A.rt + rt;
  if (tid == 0) *flag = (counter_add(counter) == (uint32_t)(A.S - 1)) ? 1u : 0u;
  __syncthreads();
  if (*flag == 0u) return;
  // last workgroup: reduce this row tile for all rows of the chunk. Thread t owns elements
  // t + 256 i (activation row 4 i + t / 64, tile row t % 64); the partials of four splits are in
  // flight at a time and summed in split order.
  constexpr int kPer = NT * 16 * kTileRows / kGemmThreads;
  const int trow = rt * kTileRows + (tid & 63);
  const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(
      part, (uint32_t)((int64_t)A.S * A.mrows_chunk * rows_pad * (int64_t)sizeof(float)));
  float sum[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) sum[i] = 0.0f;
  for (int sp0 = 0; sp0 < A.S; sp0 += 4) {
    float v[4][kPer];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int m = 4 * i + (tid >> 6);
        const int sp = min(sp0 + q, A.S - 1);
        v[q][i] = load_coherent_at(
            rs, (uint32_t)((((int64_t)sp * A.mrows_chunk + m) * rows_pad + trow) * sizeof(float)));
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (sp0 + q < A.S) sum[i] += v[q][i];
  }
  if (trow < A.d_out) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = 4 * i + (tid >> 6);
      if (m < mrows) A.Y[(int64_t)(m0 + m) * A.ldy + trow] = f2h(sum[i]);
    }
  }
  if (tid == 0) counter_reset(counter);
}

template <int NT>
__global__ void __launch_bounds__(kGemmThreads) gemm_kernel(GemmArgs A) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int per_chunk = A.rt * A.S;
  const int mchunk = blockIdx.x / per_chunk;
  const int local = blockIdx.x - mchunk * per_chunk;
  const int rt = local / A.S;
  const int split = local - rt * A.S;
  switch (A.L) {
    case 4: gemm_body<4, NT>(A, rt, split, mchunk, smem); break;
    case 5: gemm_body<5, NT>(A, rt, split, mchunk, smem); break;
    case 6: gemm_body<6, NT>(A, rt, split, mchunk, smem); break;
    case 7: gemm_body<7, NT>(A, rt, split, mchunk, smem); break;
    default: gemm_body<8, NT>(A, rt, split, mchunk, smem); break;
  }
}

int tiles_for(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

constexpr size_t kLdsLimit = 160 * 1024;

size_t lds_for(int L, int nt, int gs) {
  return ((size_t)1 << L) * 256 + 128 + (size_t)nt * 16 * ((size_t)gs * kGroupCols + 8) * 2;
}

void plan(GemmArgs& A, int M) {
  A.rt = ceil_div(A.d_out, kTileRows);
  A.ng = A.d_in / kGroupCols;
  A.mrows_chunk = 16 * tiles_for(M);
  A.mchunks = ceil_div(M, A.mrows_chunk);
  // about 2 workgroups per compute unit in total
  const int64_t target = (int64_t)device_cu_count() * 2;
  int64_t s = target / ((int64_t)A.rt * A.mchunks);
  if (s < 1) s = 1;
  if (s > A.ng) s = A.ng;
  A.gs = ceil_div(A.ng, (int)s);
  if (A.gs > kMaxGS) A.gs = kMaxGS;
  // keep the codebook replicas plus the activation tile small enough for two workgroups per CU
  while (A.gs > 1 && lds_for(A.L, tiles_for(M), A.gs) > kLdsLimit / 2) --A.gs;
  A.S = ceil_div(A.ng, A.gs);
}

size_t permuted_bytes(int M, int d_in) {
  return M >= kPermuteMinRows ? ((size_t)M * d_in * 2 + 255) / 256 * 256 : 0;
}

size_t workspace_for(const GemmArgs& A) {
  const size_t xp = permuted_bytes(A.M, A.d_in);
  if (A.S == 1) return xp;
  const size_t part = (size_t)A.mchunks * A.S * A.mrows_chunk * A.rt * kTileRows * 4;
  const size_t cnt = (size_t)A.mchunks * A.rt * 4;
  return xp + (part + cnt + 255) / 256 * 256;
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
  int st = check_matrix(m);
  if (st != SAGE_OK) return st;
  if (X == nullptr || Y == nullptr) return SAGE_ERR_NULL;
  if (M < 1 || ldx < m->d_in || ldy < m->d_out) return SAGE_ERR_SHAPE;
  if (!aligned(X, 4) || !aligned(Y, 2) || (ldx & 1)) return SAGE_ERR_ALIGN;
  if (M == 1) return sage_gemv(m, X, Y, ws, ws_bytes, stream);
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
  if (need) {
    if (ws == nullptr || ws_bytes < need) return SAGE_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return SAGE_ERR_ALIGN;
  }
  char* wsb = static_cast<char*>(ws);
  if (A.S > 1) {
    A.partial = reinterpret_cast<float*>(wsb + xp_bytes);
    A.counters = reinterpret_cast<uint32_t*>(
        wsb + xp_bytes + (size_t)A.mchunks * A.S * A.mrows_chunk * A.rt * kTileRows * 4);
  }
  hipStream_t hs = (hipStream_t)stream;
  if (xp_bytes) {
    // reorder the activations once, then every workgroup reads contiguous 16-byte chunks
    uint16_t* Xp = reinterpret_cast<uint16_t*>(wsb);
    const int64_t n = (int64_t)M * A.d_in;
    hipLaunchKernelGGL(permute_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, hs,
                       X, (int64_t)ldx, m->pi, A.d_in, M, Xp);
    A.X = Xp;
    A.ldx = A.d_in;
    A.pi = nullptr;
    A.vec_x = 1;
  } else {
    A.vec_x = (A.pi == nullptr && aligned(X, 16) && (ldx % 8) == 0) ? 1 : 0;
  }
  const int nt = tiles_for(M);
  const size_t lds = lds_for(A.L, nt, A.gs);
  const unsigned grid = (unsigned)(A.mchunks * A.rt * A.S);
  auto launch = [&](auto kern) {
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      attr = true;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemmThreads), lds, hs, A);
  };
  if (nt == 1) launch(gemm_kernel<1>);
  else if (nt == 2) launch(gemm_kernel<2>);
  else launch(gemm_kernel<4>);
  return hip_status();
}

}  // extern "C"
