// Permuting producers for the compiled-decoding mode of SAGE §3.5: the input permutation of the
// next projection is fused into the normalization or activation that produces its input, so the
// product kernels read that input in stored column order (matrix pi = NULL) without a gather.
//   rmsnorm_permute   out[m][p] = fp16( x[m][pi[p]] / sqrt(mean_c x[m][c]^2 + eps) * gamma[pi[p]] )
//   silu_mul_permute  out[m][p] = fp16( silu(g[m][pi[p]]) * u[m][pi[p]] ),  silu(t) = t / (1 + e^-t)
// Arithmetic in fp32 without contraction (every product and sum rounds to fp32), then one
// rounding to fp16.
#include "sage_internal.hpp"

namespace sage {
namespace {

constexpr int kProdThreads = 256;
constexpr int kProdLdsMax = 60 * 1024;  // rows up to 15360 channels are staged in LDS with gamma

// Writes 8 consecutive fp16 outputs, as one 16-byte store when the address allows. The values are
// pinned in fp32 registers first: the compiler otherwise fuses some of the last products with the
// conversion (one rounding instead of two), element by element differently.
__device__ inline void store8(uint16_t* dst, float v[8], bool vec) {
#pragma unroll
  for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(v[j]));
  if (vec) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f2h(v[2 * j]) | ((uint32_t)f2h(v[2 * j + 1]) << 16);
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = f2h(v[j]);
  }
}

__device__ inline int channel(const int32_t* pi, int p, int d) {
  return pi ? (int)min((uint32_t)pi[p], (uint32_t)d - 1u) : p;
}

// One workgroup per row. When the row fits, it is staged in LDS together with gamma (16-byte
// loads when the rows are 16-byte aligned, issued four at a time), and the permutation entries of
// the thread's first two 8-column outputs are loaded at the start, so the gathers after the
// reduction read LDS only. The sum of squares has a fixed order: each thread over its elements
// in index order, a butterfly across the wave, then the four wave sums in wave order.
__global__ void __launch_bounds__(kProdThreads) rmsnorm_permute_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    const int32_t* __restrict__ pi, int d, uint16_t* __restrict__ out, int64_t ldo, int staged,
    int vec_in, int vec) {
#pragma clang fp contract(off)
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float wsum[kProdThreads / 64];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* gs = xs + d;
  const int tid = threadIdx.x;
  const uint16_t* x = X + (int64_t)blockIdx.x * ldx;
  // permutation entries of outputs tid*8 .. +7 and 2048 + tid*8 .. +7 (zeros past the end)
  const __amdgpu_buffer_rsrc_t pi_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(pi), 0, pi ? (uint32_t)d * 4u : 0u, 0x00020000);
  uint4 pv[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t off = (uint32_t)(tid * 8 + i * kProdThreads * 8) * 4u;
    pv[i][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pi_rs, off, 0, 0));
    pv[i][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pi_rs, off + 16u, 0, 0));
  }
  float ss = 0.0f;
  if (vec_in) {
    // range-checked views: a load past the row reads zeros without touching memory, so every load
    // is issued without a branch
    const int n8 = d >> 3;
    const __amdgpu_buffer_rsrc_t x_rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, (uint32_t)d * 2u, 0x00020000);
    const __amdgpu_buffer_rsrc_t g_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(gamma), 0, staged ? (uint32_t)d * 2u : 0u, 0x00020000);
    for (int c0 = tid; c0 < n8; c0 += 4 * kProdThreads) {
      uint4 v[4], g[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t off = (uint32_t)(c0 + k * kProdThreads) * 16u;
        v[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, off, 0, 0));
        g[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(g_rs, off, 0, 0));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = c0 + k * kProdThreads;
        if (c < n8 && staged) {
          *reinterpret_cast<uint4*>(xs + 8 * c) = v[k];
          *reinterpret_cast<uint4*>(gs + 8 * c) = g[k];
        }
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = h2f(w[j]), hi = h2f(w[j] >> 16);
          ss = ss + lo * lo;
          ss = ss + hi * hi;
        }
      }
    }
  } else {
    for (int c = tid; c < d; c += kProdThreads) {
      const uint16_t b = x[c];
      if (staged) {
        xs[c] = b;
        gs[c] = gamma[c];
      }
      const float v = h2f(b);
      ss = ss + v * v;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss = ss + __shfl_xor(ss, o, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  float tot = wsum[0];
#pragma unroll
  for (int w = 1; w < kProdThreads / 64; ++w) tot = tot + wsum[w];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  const uint16_t* src = staged ? xs : x;
  const uint16_t* gsrc = staged ? gs : gamma;
  uint16_t* o = out + (int64_t)blockIdx.x * ldo;
  const uint32_t last = (uint32_t)d - 1u;
  // the first two outputs of the thread use the entries loaded at the start
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p0 = tid * 8 + i * kProdThreads * 8;
    if (p0 < d) {
      const uint32_t e[8] = {pv[i][0].x, pv[i][0].y, pv[i][0].z, pv[i][0].w,
                             pv[i][1].x, pv[i][1].y, pv[i][1].z, pv[i][1].w};
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = pi ? (int)min(e[j], last) : p0 + j;
        v[j] = h2f(src[c]) * r * h2f(gsrc[c]);
      }
      store8(o + p0, v, vec != 0);
    }
  }
  for (int p0 = tid * 8 + 2 * kProdThreads * 8; p0 < d; p0 += kProdThreads * 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = channel(pi, p0 + j, d);
      v[j] = h2f(src[c]) * r * h2f(gsrc[c]);
    }
    store8(o + p0, v, vec != 0);
  }
}

// Thread t of workgroup (bx, m) writes outputs 8 t .. 8 t + 7 of the row's 2048-column range bx.
// When both rows fit, the workgroup first stages G and U of its row in LDS (16-byte loads when
// aligned) while its permutation entries load, so the gather reads LDS.
__global__ void __launch_bounds__(kProdThreads) silu_mul_permute_kernel(
    const uint16_t* __restrict__ G, const uint16_t* __restrict__ U, int64_t ld,
    const int32_t* __restrict__ pi, int d, uint16_t* __restrict__ out, int64_t ldo, int staged,
    int vec) {
#pragma clang fp contract(off)
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* gs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* us = gs + d;
  const int tid = threadIdx.x;
  const int p0 = (blockIdx.x * kProdThreads + tid) * 8;
  const int64_t row = blockIdx.y;
  const uint16_t* g = G + row * ld;
  const uint16_t* u = U + row * ld;
  const __amdgpu_buffer_rsrc_t pi_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(pi), 0, pi ? (uint32_t)d * 4u : 0u, 0x00020000);
  const uint32_t poff = p0 < d ? (uint32_t)p0 * 4u : 0x40000000u;
  const uint4 e0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pi_rs, poff, 0, 0));
  const uint4 e1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pi_rs, poff + 16u, 0, 0));
  if (staged) {
    const int n8 = d >> 3;
    const __amdgpu_buffer_rsrc_t g_rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(g), 0, (uint32_t)d * 2u, 0x00020000);
    const __amdgpu_buffer_rsrc_t u_rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(u), 0, (uint32_t)d * 2u, 0x00020000);
    for (int c0 = tid; c0 < n8; c0 += 4 * kProdThreads) {
      uint4 a[4], b[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t off = (uint32_t)(c0 + k * kProdThreads) * 16u;
        a[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(g_rs, off, 0, 0));
        b[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(u_rs, off, 0, 0));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = c0 + k * kProdThreads;
        if (c < n8) {
          *reinterpret_cast<uint4*>(gs + 8 * c) = a[k];
          *reinterpret_cast<uint4*>(us + 8 * c) = b[k];
        }
      }
    }
    __syncthreads();
  }
  if (p0 >= d) return;
  const uint16_t* gsrc = staged ? gs : g;
  const uint16_t* usrc = staged ? us : u;
  const uint32_t last = (uint32_t)d - 1u;
  const uint32_t e[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = pi ? (int)min(e[j], last) : p0 + j;
    const float gv = h2f(gsrc[c]);
    v[j] = gv / (1.0f + expf(-gv)) * h2f(usrc[c]);
  }
  store8(out + row * ldo + p0, v, vec != 0);
}

int check_producer(int M, int d, int64_t ld_in, int64_t ld_out) {
  if (M < 1 || M > 65535 || d < 8 || (d % 8) != 0 || ld_in < d || ld_out < d) return SAGE_ERR_SHAPE;
  return SAGE_OK;
}

}  // namespace
}  // namespace sage

using namespace sage;

extern "C" {

int sage_rmsnorm_permute(const uint16_t* X, int M, int d, int64_t ldx, const uint16_t* gamma,
                         float eps, const int32_t* pi, uint16_t* out, int64_t ldo,
                         sage_stream_t stream) {
  if (!X || !gamma || !out) return SAGE_ERR_NULL;
  const int st = check_producer(M, d, ldx, ldo);
  if (st != SAGE_OK) return st;
  if (!(eps >= 0.0f)) return SAGE_ERR_ARG;
  if (!aligned(X, 2) || !aligned(gamma, 2) || !aligned(out, 2) || (pi && !aligned(pi, 4)))
    return SAGE_ERR_ALIGN;
  const int staged = (size_t)d * 4 <= (size_t)kProdLdsMax ? 1 : 0;
  const int vec = (aligned(out, 16) && (ldo % 8) == 0) ? 1 : 0;
  const int vec_in = (aligned(X, 16) && (ldx % 8) == 0 && aligned(gamma, 16)) ? 1 : 0;
  hipLaunchKernelGGL(rmsnorm_permute_kernel, dim3((unsigned)M), dim3(kProdThreads),
                     staged ? (size_t)d * 4 : 0, (hipStream_t)stream, X, ldx, gamma, eps, pi, d,
                     out, ldo, staged, vec_in, vec);
  return hip_status();
}

int sage_silu_mul_permute(const uint16_t* G, const uint16_t* U, int M, int d, int64_t ld,
                          const int32_t* pi, uint16_t* out, int64_t ldo, sage_stream_t stream) {
  if (!G || !U || !out) return SAGE_ERR_NULL;
  const int st = check_producer(M, d, ld, ldo);
  if (st != SAGE_OK) return st;
  if (!aligned(G, 2) || !aligned(U, 2) || !aligned(out, 2) || (pi && !aligned(pi, 4)))
    return SAGE_ERR_ALIGN;
  const int vec = (aligned(out, 16) && (ldo % 8) == 0) ? 1 : 0;
  // staging needs both rows in LDS and 16-byte aligned rows
  const int staged = ((size_t)d * 4 <= (size_t)kProdLdsMax && aligned(G, 16) && aligned(U, 16) &&
                      (ld % 8) == 0) ? 1 : 0;
  const dim3 grid((unsigned)ceil_div(d, kProdThreads * 8), (unsigned)M);
  hipLaunchKernelGGL(silu_mul_permute_kernel, grid, dim3(kProdThreads),
                     staged ? (size_t)d * 4 : 0, (hipStream_t)stream, G, U, ld, pi, d, out, ldo,
                     staged, vec);
  return hip_status();
}

}  // extern "C"
