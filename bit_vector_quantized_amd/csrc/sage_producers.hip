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
constexpr int kProdLdsMax = 60 * 1024;  // rows up to 30720 channels are staged in LDS

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

// One workgroup per row. The row is staged in LDS (when it fits) while the sum of squares is
// taken in a fixed order: each thread over its strided elements, then the 256 partial sums by a
// tree in LDS.
__global__ void __launch_bounds__(kProdThreads) rmsnorm_permute_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    const int32_t* __restrict__ pi, int d, uint16_t* __restrict__ out, int64_t ldo, int staged,
    int vec) {
#pragma clang fp contract(off)
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float red[kProdThreads];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  const int tid = threadIdx.x;
  const uint16_t* x = X + (int64_t)blockIdx.x * ldx;
  float ss = 0.0f;
  for (int c = tid; c < d; c += kProdThreads) {
    const uint16_t b = x[c];
    if (staged) xs[c] = b;
    const float v = h2f(b);
    ss = ss + v * v;
  }
  red[tid] = ss;
  __syncthreads();
  for (int h = kProdThreads / 2; h > 0; h >>= 1) {
    if (tid < h) red[tid] += red[tid + h];
    __syncthreads();
  }
  const float r = 1.0f / sqrtf(red[0] / (float)d + eps);
  const uint16_t* src = staged ? xs : x;
  uint16_t* o = out + (int64_t)blockIdx.x * ldo;
  for (int p0 = tid * 8; p0 < d; p0 += kProdThreads * 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = channel(pi, p0 + j, d);
      v[j] = h2f(src[c]) * r * h2f(gamma[c]);
    }
    store8(o + p0, v, vec != 0);
  }
}

// Element-wise: thread t of workgroup (bx, m) writes outputs 8 t .. 8 t + 7 of the row's
// 2048-column range bx.
__global__ void __launch_bounds__(kProdThreads) silu_mul_permute_kernel(
    const uint16_t* __restrict__ G, const uint16_t* __restrict__ U, int64_t ld,
    const int32_t* __restrict__ pi, int d, uint16_t* __restrict__ out, int64_t ldo, int vec) {
#pragma clang fp contract(off)
  const int p0 = (blockIdx.x * kProdThreads + threadIdx.x) * 8;
  if (p0 >= d) return;
  const int64_t row = blockIdx.y;
  const uint16_t* g = G + row * ld;
  const uint16_t* u = U + row * ld;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = channel(pi, p0 + j, d);
    const float gv = h2f(g[c]);
    v[j] = gv / (1.0f + expf(-gv)) * h2f(u[c]);
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
  const int staged = (size_t)d * 2 <= (size_t)kProdLdsMax ? 1 : 0;
  const int vec = (aligned(out, 16) && (ldo % 8) == 0) ? 1 : 0;
  hipLaunchKernelGGL(rmsnorm_permute_kernel, dim3((unsigned)M), dim3(kProdThreads),
                     staged ? (size_t)d * 2 : 0, (hipStream_t)stream, X, ldx, gamma, eps, pi, d,
                     out, ldo, staged, vec);
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
  const dim3 grid((unsigned)ceil_div(d, kProdThreads * 8), (unsigned)M);
  hipLaunchKernelGGL(silu_mul_permute_kernel, grid, dim3(kProdThreads), 0, (hipStream_t)stream, G,
                     U, ld, pi, d, out, ldo, vec);
  return hip_status();
}

}  // extern "C"
