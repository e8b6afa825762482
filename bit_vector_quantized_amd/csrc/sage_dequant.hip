// sage_dequant: dense fp16 copy of the decoded weights, in original column order.
//
// Decode per SAGE paper §3.1: radius = mu_g + q * delta_g (Eq. (2), fp16 grid parameters per App.
// A.6), weight_i = radius * (+-1 from sign bit i) * c_{z,i} (Eq. (1)); permuted column p is written
// to original column pi[p] (§3.2). The arithmetic is done in fp64, where it is exact (mu, delta and
// c are fp16 values and q has at most 6 bits), and the result is rounded once to fp16.
#include "sage_internal.hpp"

namespace sage {
namespace {

__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ packed,
                                                      const uint16_t* __restrict__ codebook,
                                                      const int32_t* __restrict__ pi, int d_out,
                                                      int d_in, int L, uint16_t* __restrict__ w) {
  const int m = d_in / 8;
  const int ng = d_in / kGroupCols;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)d_out * m) return;
  const int row = (int)(t / m);
  const int sv = (int)(t % m);
  const int g = sv / kSubPerGroup;
  const int j = sv % kSubPerGroup;
  const int lane = row % kTileRows;
  const uint8_t* b = packed + ((int64_t)(row / kTileRows) * ng + g) * kBlockBytes;
  uint32_t p[8], x, grid, sbyte, z, q;
  read_lane_block(b, lane, p, &x, &grid);
  v3_fields(p, x, j, L, &sbyte, &z, &q);
  const double mu = (double)h2f(grid);
  const double delta = (double)h2f(grid >> 16);
  const double r = mu + (double)q * delta;
  const uint16_t* c = codebook + z * 8;
  uint16_t* wrow = w + (int64_t)row * d_in;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double ci = (double)h2f(c[i]);
    const double wi = r * (((sbyte >> i) & 1u) ? -ci : ci);
    const int p = sv * 8 + i;
    const int col = pi ? (int)min((uint32_t)pi[p], (uint32_t)d_in - 1u) : p;
    wrow[col] = f64_to_f16_rne(wi);
  }
}

}  // namespace
}  // namespace sage

extern "C" int sage_dequant(const sage_matrix_t* m, uint16_t* w, sage_stream_t stream) {
  using namespace sage;
  int st = check_matrix(m);
  if (st != SAGE_OK) return st;
  if (w == nullptr) return SAGE_ERR_NULL;
  if (!aligned(w, 4)) return SAGE_ERR_ALIGN;
  const int64_t threads = (int64_t)m->d_out * (m->d_in / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(dequant_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint8_t*)m->packed, m->codebook, m->pi, m->d_out, m->d_in, m->log2K,
                     w);
  return hip_status();
}
