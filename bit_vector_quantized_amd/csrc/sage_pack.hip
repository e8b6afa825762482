// sage_pack / sage_unpack: move the separate code fields of a matrix (SAGE paper §3.1: sign bits,
// codeword index, radius code, and the fp16 grid of every 128-weight group) into and out of the
// packed streaming layout (format version 3) described in sage_internal.hpp.
#include "sage_internal.hpp"

namespace sage {
namespace {

// One thread per (row of the padded row tile, column group); lanes of a wavefront are consecutive
// rows of one block so every plane is written as one contiguous span.
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t* __restrict__ signs,
                                                   const uint8_t* __restrict__ idx,
                                                   const uint8_t* __restrict__ rcode,
                                                   const uint16_t* __restrict__ mu,
                                                   const uint16_t* __restrict__ delta, int d_out,
                                                   int d_in, int L, uint8_t* __restrict__ packed) {
  const int ng = d_in / kGroupCols;
  const int m = d_in / 8;
  const int rt_count = (d_out + kTileRows - 1) / kTileRows;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)rt_count * ng * kTileRows) return;
  const int lane = (int)(t & 63);
  const int64_t blk = t >> 6;
  const int g = (int)(blk % ng);
  const int row = (int)(blk / ng) * kTileRows + lane;
  uint8_t* b = packed + blk * kBlockBytes;

  uint32_t p[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint32_t x = 0, grid = 0;
  if (row < d_out) {
    const size_t off = (size_t)row * m + (size_t)g * kSubPerGroup;
    const uint4 si = *reinterpret_cast<const uint4*>(signs + off);
    const uint4 zi = *reinterpret_cast<const uint4*>(idx + off);
    const uint4 qi = *reinterpret_cast<const uint4*>(rcode + off);
    const uint32_t sw[4] = {si.x, si.y, si.z, si.w};
    const uint32_t zw[4] = {zi.x, zi.y, zi.z, zi.w};
    const uint32_t qw[4] = {qi.x, qi.y, qi.z, qi.w};
    const uint32_t kmask = (1u << L) - 1u;
    const uint32_t vmask = (1u << (10 - L)) - 1u;
    uint32_t sj[kSubPerGroup], zj[kSubPerGroup], qj[kSubPerGroup];
    for (int j = 0; j < kSubPerGroup; ++j) {
      const int sh = 8 * (j & 3);
      sj[j] = (sw[j >> 2] >> sh) & 0xFFu;
      zj[j] = (zw[j >> 2] >> sh) & kmask;
      qj[j] = (qw[j >> 2] >> sh) & vmask;
    }
    for (int i = 0; i < 8; ++i) {
      const int a = 2 * i, bb = 2 * i + 1;
      p[i] = v3_pair(sj[a], zj[a], qj[a], sj[bb], zj[bb], qj[bb], L);
      x |= (sj[a] >> 4) << (4 * i);
    }
    const size_t go = (size_t)row * ng + g;
    grid = (uint32_t)mu[go] | ((uint32_t)delta[go] << 16);
  }
  *reinterpret_cast<uint4*>(b + kPlaneA + lane * 16) = make_uint4(p[0], p[1], p[2], p[3]);
  *reinterpret_cast<uint4*>(b + kPlaneB + lane * 16) = make_uint4(p[4], p[5], p[6], p[7]);
  *reinterpret_cast<uint2*>(b + kSidePlane + lane * 8) = make_uint2(x, grid);
}

__global__ void __launch_bounds__(256) unpack_kernel(const uint8_t* __restrict__ packed, int d_out,
                                                     int d_in, int L, uint8_t* __restrict__ signs,
                                                     uint8_t* __restrict__ idx,
                                                     uint8_t* __restrict__ rcode,
                                                     uint16_t* __restrict__ mu,
                                                     uint16_t* __restrict__ delta) {
  const int ng = d_in / kGroupCols;
  const int m = d_in / 8;
  const int rt_count = (d_out + kTileRows - 1) / kTileRows;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)rt_count * ng * kTileRows) return;
  const int lane = (int)(t & 63);
  const int64_t blk = t >> 6;
  const int g = (int)(blk % ng);
  const int row = (int)(blk / ng) * kTileRows + lane;
  if (row >= d_out) return;
  const uint8_t* b = packed + blk * kBlockBytes;
  uint32_t p[8], x, grid;
  read_lane_block(b, lane, p, &x, &grid);
  uint32_t so[4] = {0, 0, 0, 0}, zo[4] = {0, 0, 0, 0}, qo[4] = {0, 0, 0, 0};
  for (int j = 0; j < kSubPerGroup; ++j) {
    const int sh = 8 * (j & 3);
    uint32_t sv, zv, qv;
    v3_fields(p, x, j, L, &sv, &zv, &qv);
    so[j >> 2] |= sv << sh;
    zo[j >> 2] |= zv << sh;
    qo[j >> 2] |= qv << sh;
  }
  const size_t off = (size_t)row * m + (size_t)g * kSubPerGroup;
  *reinterpret_cast<uint4*>(signs + off) = make_uint4(so[0], so[1], so[2], so[3]);
  *reinterpret_cast<uint4*>(idx + off) = make_uint4(zo[0], zo[1], zo[2], zo[3]);
  *reinterpret_cast<uint4*>(rcode + off) = make_uint4(qo[0], qo[1], qo[2], qo[3]);
  const size_t go = (size_t)row * ng + g;
  mu[go] = (uint16_t)(grid & 0xFFFFu);
  delta[go] = (uint16_t)(grid >> 16);
}

int check_fields(const void* signs, const void* idx, const void* rcode, const void* mu,
                 const void* delta) {
  if (!signs || !idx || !rcode || !mu || !delta) return SAGE_ERR_NULL;
  if (!aligned(signs, 16) || !aligned(idx, 16) || !aligned(rcode, 16) || !aligned(mu, 2) ||
      !aligned(delta, 2))
    return SAGE_ERR_ALIGN;
  return SAGE_OK;
}

}  // namespace
}  // namespace sage

extern "C" {

int sage_pack(const uint8_t* signs, const uint8_t* idx, const uint8_t* rcode, const uint16_t* mu,
              const uint16_t* delta, int d_out, int d_in, int log2K, int V, void* packed,
              sage_stream_t stream) {
  using namespace sage;
  int st = check_shape(d_out, d_in);
  if (st != SAGE_OK) return st;
  if ((st = check_split(log2K, V)) != SAGE_OK) return st;
  if ((st = check_fields(signs, idx, rcode, mu, delta)) != SAGE_OK) return st;
  if (packed == nullptr) return SAGE_ERR_NULL;
  if (!aligned(packed, 256)) return SAGE_ERR_ALIGN;
  const int64_t threads = (int64_t)ceil_div(d_out, kTileRows) * (d_in / kGroupCols) * kTileRows;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, signs, idx,
                     rcode, mu, delta, d_out, d_in, log2K, (uint8_t*)packed);
  return hip_status();
}

int sage_unpack(const void* packed, int d_out, int d_in, int log2K, int V, uint8_t* signs,
                uint8_t* idx, uint8_t* rcode, uint16_t* mu, uint16_t* delta,
                sage_stream_t stream) {
  using namespace sage;
  int st = check_shape(d_out, d_in);
  if (st != SAGE_OK) return st;
  if ((st = check_split(log2K, V)) != SAGE_OK) return st;
  if ((st = check_fields(signs, idx, rcode, mu, delta)) != SAGE_OK) return st;
  if (packed == nullptr) return SAGE_ERR_NULL;
  if (!aligned(packed, 256)) return SAGE_ERR_ALIGN;
  const int64_t threads = (int64_t)ceil_div(d_out, kTileRows) * (d_in / kGroupCols) * kTileRows;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(unpack_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint8_t*)packed, d_out, d_in, log2K, signs, idx, rcode, mu, delta);
  return hip_status();
}

}  // extern "C"
