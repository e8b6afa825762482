// Streaming-read reference: one launch that reads a buffer once with the 16-byte non-temporal
// buffer loads the decode kernels use for packed weights (see sage_stream_read in sage.h).
#include "sage_internal.hpp"

namespace sage {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadPerThread = 16;  // 16-byte loads in flight per thread
constexpr size_t kReadBytesPerWg = (size_t)kReadThreads * kReadPerThread * 16;

__global__ void __launch_bounds__(kReadThreads) stream_read_kernel(const uint8_t* p, size_t bytes,
                                                                   uint32_t* sink) {
  const size_t base = (size_t)blockIdx.x * kReadBytesPerWg;
  const size_t left = bytes - base;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p + base), 0,
      (uint32_t)(left < kReadBytesPerWg ? left : kReadBytesPerWg), 0x00020000);
  u32x4 v[kReadPerThread];
#pragma unroll
  for (int k = 0; k < kReadPerThread; ++k)
    v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (k * kReadThreads + threadIdx.x) * 16, 0, 2);
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < kReadPerThread; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace
}  // namespace sage

using namespace sage;

extern "C" int sage_stream_read(const void* p, size_t bytes, uint32_t* sink,
                                sage_stream_t stream) {
  if (p == nullptr || sink == nullptr) return SAGE_ERR_NULL;
  if (!aligned(p, 16) || bytes % 16 != 0) return SAGE_ERR_ALIGN;
  if (bytes == 0) return SAGE_OK;
  const size_t wgs = (bytes + kReadBytesPerWg - 1) / kReadBytesPerWg;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)wgs), dim3(kReadThreads), 0,
                     (hipStream_t)stream, static_cast<const uint8_t*>(p), bytes, sink);
  return hip_status();
}
