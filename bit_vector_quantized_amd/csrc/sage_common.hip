// Host-side helpers of libsage: status text, versions, argument checks, device queries.
#include <mutex>

#include "sage_internal.hpp"

namespace sage {

int check_matrix(const sage_matrix_t* m) {
  if (m == nullptr) return SAGE_ERR_NULL;
  int st = check_shape(m->d_out, m->d_in);
  if (st != SAGE_OK) return st;
  st = check_split(m->log2K, m->V);
  if (st != SAGE_OK) return st;
  if (m->packed == nullptr || m->codebook == nullptr) return SAGE_ERR_NULL;
  if (!aligned(m->packed, 256) || !aligned(m->codebook, 16) || !aligned(m->pi, 4))
    return SAGE_ERR_ALIGN;
  return SAGE_OK;
}

int hip_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace sage

extern "C" {

const char* sage_status_string(int status) {
  switch (status) {
    case SAGE_OK: return "ok";
    case SAGE_ERR_NULL: return "a required pointer is NULL";
    case SAGE_ERR_SHAPE: return "invalid shape (d_out >= 1, d_in a positive multiple of 128, M >= 1, leading dims)";
    case SAGE_ERR_SPLIT: return "invalid split (need 4 <= log2K <= 8 and log2K + V == 10)";
    case SAGE_ERR_ALIGN: return "misaligned pointer";
    case SAGE_ERR_WORKSPACE: return "workspace missing or too small";
    case SAGE_ERR_HIP: return "HIP runtime error while queueing work";
    case SAGE_ERR_ARG: return "invalid argument";
    case SAGE_ERR_SCRATCH: return "problem needs more workspace than the no-allocation entry point's fixed scratch (16 MiB)";
    default: return "unknown status";
  }
}

int sage_version(void) { return 2 * 10000 + 0 * 100 + 0; }

#ifndef SAGE_SOURCE_DIGEST
#define SAGE_SOURCE_DIGEST "unknown"
#endif
const char* sage_source_digest(void) { return SAGE_SOURCE_DIGEST; }

int sage_format_version(void) { return sage::kFormatVersion; }

int sage_packed_bytes(int d_out, int d_in, int log2K, int V, size_t* bytes) {
  if (bytes == nullptr) return SAGE_ERR_NULL;
  int st = sage::check_shape(d_out, d_in);
  if (st != SAGE_OK) return st;
  st = sage::check_split(log2K, V);
  if (st != SAGE_OK) return st;
  *bytes = sage::packed_bytes(d_out, d_in);
  return SAGE_OK;
}

}  // extern "C"
