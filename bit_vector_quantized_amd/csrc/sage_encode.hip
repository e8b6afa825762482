// GPU encoder for a fixed codebook: the final assignment of SAGE §3.2 Eq. (6) and the per-group
// fp16 radius grid of §3.1 Eq. (2) / App. A.6 Eq. (14), plus the energy-weighted reconstruction
// error of §3.3 Eq. (8) that the Adaptive Bit Split ranks candidate splits by.
//
// Every decision (the argmax over codewords, the grid rounding, the radius code) is taken in
// float64 with a fixed evaluation order and without fused operations, so it is reproducible
// operation for operation: t_i = w_i p_i; num_k = t_0 c_k0 + t_1 c_k1 + ... (left to right);
// den_k = w_0 (c_k0 c_k0) + ... (left to right); score_k = (num_k num_k) / den_k, 0 where den_k = 0;
// z = the first maximum; r = num_z / den_z.
#include "sage_internal.hpp"

namespace sage {
namespace {

constexpr int kEncThreads = 256;         // 4 waves; a wave encodes 64 consecutive subvectors of a row

__device__ inline __amdgpu_buffer_rsrc_t enc_view(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

template <int L>
__global__ void __launch_bounds__(kEncThreads) encode_kernel(
    const float* __restrict__ W, int64_t ldw, const int32_t* __restrict__ pi,
    const double* __restrict__ omega, const uint16_t* __restrict__ codebook, int d_in, int V,
    uint8_t* __restrict__ signs, uint8_t* __restrict__ idx, uint8_t* __restrict__ rcode,
    uint16_t* __restrict__ mu_out, uint16_t* __restrict__ delta_out, uint32_t* overflow) {
#pragma clang fp contract(off)
  constexpr int kK = 1 << L;
  __shared__ double cb[kK][8];
  __shared__ double cb2[kK][8];
  const int tid = threadIdx.x;
  for (int e = tid; e < kK * 8; e += kEncThreads) {
    const double c = (double)__builtin_bit_cast(_Float16, codebook[e]);
    cb[e >> 3][e & 7] = c;
    cb2[e >> 3][e & 7] = c * c;
  }
  __syncthreads();

  const int m = d_in >> 3;                       // subvectors per row
  const int row = blockIdx.x;
  const int j = (blockIdx.y * (kEncThreads / 64) + (tid >> 6)) * 64 + (tid & 63);
  // whole groups of 16 lanes are either all inside the row or all past it (m is a multiple of 16)
  if (j >= m) return;

  // the permuted subvector: weights W[row, pi[8j + i]]
  const __amdgpu_buffer_rsrc_t pi_rs = enc_view(pi, pi ? (uint32_t)d_in * 4u : 0u);
  int col[8];
  if (pi) {
    const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pi_rs, j * 32, 0, 0));
    const uint4 b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pi_rs, j * 32 + 16, 0, 0));
    const uint32_t last = (uint32_t)d_in - 1u;
    col[0] = (int)min(a.x, last); col[1] = (int)min(a.y, last);
    col[2] = (int)min(a.z, last); col[3] = (int)min(a.w, last);
    col[4] = (int)min(b.x, last); col[5] = (int)min(b.y, last);
    col[6] = (int)min(b.z, last); col[7] = (int)min(b.w, last);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) col[i] = 8 * j + i;
  }
  const float* wr = W + (int64_t)row * ldw;
  double w[8], p[8], om[8], t[8];
  uint32_t sbits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w[i] = (double)wr[col[i]];
    om[i] = omega[8 * j + i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sbits |= (w[i] < 0.0 ? 1u : 0u) << i;
    p[i] = fabs(w[i]);
    t[i] = om[i] * p[i];
  }

  // Eq. (6): first maximum of the score over the codebook
  double best = -1.0, bnum = 0.0, bden = 0.0;
  int bz = 0;
  for (int k = 0; k < kK; ++k) {
    double num = t[0] * cb[k][0];
    double den = om[0] * cb2[k][0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      num = num + t[i] * cb[k][i];
      den = den + om[i] * cb2[k][i];
    }
    const double score = den > 0.0 ? (num * num) / den : 0.0;
    if (score > best) {
      best = score;
      bz = k;
      bnum = num;
      bden = den;
    }
  }
  const double r = bden > 0.0 ? bnum / bden : 0.0;

  // Eq. (2) / (14): the 16 lanes of a group share mu = min r and delta = (max r - mu) / (2^V - 1),
  // both stored in fp16; the code is taken against the stored values
  double lo = r, hi = r;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    lo = fmin(lo, __shfl_xor(lo, o, 16));
    hi = fmax(hi, __shfl_xor(hi, o, 16));
  }
  const int qmax = (1 << V) - 1;
  const double step = (hi - lo) / (double)qmax;
  const uint16_t mu16 = f64_to_f16_rne(lo);
  const uint16_t de16 = f64_to_f16_rne(step);
  const double mu = (double)__builtin_bit_cast(_Float16, mu16);
  const double de = (double)__builtin_bit_cast(_Float16, de16);
  int q = 0;
  if (de > 0.0) {
    const double v = rint((r - mu) / de);
    q = (int)fmin(fmax(v, 0.0), (double)qmax);
  }
  const int64_t o = (int64_t)row * m + j;
  signs[o] = (uint8_t)sbits;
  idx[o] = (uint8_t)bz;
  rcode[o] = (uint8_t)q;
  if ((tid & 15) == 0) {
    const int64_t g = (int64_t)row * (m >> 4) + (j >> 4);
    mu_out[g] = mu16;
    delta_out[g] = de16;
    if (overflow && !(isfinite(mu) && isfinite(de))) atomicAdd(overflow, 1u);
  }
}

// Eq. (8) partial sums: workgroup b of the grid adds e_c (W - W_hat)^2 and e_c W^2 over its
// elements (row-major over the permuted positions, 256 per thread-round) into part[2b], part[2b+1].
// W_hat at permuted position (r, 8j + i) is (mu + q delta) * (s ? -c : c), the decode of §3.1
// Eq. (1)-(2) in float64, and belongs to original column pi[8j + i].
__global__ void __launch_bounds__(256) abs_partial_kernel(
    const float* __restrict__ W, int64_t ldw, const double* __restrict__ e, int d_out, int d_in,
    const uint8_t* __restrict__ signs, const uint8_t* __restrict__ idx,
    const uint8_t* __restrict__ rcode, const uint16_t* __restrict__ mu,
    const uint16_t* __restrict__ delta, const uint16_t* __restrict__ codebook, int K,
    const int32_t* __restrict__ pi, int64_t per_block, double* __restrict__ part) {
#pragma clang fp contract(off)
  __shared__ double sn[256], sd[256];
  const int tid = threadIdx.x;
  const int64_t total = (int64_t)d_out * d_in;
  const int64_t beg = (int64_t)blockIdx.x * per_block;
  const int64_t end = beg + per_block < total ? beg + per_block : total;
  const int m = d_in >> 3;
  double accn = 0.0, accd = 0.0;
  for (int64_t x = beg + tid; x < end; x += 256) {
    const int r = (int)(x / d_in);
    const int pp = (int)(x - (int64_t)r * d_in);
    const int j = pp >> 3, i = pp & 7;
    const int64_t s = (int64_t)r * m + j;
    const int64_t g = (int64_t)r * (m >> 4) + (j >> 4);
    const uint32_t z = min((uint32_t)idx[s], (uint32_t)K - 1u);
    const double rad = (double)__builtin_bit_cast(_Float16, mu[g]) +
                       (double)rcode[s] * (double)__builtin_bit_cast(_Float16, delta[g]);
    const double c = (double)__builtin_bit_cast(_Float16, codebook[z * 8 + i]);
    const double sc = ((signs[s] >> i) & 1) ? -c : c;
    const double wh = rad * sc;
    const int colm = pi ? (int)min((uint32_t)pi[pp], (uint32_t)d_in - 1u) : pp;
    const double wv = (double)W[(int64_t)r * ldw + colm];
    const double ec = e[colm];
    const double d = wv - wh;
    accn = accn + ec * (d * d);
    accd = accd + ec * (wv * wv);
  }
  sn[tid] = accn;
  sd[tid] = accd;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) {
      sn[tid] = sn[tid] + sn[tid + h];
      sd[tid] = sd[tid] + sd[tid + h];
    }
    __syncthreads();
  }
  if (tid == 0) {
    part[2 * blockIdx.x] = sn[0];
    part[2 * blockIdx.x + 1] = sd[0];
  }
}

// Adds the partial sums in block order (deterministic) and writes out[0] = numerator,
// out[1] = denominator, out[2] = their ratio (0 when the denominator is 0).
__global__ void abs_finish_kernel(const double* __restrict__ part, int nblocks,
                                  double* __restrict__ out) {
#pragma clang fp contract(off)
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double n = 0.0, d = 0.0;
  for (int b = 0; b < nblocks; ++b) {
    n = n + part[2 * b];
    d = d + part[2 * b + 1];
  }
  out[0] = n;
  out[1] = d;
  out[2] = d > 0.0 ? n / d : 0.0;
}

constexpr int kAbsBlocks = 1024;

int abs_blocks(int d_out, int d_in) {
  const int64_t total = (int64_t)d_out * d_in;
  const int64_t per = (total + kAbsBlocks - 1) / kAbsBlocks;
  return (int)((total + per - 1) / per);
}

}  // namespace
}  // namespace sage

using namespace sage;

extern "C" {

int sage_encode_fields(const float* W, int d_out, int d_in, int64_t ldw, const int32_t* pi,
                       const double* omega, const uint16_t* codebook, int log2K, int V,
                       uint8_t* signs, uint8_t* idx, uint8_t* rcode, uint16_t* mu, uint16_t* delta,
                       uint32_t* overflow, sage_stream_t stream) {
  if (!W || !omega || !codebook || !signs || !idx || !rcode || !mu || !delta) return SAGE_ERR_NULL;
  int st = check_shape(d_out, d_in);
  if (st != SAGE_OK) return st;
  st = check_split(log2K, V);
  if (st != SAGE_OK) return st;
  if (ldw < d_in) return SAGE_ERR_SHAPE;
  if (!aligned(W, 4) || !aligned(omega, 8) || !aligned(codebook, 2) ||
      (pi && !aligned(pi, 16)) || !aligned(mu, 2) || !aligned(delta, 2) ||
      (overflow && !aligned(overflow, 4)))
    return SAGE_ERR_ALIGN;
  const int m = d_in / 8;
  const dim3 grid((unsigned)d_out, (unsigned)ceil_div(m, kEncThreads));
  hipStream_t hs = (hipStream_t)stream;
  switch (log2K) {
    case 4: hipLaunchKernelGGL(encode_kernel<4>, grid, dim3(kEncThreads), 0, hs, W, ldw, pi, omega, codebook, d_in, V, signs, idx, rcode, mu, delta, overflow); break;
    case 5: hipLaunchKernelGGL(encode_kernel<5>, grid, dim3(kEncThreads), 0, hs, W, ldw, pi, omega, codebook, d_in, V, signs, idx, rcode, mu, delta, overflow); break;
    case 6: hipLaunchKernelGGL(encode_kernel<6>, grid, dim3(kEncThreads), 0, hs, W, ldw, pi, omega, codebook, d_in, V, signs, idx, rcode, mu, delta, overflow); break;
    case 7: hipLaunchKernelGGL(encode_kernel<7>, grid, dim3(kEncThreads), 0, hs, W, ldw, pi, omega, codebook, d_in, V, signs, idx, rcode, mu, delta, overflow); break;
    default: hipLaunchKernelGGL(encode_kernel<8>, grid, dim3(kEncThreads), 0, hs, W, ldw, pi, omega, codebook, d_in, V, signs, idx, rcode, mu, delta, overflow); break;
  }
  return hip_status();
}

int sage_abs_score_workspace_bytes(int d_out, int d_in, size_t* bytes) {
  if (!bytes) return SAGE_ERR_NULL;
  const int st = check_shape(d_out, d_in);
  if (st != SAGE_OK) return st;
  *bytes = (size_t)abs_blocks(d_out, d_in) * 2 * sizeof(double);
  return SAGE_OK;
}

int sage_abs_score(const float* W, int d_out, int d_in, int64_t ldw, const double* e,
                   const uint8_t* signs, const uint8_t* idx, const uint8_t* rcode,
                   const uint16_t* mu, const uint16_t* delta, const uint16_t* codebook,
                   int log2K, int V, const int32_t* pi, double* out, void* ws, size_t ws_bytes,
                   sage_stream_t stream) {
  if (!W || !e || !signs || !idx || !rcode || !mu || !delta || !codebook || !out)
    return SAGE_ERR_NULL;
  int st = check_shape(d_out, d_in);
  if (st != SAGE_OK) return st;
  st = check_split(log2K, V);
  if (st != SAGE_OK) return st;
  if (ldw < d_in) return SAGE_ERR_SHAPE;
  if (!aligned(W, 4) || !aligned(e, 8) || !aligned(out, 8) || !aligned(mu, 2) ||
      !aligned(delta, 2) || !aligned(codebook, 2) || (pi && !aligned(pi, 4)))
    return SAGE_ERR_ALIGN;
  const int nb = abs_blocks(d_out, d_in);
  if (!ws || ws_bytes < (size_t)nb * 2 * sizeof(double)) return SAGE_ERR_WORKSPACE;
  if (!aligned(ws, 8)) return SAGE_ERR_ALIGN;
  const int64_t total = (int64_t)d_out * d_in;
  const int64_t per = (total + kAbsBlocks - 1) / kAbsBlocks;
  hipStream_t hs = (hipStream_t)stream;
  double* part = static_cast<double*>(ws);
  hipLaunchKernelGGL(abs_partial_kernel, dim3((unsigned)nb), dim3(256), 0, hs, W, ldw, e, d_out,
                     d_in, signs, idx, rcode, mu, delta, codebook, 1 << log2K, pi, per, part);
  hipLaunchKernelGGL(abs_finish_kernel, dim3(1), dim3(64), 0, hs, part, nb, out);
  return hip_status();
}

}  // extern "C"
