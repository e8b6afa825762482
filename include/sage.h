/*
 * sage.h -- C ABI of libsage, the MI355X (gfx950) decode library for SAGE's 2.25-bit spherical
 * vector-quantised weights.
 *
 * Method: "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World Usability".
 *   - Every row of a d_out x d_in weight is cut into subvectors of 8 consecutive weights along the
 *     input axis (§3.1). A subvector stores 8 sign bits, a log2(K)-bit index z into a per-matrix
 *     codebook of K nonnegative unit directions, and a V-bit radius code q (§3.1, Eq. (3):
 *     8 + log2(K) + V = 18 bits).
 *   - Every 128 weights of a row (16 consecutive subvectors) share an fp16 radius grid, offset mu
 *     and step delta; the decoded radius is mu + q*delta (§3.1 Eq. (2); fp16 grid: App. A.6).
 *   - The decoded weight is radius * (signs (.) c_z) (§3.1 Eq. (1)).
 *   - Columns are stored in the ESG-permuted order pi (§3.2 Eq. (5)); at inference the input
 *     vector is gathered through pi (§3.2, §3.5).
 *   - The supported (K, V) splits are the five with log2(K) + V = 10 and 16 <= K <= 256 (the
 *     paper's ABS candidates (64,4), (128,3), (256,2) of §3.3 Eq. (7), plus (16,6) and (32,5)).
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers owned by the caller; the library never allocates,
 *     frees or retains them. Host pointers are only the descriptor arguments (sage_matrix_t*,
 *     size_t*), read before the call returns.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream). Buffers must
 *     stay valid until the work queued on that stream has completed. No call synchronises.
 *   - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *   - Field arrays use permuted column order (the order of storage); x and y use original order.
 *   - Return value: SAGE_OK (0) or one of the error codes below. Arguments are validated on the
 *     host before anything is queued; an invalid call queues nothing. Data-dependent faults
 *     (idx >= K, an out-of-range permutation entry or expert id) are not checked on the device
 *     and give undefined results.
 *   - Thread safety: calls may be made from several host threads. Calls that overlap on the same
 *     stream run in order; concurrent calls that share an output or workspace buffer race (the
 *     no-allocation entry point's fixed workspace is shared by all its calls on a device).
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* sage_stream_t; /* a hipStream_t */

enum sage_status {
  SAGE_OK = 0,
  SAGE_ERR_NULL = 1,      /* a required pointer argument is NULL */
  SAGE_ERR_SHAPE = 2,     /* d_out < 1, d_in < 128, d_in % 128 != 0, M < 1, bad leading dims */
  SAGE_ERR_SPLIT = 3,     /* log2K outside [4, 8] or log2K + V != 10 */
  SAGE_ERR_ALIGN = 4,     /* a pointer does not have the alignment stated for it */
  SAGE_ERR_WORKSPACE = 5, /* workspace pointer NULL or smaller than required */
  SAGE_ERR_HIP = 6,       /* the HIP runtime reported an error while queueing */
  SAGE_ERR_ARG = 7,       /* any other invalid argument (counts, strides, ids) */
  SAGE_ERR_SCRATCH = 8    /* the problem needs more than the no-allocation entry point's fixed
                             scratch (SAGE_NOALLOC_SCRATCH_BYTES) */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char* sage_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH; packed-format version as a separate number.
 * A packed buffer written by one format version is only readable by the same version. */
int sage_version(void);
int sage_format_version(void);

/* sha256 prefix (16 hex digits) of the library's sources as built (static storage), so a result
 * can name the exact sources it was measured on. */
const char* sage_source_digest(void);

/*
 * A quantised matrix as the decode kernels read it.
 *   d_out, d_in  weight shape (rows are outputs); d_in is a multiple of 128.
 *   log2K, V     the split: K = 2^log2K codewords, V radius bits, log2K + V = 10.
 *   packed       device buffer written by sage_pack (payload + fp16 grids), 256-byte aligned,
 *                sage_packed_bytes() bytes.
 *   codebook     device fp16 [K][8], codeword k at codebook + 8k, 16-byte aligned.
 *   pi           device int32 [d_in]: pi[p] is the original input channel at permuted position p
 *                (the gather form of §3.2 Eq. (5)). NULL means the identity permutation.
 * The struct is plain data and may also live in device memory (see sage_moe_gemv).
 */
typedef struct sage_matrix {
  int32_t d_out;
  int32_t d_in;
  int32_t log2K;
  int32_t V;
  const void* packed;
  const uint16_t* codebook;
  const int32_t* pi;
} sage_matrix_t;

/* Bytes of the packed buffer for a matrix (host only; no device work). */
int sage_packed_bytes(int d_out, int d_in, int log2K, int V, size_t* bytes);

/*
 * sage_pack: re-lay the separate code fields of a matrix into the packed streaming layout.
 *   signs  uint8 [d_out][d_in/8]   bit i set <=> weight i of the subvector is negative (§3.1)
 *   idx    uint8 [d_out][d_in/8]   codeword index z, must be < K (§3.1, Eq. (1))
 *   rcode  uint8 [d_out][d_in/8]   radius code q, must be < 2^V (§3.1, Eq. (2))
 *   mu     fp16  [d_out][d_in/128] grid offset per 128-weight group (§3.1 Eq. (2), App. A.6)
 *   delta  fp16  [d_out][d_in/128] grid step per 128-weight group
 *   packed output, 256-byte aligned, sage_packed_bytes() bytes; fully overwritten (row padding
 *          included).
 * Bits of idx/rcode above log2K / V are ignored.
 */
int sage_pack(const uint8_t* signs, const uint8_t* idx, const uint8_t* rcode, const uint16_t* mu,
              const uint16_t* delta, int d_out, int d_in, int log2K, int V, void* packed,
              sage_stream_t stream);

/* sage_unpack: the exact inverse of sage_pack, writing the same five field arrays. */
int sage_unpack(const void* packed, int d_out, int d_in, int log2K, int V, uint8_t* signs,
                uint8_t* idx, uint8_t* rcode, uint16_t* mu, uint16_t* delta, sage_stream_t stream);

/*
 * sage_dequant: dense fp16 copy of the decoded weights (a QDQ reference), original column order.
 *   w  fp16 [d_out][d_in], row-major, 4-byte aligned. Each entry is the decoded weight
 *      (mu + q*delta) * (+-c_z,i) of §3.1 Eq. (1)-(2) rounded once to nearest-even fp16, scattered
 *      to column pi[p] (§3.2).
 */
int sage_dequant(const sage_matrix_t* m, uint16_t* w, sage_stream_t stream);

/*
 * sage_gemv: y = W_hat x for one input vector (batch one), the decode step of §3.5 / App. A.1.
 *   x   fp16 [d_in], 4-byte aligned: original channel order (gathered through pi inside the
 *       call, §3.5 eager decoding), or stored order when the descriptor's pi is NULL (the input's
 *       producer applied the permutation, §3.5 compiled decoding).
 *   y   fp16 [d_out], 2-byte aligned; written, not accumulated.
 *   ws  unused (the product needs no workspace; sage_gemv_workspace_bytes() reports 0); may be
 *       NULL.
 * d_in is at most 32768 (16384 when pi is not NULL); larger inputs return SAGE_ERR_SHAPE.
 * Accumulation is fp32; the result is rounded once to fp16. Repeated calls give the same bits.
 */
int sage_gemv_workspace_bytes(const sage_matrix_t* m, size_t* bytes);
int sage_gemv(const sage_matrix_t* m, const uint16_t* x, uint16_t* y, void* ws, size_t ws_bytes,
              sage_stream_t stream);

/*
 * sage_gemv_multi: up to 16 independent products y_j = W_j x_j in one launch (for example the
 * q/k/v or gate/up projections that read the same input). mats, xs and ys are HOST arrays of
 * n entries; the pointers inside are device pointers with the alignments of sage_gemv. No
 * workspace is used (the *_workspace_bytes query reports 0; ws may be NULL).
 */
int sage_gemv_multi_workspace_bytes(const sage_matrix_t* mats, int n, size_t* bytes);
int sage_gemv_multi(const sage_matrix_t* mats, const uint16_t* const* xs, uint16_t* const* ys,
                    int n, void* ws, size_t ws_bytes, sage_stream_t stream);

/*
 * sage_gemm_small: Y = X W_hat^T for a few activation rows (the small-batch / prefill path of
 * §3.5 and App. A.1, where each decoded weight is reused across the rows).
 *   X   fp16 [M][ldx] row-major, original channel order, ldx >= d_in, ldx even, 4-byte aligned.
 *   Y   fp16 [M][ldy] row-major, ldy >= d_out.
 *   M   >= 1. M = 1 runs the batch-one kernel; up to about a hundred rows a small-batch kernel
 *       (one decode feeds 16-64 rows); larger batches run the prefill kernel, which decodes each
 *       weight once per 64, 128 or 256 rows and, on grids narrower than the device, splits the
 *       column groups and adds the splits in a second kernel (deterministic order).
 *   ws  as for sage_gemv, size from sage_gemm_small_workspace_bytes(); from 8 rows on it also
 *       holds X in permuted column order (written by the call) and the split partial sums.
 *       When the matrix has pi = NULL (X already in stored column order, e.g. written permuted
 *       by its producer) and X is 16-byte aligned with ldx a multiple of 8, X is read in place
 *       and no reorder runs. The workspace must be zero-filled before its first use; every call
 *       leaves it ready for the next call with the same d_out, d_in and M (where the arrival
 *       counters sit depends on them: zero it again before using it for another shape or M).
 *       Calls that share a workspace must not overlap.
 */
int sage_gemm_small_workspace_bytes(const sage_matrix_t* m, int M, size_t* bytes);
int sage_gemm_small(const sage_matrix_t* m, const uint16_t* X, int M, int ldx, uint16_t* Y,
                    int ldy, void* ws, size_t ws_bytes, sage_stream_t stream);

/*
 * sage_gemm_small_noalloc: sage_gemm_small for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same product,
 * arguments, kernels and results as sage_gemm_small, with no workspace argument: the workspace is
 * a fixed array of SAGE_NOALLOC_SCRATCH_BYTES (16 MiB) in the library's device code, one copy per
 * device, held from the library's first use on that device until the process ends. The call
 * allocates nothing (no hipMalloc or hipFree, no allocating library routine); on its first use on
 * a device it looks up that device's copy of the array.
 *   Limit: problems whose sage_gemm_small_workspace_bytes() exceeds SAGE_NOALLOC_SCRATCH_BYTES
 *   return SAGE_ERR_SCRATCH and queue nothing. Every Qwen3-4B-sized projection (d_out, d_in up
 *   to 19456 x 2560 and 2560 x 9728) fits up to M = 64; prefill-sized M may not.
 *   The array keeps the previous call's contents; each call zeroes what must start at zero (the
 *   split-K arrival counters, by a kernel on `stream`) before its product.
 *   All calls on one device share its array: calls that overlap in time on one device (other
 *   streams, other host threads) race and give undefined results. Calls queued on one stream run
 *   in order and are safe.
 */
#define SAGE_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
int sage_gemm_small_noalloc(const sage_matrix_t* m, const uint16_t* X, int M, int ldx, uint16_t* Y,
                            int ldy, sage_stream_t stream);

/*
 * sage_moe_gemv: batch-one products of the routed experts of a mixture-of-experts layer in one
 * launch. The paper evaluates mixture-of-experts models (Qwen3-30B-A3B) but describes no expert
 * kernel; this is the batch-one product above applied to each routed expert's own matrix.
 *   experts_dev  DEVICE array [n_experts] of sage_matrix_t (8-byte aligned): expert e's matrix,
 *                with its own shape, split, codebook, pi and packed buffer (all read on the
 *                device). d_in at most 32768 (16384 with a pi).
 *   ids_dev      DEVICE int32 [n_sel], 4-byte aligned: the routed experts, each in [0, n_experts).
 *   x, x_stride  slot s reads x + s*x_stride (x_stride in elements, even; 0 = one input shared by
 *                every slot, e.g. the token for the gate/up projections). 4-byte aligned.
 *   y, y_stride  slot s writes y + s*y_stride (d_out of its expert values); y_stride >= every
 *                selected expert's d_out when n_sel > 1. 2-byte aligned.
 * A slot whose id is out of range, or whose descriptor has an invalid shape or split, is skipped:
 * its output is not written. The router's weighted combine stays with the caller. No workspace.
 * Errors: SAGE_ERR_NULL, SAGE_ERR_ALIGN, SAGE_ERR_ARG (n_experts, n_sel < 1, bad strides),
 * SAGE_ERR_HIP.
 */
int sage_moe_gemv(const sage_matrix_t* experts_dev, int n_experts, const int32_t* ids_dev,
                  int n_sel, const uint16_t* x, int64_t x_stride, uint16_t* y, int64_t y_stride,
                  sage_stream_t stream);

/*
 * sage_moe_gemv_grouped: sage_moe_gemv over n_mats (1..4) matrices per expert in one launch, for
 * example an expert's gate and up projections on the shared token. experts_dev holds
 * [n_experts * n_mats] descriptors, expert e's matrix j at e*n_mats + j; xs, ys, x_strides and
 * y_strides are HOST arrays [n_mats] giving matrix j's input and output as x and y above.
 */
int sage_moe_gemv_grouped(const sage_matrix_t* experts_dev, int n_experts, int n_mats,
                          const int32_t* ids_dev, int n_sel, const uint16_t* const* xs,
                          const int64_t* x_strides, uint16_t* const* ys, const int64_t* y_strides,
                          sage_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * sage_stream_read: measurement helper, not part of the decode path. Reads `bytes` bytes at `p`
 * once, in one launch, with the same 16-byte non-temporal buffer loads the decode kernels use for
 * packed weights, and writes nothing unless the data XOR-reduces to a fixed improbable value (then
 * one uint32 goes to *sink). Its time is the floor a single streaming launch of that size can
 * reach on this device (launch, wave dispatch and first-data latency included), the reference
 * against which the decode kernels' launch times are read.
 *   p      device buffer, 16-byte aligned; bytes a multiple of 16 (0 launches nothing).
 *   sink   device uint32 [1].
 * Errors: SAGE_ERR_NULL, SAGE_ERR_ALIGN (p not 16-byte aligned or bytes % 16 != 0), SAGE_ERR_HIP.
 */
int sage_stream_read(const void* p, size_t bytes, uint32_t* sink, sage_stream_t stream);

/*
 * Permuting producers (the compiled-decoding mode of §3.5: the next projection's input
 * permutation is fused into the normalization or activation that produces its input). Their
 * output is in the stored column order of a matrix whose pi is given here, so that matrix is then
 * used with pi = NULL (its descriptor's pi set to NULL), which skips the gather in sage_gemv and
 * the reorder in sage_gemm_small. pi NULL here gives the plain operation.
 *   M rows (1 .. 65535) of d channels (d a multiple of 8); row m of an input starts at
 *   element m*ld; row m of out at m*ldo (ld, ldo >= d). fp16 arrays 2-byte aligned (16-byte
 *   aligned out with ldo % 8 == 0 gets vector stores), pi 4-byte aligned. out must not overlap
 *   the inputs.
 *
 * sage_rmsnorm_permute: out[m][p] = fp16( X[m][c] / sqrt(mean_k X[m][k]^2 + eps) * gamma[c] ),
 *   c = pi[p]; gamma fp16 [d] in original channel order; eps >= 0. The mean is over all d
 *   channels, summed in fp32 in a fixed order; one rounding to fp16.
 * sage_silu_mul_permute: out[m][p] = fp16( silu(G[m][c]) * U[m][c] ), c = pi[p],
 *   silu(t) = t / (1 + e^-t); G and U share the row stride ld. fp32 arithmetic, one rounding.
 */
int sage_rmsnorm_permute(const uint16_t* X, int M, int d, int64_t ldx, const uint16_t* gamma,
                         float eps, const int32_t* pi, uint16_t* out, int64_t ldo,
                         sage_stream_t stream);
int sage_silu_mul_permute(const uint16_t* G, const uint16_t* U, int M, int d, int64_t ld,
                          const int32_t* pi, uint16_t* out, int64_t ldo, sage_stream_t stream);

/*
 * sage_encode_fields: the code fields of a matrix for a GIVEN codebook, permutation and position
 * weights (the encoder's final assignment; the codebook fit itself is not done here).
 *   W        fp32 [d_out][ldw] row-major, original column order, 4-byte aligned (ldw >= d_in).
 *   pi       int32 [d_in], gather form as in sage_matrix_t (NULL = identity), 16-byte aligned.
 *   omega    float64 [d_in], the position weights of §3.2 Eq. (4) in permuted order (omega[8j+i]
 *            weighs position i of column subvector j), 8-byte aligned.
 *   codebook fp16 [K][8], K = 2^log2K; (log2K, V) as for every matrix.
 *   signs, idx, rcode  uint8 [d_out][d_in/8] and mu, delta fp16 [d_out][d_in/128]: written in the
 *            layout sage_pack reads.
 *   overflow optional uint32 counter in device memory (NULL = none): incremented once for every
 *            group whose fp16 mu or delta is not finite (weights beyond the fp16 range); the
 *            caller clears it.
 * For subvector j of row r, with w the weights W[r, pi[8j+i]] and p = |w|: the sign bits are
 * w_i < 0 (bit i; a zero weight is positive), z is the first maximum over codewords k of
 * (sum_i omega_i p_i c_ki)^2 / sum_i omega_i c_ki^2 (§3.2 Eq. (6); 0 where the denominator is 0)
 * and the fitted radius r~ = num_z / den_z. Per 128-weight group, mu = min r~ and delta =
 * (max r~ - mu) / (2^V - 1) (§3.1 Eq. (2), App. A.6 Eq. (14)) are rounded to fp16 and
 * q = clip(rint((r~ - mu16) / delta16), 0, 2^V - 1), q = 0 where delta16 = 0. Everything is
 * computed in float64, sums left to right (i = 0..7) without fused multiply-adds, so the result is
 * reproducible bit for bit by any implementation that follows the same order.
 */
int sage_encode_fields(const float* W, int d_out, int d_in, int64_t ldw, const int32_t* pi,
                       const double* omega, const uint16_t* codebook, int log2K, int V,
                       uint8_t* signs, uint8_t* idx, uint8_t* rcode, uint16_t* mu, uint16_t* delta,
                       uint32_t* overflow, sage_stream_t stream);

/*
 * sage_abs_score: the energy-weighted relative reconstruction error of one encoding, §3.3
 * Eq. (8): sum_c e_c ||W[:,c] - W_hat[:,c]||^2 / sum_c e_c ||W[:,c]||^2, the score the Adaptive
 * Bit Split minimises over candidate splits (Eq. (9)); W_hat is the float64 decode of the fields
 * (mu + q delta) * (+-c_z) placed at original column pi[p].
 *   W, ldw, pi, fields, codebook, log2K, V  as for sage_encode_fields (pi 4-byte aligned here).
 *   e        float64 [d_in] channel energies in ORIGINAL column order, 8-byte aligned.
 *   out      float64 [3] in device memory: numerator, denominator, ratio (0 if the denominator is 0).
 *   ws       workspace of sage_abs_score_workspace_bytes() bytes, 8-byte aligned: per-workgroup
 *            partial sums, added in a fixed order (the result does not depend on scheduling).
 */
int sage_abs_score_workspace_bytes(int d_out, int d_in, size_t* bytes);
int sage_abs_score(const float* W, int d_out, int d_in, int64_t ldw, const double* e,
                   const uint8_t* signs, const uint8_t* idx, const uint8_t* rcode,
                   const uint16_t* mu, const uint16_t* delta, const uint16_t* codebook,
                   int log2K, int V, const int32_t* pi, double* out, void* ws, size_t ws_bytes,
                   sage_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H */
