"""Decoder side of SAGE in float64 (TEST INFRASTRUCTURE ONLY; see oracle/__init__).

Written from "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World Usability":
  radii          §3.1, Eq. (2): the quantised radius is mu_g + q * delta_g, using the stored fp16
                 offset and step of the subvector's 128-weight group (fp16 grid: Appendix A.6).
  decode         §3.1, Eq. (1): each weight is that radius times the signed codeword component;
                 §3.2: the matrix is stored in permuted column order, so permuted column p is
                 written back to original column pi[p].
  dequant_fp16   the decoded weights rounded once, half-to-even, to fp16 (a dense QDQ copy).
  gemv / gemm    y = W_hat x and Y = X W_hat^T in float64 with the fp16 inputs widened exactly.
  moe_gemv       the same product for each routed expert with that expert's own fields.
  tolerance      the output bound used by the parity tests: 2e-3 * max over rows of sum |W_hat||x|.
  silu, swiglu_mlp
                 the SwiGLU feed-forward block of the decoder family the paper evaluates (the
                 paper quantizes these linear layers but does not define the block): the gate and
                 up products rounded to fp16, h = fp16(silu(gate) * up) with silu(t) = t/(1+e^-t),
                 then y = W_down h. Only this composition is new here; each product is gemv above.
  rmsnorm_permute, silu_mul_permute
                 the producers of §3.5's compiled decoding, which fuse each projection's input
                 permutation into the preceding normalization or activation: out[:, p] =
                 f(X)[:, pi[p]] for f = RMSNorm (x / sqrt(mean(x^2) + eps) times a weight gamma,
                 the normalization of the decoder family evaluated; the paper does not define it)
                 or f = silu(g) * u. Returned in float64, before the fp16 rounding a producer
                 applies.

Every step here is exact in float64: mu, delta and codeword entries are fp16 values, q has at most
6 bits, so mu + q*delta and its product with a codeword entry need far fewer than 53 bits.
dequant_fp16 is therefore the correctly rounded fp16 of the exact decoded weight.

Parity status: pinned by the CPU tests (exact recovery of planted matrices, the equal-radii special
case of Appendix A.6, unit-vector probes of the permutation direction and a brute-force loop
matrix-vector product on tiny shapes; silu at closed-form points and the identity
silu(t) - silu(-t) = t; the block's zero-gate and zero-up cases; RMSNorm's unit root-mean-square
output, scale invariance and a hand-worked vector; the producers' permutation as a column gather
checked with unit probes).
"""
from __future__ import annotations

from typing import Any, Dict, Sequence

import numpy as np

V_SUB = 8
G_SUBVECS = 16     # 128-weight groups hold 16 consecutive subvectors of a row (Appendix A.6)


def _get(c: Any, name: str):
    return c[name] if isinstance(c, dict) else getattr(c, name)


def _f16(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def radii(c: Any) -> np.ndarray:
    """Quantised radius of every subvector: [d_out, d_in/8] float64 (Eq. (2))."""
    mu = _f16(_get(c, "mu"))
    delta = _f16(_get(c, "delta"))
    q = np.asarray(_get(c, "rcode"), dtype=np.float64)
    g = np.arange(q.shape[1]) // G_SUBVECS
    return mu[:, g] + q * delta[:, g]


def decode_permuted(c: Any) -> np.ndarray:
    """Decoded weights in stored (permuted) column order: [d_out, d_in] float64 (Eq. (1))."""
    C = _f16(_get(c, "codebook")).reshape(-1, V_SUB)
    idx = np.asarray(_get(c, "idx"), dtype=np.int64)
    s = np.asarray(_get(c, "signs"), dtype=np.uint8)
    K = int(_get(c, "K"))
    if idx.max(initial=0) >= K or C.shape[0] != K:
        raise ValueError("codeword index out of range")
    r = radii(c)
    d_out, m = idx.shape
    sign = np.empty((d_out, m, V_SUB))
    for i in range(V_SUB):
        sign[..., i] = np.where((s >> i) & 1, -1.0, 1.0)
    Wp = r[..., None] * (sign * C[idx])
    return Wp.reshape(d_out, m * V_SUB)


def decode(c: Any) -> np.ndarray:
    """Decoded weights in original column order: W_hat[:, pi[p]] = W_hat_perm[:, p]."""
    Wp = decode_permuted(c)
    pi = np.asarray(_get(c, "pi"), dtype=np.int64)
    if np.any(np.sort(pi) != np.arange(pi.size)):
        raise ValueError("pi is not a permutation")
    W = np.empty_like(Wp)
    W[:, pi] = Wp
    return W


def dequant_fp16(c: Any) -> np.ndarray:
    """fp16 [d_out, d_in] dense copy in original order, rounded half-to-even from the exact decode.
    Returned as uint16 bit patterns."""
    return decode(c).astype(np.float16).view(np.uint16)


def gemv(c: Any, x: np.ndarray) -> np.ndarray:
    """y = W_hat x; x is fp16 [d_in] in original channel order; y float64 [d_out]."""
    return decode(c) @ np.asarray(x, dtype=np.float64)


def gemm(c: Any, X: np.ndarray) -> np.ndarray:
    """Y = X W_hat^T; X is fp16 [M, d_in]; Y float64 [M, d_out]."""
    return np.asarray(X, dtype=np.float64) @ decode(c).T


def moe_gemv(experts: Sequence[Dict[str, Any]], ids: np.ndarray, x: np.ndarray,
             h: np.ndarray) -> Dict[str, np.ndarray]:
    """Grouped product over routed experts: gate/up read the shared x, down reads the routed
    expert's own h row. Returns float64 [top_k, d_out] per matrix name."""
    out = {"gate": [], "up": [], "down": []}
    for s, e in enumerate(np.asarray(ids)):
        ex = experts[int(e)]
        out["gate"].append(gemv(ex["gate"], x))
        out["up"].append(gemv(ex["up"], x))
        out["down"].append(gemv(ex["down"], h[s]))
    return {k: np.stack(v) for k, v in out.items()}


def abs_weighted_sum(c: Any, x: np.ndarray) -> np.ndarray:
    """sum_c |W_hat_rc| |x_c| per output row (float64)."""
    return np.abs(decode(c)) @ np.abs(np.asarray(x, dtype=np.float64))


def tolerance(c: Any, x: np.ndarray, rel: float = 2e-3) -> float:
    """Bound for max |y - y_ref|: rel * max over rows of sum_c |W_hat_rc| |x_c|."""
    return float(rel * np.max(abs_weighted_sum(c, x)))


def silu(t: np.ndarray) -> np.ndarray:
    """t * sigmoid(t) = t / (1 + exp(-t)) in float64."""
    t = np.asarray(t, np.float64)
    return t / (1.0 + np.exp(-t))


def swiglu_mlp(gate: Any, up: Any, down: Any, x: np.ndarray):
    """Returns (h, y): h = fp16(silu(fp16(W_gate x)) * fp16(W_up x)) as float64, y = W_down h."""
    g16 = gemv(gate, x).astype(np.float16).astype(np.float64)
    u16 = gemv(up, x).astype(np.float16).astype(np.float64)
    h = (silu(g16) * u16).astype(np.float16).astype(np.float64)
    return h, decode(down) @ h


def rmsnorm_permute(X: np.ndarray, gamma: np.ndarray, eps: float, pi=None) -> np.ndarray:
    """Rows of X [M, d] (or one vector [d]) normalised by their root mean square and scaled by
    gamma [d], in original channel order; then column p of the result is column pi[p] of that
    (pi None: identity). float64."""
    X = np.asarray(X, np.float64)
    g = np.asarray(gamma, np.float64)
    ms = np.mean(X * X, axis=-1, keepdims=True)
    Y = X / np.sqrt(ms + float(eps)) * g
    return Y if pi is None else Y[..., np.asarray(pi, np.int64)]


def silu_mul_permute(G: np.ndarray, U: np.ndarray, pi=None) -> np.ndarray:
    """silu(G) * U element-wise (G, U: [M, d] or [d], fp16 values widened exactly), then column p of
    the result is column pi[p] (pi None: identity). float64."""
    Y = silu(G) * np.asarray(U, np.float64)
    return Y if pi is None else Y[..., np.asarray(pi, np.int64)]
