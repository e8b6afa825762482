"""Helpers shared by the GPU tests: device upload of seeded fields, fp16 comparisons."""
from __future__ import annotations

import sys

import numpy as np

import bit_vector_quantized_amd as sage


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def field(c, name):
    return c[name] if isinstance(c, dict) else getattr(c, name)


def log2k(c) -> int:
    return int(field(c, "K")).bit_length() - 1


def upload(c, device="cuda"):
    import torch

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return dict(
        signs=t(field(c, "signs")), idx=t(field(c, "idx")), rcode=t(field(c, "rcode")),
        mu=t(np.asarray(field(c, "mu"), np.uint16).view(np.float16)),
        delta=t(np.asarray(field(c, "delta"), np.uint16).view(np.float16)),
        codebook=t(np.asarray(field(c, "codebook"), np.uint16).view(np.float16)),
        pi=t(np.asarray(field(c, "pi"), np.int32)),
    )


def upload_pack(c, device="cuda", identity_pi=False) -> sage.Packed:
    d = upload(c, device)
    L = log2k(c)
    V = int(field(c, "V"))
    return sage.pack(d["signs"], d["idx"], d["rcode"], d["mu"], d["delta"], d["codebook"],
                     None if identity_pi else d["pi"], L, V)


def fp16_ordered(bits: np.ndarray) -> np.ndarray:
    """Map fp16 bit patterns to integers ordered like the values (+0 and -0 both map to 0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(fp16_ordered(a_bits) - fp16_ordered(b_bits))


# ------------------------------------------------------------------------------------------------
# Output bounds. The contract bound is the fixed 2e-3 relative bound; the tight bound is what the
# arithmetic allows, so that one wrong subvector (a wrong codeword index, sign or radius code)
# exceeds it.
# ------------------------------------------------------------------------------------------------

CONTRACT_REL = 2e-3


def half_ulp16(ref):
    """Half an fp16 ulp at |ref| (taken a hair above |ref|, so a result that rounds across a power
    of two is still covered)."""
    mag = (np.abs(np.asarray(ref, np.float64)) * (1.0 + 2.0 ** -9)).astype(np.float16)
    return 0.5 * np.spacing(mag).astype(np.float64)


def batch_one_bounds(c, x, stored_order=False):
    """Reference and bounds of the batch-one kernel's y = W_hat x.

    ref is the float64 product. The tight bound adds, to one fp16 rounding of the output,
      2^-16 * sum |W_hat| |x|   the fp32 accumulation (its typical error grows like sqrt(n) u;
                                2^-16 is far above what the sums here reach and far below what one
                                wrong subvector changes), and
      2^-23 * sum_j (2^(16-L) delta_g + mu_g + r_j) * sum_i |c_z,i x_8j+i|
                                the kernel's radius: it forms r = (2^(16-L) + q) delta +
                                (mu - 2^(16-L) delta) in fp32, so each radius carries up to one
                                fp32 rounding of |mu - 2^(16-L) delta| and one of r.
    x is in original order unless stored_order (the matrix then runs with pi = NULL)."""
    from oracle import decoder
    xf = np.asarray(x, np.float64)
    Wp = decoder.decode_permuted(c)
    xp = xf if stored_order else xf[np.asarray(field(c, "pi"), np.int64)]
    ref = Wp @ xp
    absrow = np.abs(Wp) @ np.abs(xp)
    L = log2k(c)
    C = np.abs(np.asarray(field(c, "codebook"), np.uint16).view(np.float16)
               .astype(np.float64).reshape(-1, 8))
    idx = np.asarray(field(c, "idx"), np.int64)
    m = idx.shape[1]
    xa = np.abs(xp).reshape(m, 8)
    t = np.zeros(idx.shape)
    for i in range(8):
        t += C[idx, i] * xa[None, :, i]
    g = np.arange(m) // 16
    mu = np.asarray(field(c, "mu"), np.uint16).view(np.float16).astype(np.float64)[:, g]
    de = np.asarray(field(c, "delta"), np.uint16).view(np.float16).astype(np.float64)[:, g]
    r = mu + np.asarray(field(c, "rcode"), np.float64) * de
    radius_term = np.sum((2.0 ** (16 - L) * de + mu + r) * t, axis=1)
    tight = half_ulp16(ref) + 2.0 ** -16 * absrow + 2.0 ** -23 * radius_term
    contract = CONTRACT_REL * float(np.max(absrow))
    return ref, tight, contract


def rounded_weight_bounds(c, X):
    """Reference and bounds of the MFMA kernels, which decode each weight to fp16 once (the
    paper's prefill kernel does the same, App. A.1): ref = X RNE16(W_hat)^T in float64. The tight
    bound is one fp16 rounding of the output, 2^-16 sum |X| |W_hat| for the fp32 accumulation, and
    for every weight that lies within 2^-21 (relative) of an fp16 rounding midpoint its rounding
    step times |x|: the kernel rounds the fp32 product r * c (itself within ~2^-23 of the exact
    weight) to fp16, which can land on the other side of such a midpoint."""
    from oracle import decoder
    Xf = np.asarray(X, np.float64)
    Wx = decoder.decode(c)
    W16 = Wx.astype(np.float16)
    W16f = W16.astype(np.float64)
    other = np.where(Wx >= W16f, np.nextafter(W16, np.float16(np.inf)),
                     np.nextafter(W16, np.float16(-np.inf))).astype(np.float64)
    near = np.abs(Wx - 0.5 * (W16f + other)) <= 2.0 ** -21 * np.abs(Wx)
    step = np.where(near, np.abs(other - W16f), 0.0)
    ref = Xf @ W16f.T
    absmat = np.abs(Xf) @ np.abs(Wx).T
    tight = half_ulp16(ref) + 2.0 ** -16 * absmat + np.abs(Xf) @ step.T
    contract = CONTRACT_REL * np.max(absmat, axis=1, keepdims=True)
    return ref, tight, contract
