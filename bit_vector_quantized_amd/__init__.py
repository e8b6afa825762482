"""Python binding of libsage, the MI355X decode library for SAGE's 2.25-bit spherical VQ weights.

"SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World Usability" defines the stored fields
(§3.1: sign bits, codeword index, radius code, per-128-weight fp16 grid; §3.2: the ESG permutation)
and the fused decode-and-multiply this library implements on gfx950.

This module only marshals arguments: every step of the computation runs in the HIP kernels behind
the C ABI in include/sage.h. PyTorch is used for device memory and streams. There is no CPU
fallback: if libsage.so has not been built, importing the kernels' entry points raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import List, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsage.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "sage.h")

SAGE_OK = 0


class SageError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


class SageMatrix(ctypes.Structure):
    """Mirror of sage_matrix_t."""

    _fields_ = [
        ("d_out", ctypes.c_int32), ("d_in", ctypes.c_int32),
        ("log2K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("packed", ctypes.c_void_p), ("codebook", ctypes.c_void_p), ("pi", ctypes.c_void_p),
    ]


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_PSZ = ctypes.POINTER(ctypes.c_size_t)
_PM = ctypes.POINTER(SageMatrix)
_PP = ctypes.POINTER(ctypes.c_void_p)
_PI64 = ctypes.POINTER(ctypes.c_int64)

_SIGNATURES = {
    "sage_status_string": (ctypes.c_char_p, [_I]),
    "sage_version": (_I, []),
    "sage_source_digest": (ctypes.c_char_p, []),
    "sage_format_version": (_I, []),
    "sage_packed_bytes": (_I, [_I, _I, _I, _I, _PSZ]),
    "sage_pack": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "sage_unpack": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "sage_dequant": (_I, [_PM, _P, _P]),
    "sage_gemv_workspace_bytes": (_I, [_PM, _PSZ]),
    "sage_gemv": (_I, [_PM, _P, _P, _P, _SZ, _P]),
    "sage_gemv_multi_workspace_bytes": (_I, [_PM, _I, _PSZ]),
    "sage_gemv_multi": (_I, [_PM, _PP, _PP, _I, _P, _SZ, _P]),
    "sage_gemm_small_workspace_bytes": (_I, [_PM, _I, _PSZ]),
    "sage_gemm_small": (_I, [_PM, _P, _I, _I, _P, _I, _P, _SZ, _P]),
    "sage_gemm_small_noalloc": (_I, [_PM, _P, _I, _I, _P, _I, _P]),
    "sage_moe_gemv": (_I, [_PM, _I, _P, _I, _P, ctypes.c_int64, _P, ctypes.c_int64, _P]),
    "sage_moe_gemv_grouped": (_I, [_PM, _I, _I, _P, _I, _PP, _PI64, _PP, _PI64, _P]),
    "sage_stream_read": (_I, [_P, _SZ, _P, _P]),
    "sage_encode_fields": (_I, [_P, _I, _I, ctypes.c_int64, _P, _P, _P, _I, _I,
                                _P, _P, _P, _P, _P, _P, _P]),
    "sage_abs_score_workspace_bytes": (_I, [_I, _I, _PSZ]),
    "sage_rmsnorm_permute": (_I, [_P, _I, _I, ctypes.c_int64, _P, ctypes.c_float, _P, _P,
                                  ctypes.c_int64, _P]),
    "sage_silu_mul_permute": (_I, [_P, _P, _I, _I, ctypes.c_int64, _P, _P, ctypes.c_int64, _P]),
    "sage_abs_score": (_I, [_P, _I, _I, ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P,
                            _P, _P, _SZ, _P]),
}


def lib() -> ctypes.CDLL:
    """The loaded libsage.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_vector_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions() -> List[str]:
    """Names of the functions declared in include/sage.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(sage_\w+)\s*\(", text, flags=re.M)))


def source_digest() -> str:
    """sha256 prefix of the sources the loaded libsage.so was built from."""
    return lib().sage_source_digest().decode()


def status_string(status: int) -> str:
    try:
        return lib().sage_status_string(status).decode()
    except Exception:  # pragma: no cover
        return "?"


def _check(fn: str, st: int) -> None:
    if st != SAGE_OK:
        raise SageError(fn, st)


# ------------------------------------------------------------------------------------------------
# torch glue
# ------------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libsage arguments must be device tensors")


def _require_vec(name: str, t, n: int, dtype_name: str = "float16"):
    """t must be a contiguous device tensor of the given dtype with at least n elements."""
    _require_cuda(t)
    if str(t.dtype) != "torch." + dtype_name:
        raise ValueError(f"{name} must be {dtype_name}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {n}")


def _check_packed(p) -> None:
    """The matrix's own buffers match its shape and split (what the kernels will address)."""
    _require_vec("codebook", p.codebook, 8 * p.K)
    if p.codebook.numel() != 8 * p.K:
        raise ValueError(f"codebook must hold exactly {p.K} x 8 values")
    if p.pi is not None:
        _require_vec("pi", p.pi, p.d_in, "int32")
        if p.pi.numel() != p.d_in:
            raise ValueError(f"pi must hold exactly d_in = {p.d_in} entries")
    need = packed_bytes(p.d_out, p.d_in, p.log2K, p.V)
    if p.packed.numel() * p.packed.element_size() < need:
        raise ValueError(f"packed buffer holds fewer than {need} bytes")


@dataclass
class Packed:
    """A packed matrix resident on the device (owns its buffers)."""

    d_out: int
    d_in: int
    log2K: int
    V: int
    packed: "object"      # torch.uint8 [bytes]
    codebook: "object"    # torch.float16 [K, 8]
    pi: "object"          # torch.int32 [d_in] or None

    def desc(self) -> SageMatrix:
        return SageMatrix(self.d_out, self.d_in, self.log2K, self.V, _ptr(self.packed),
                          _ptr(self.codebook), _ptr(self.pi))

    @property
    def K(self) -> int:
        return 1 << self.log2K


def packed_bytes(d_out: int, d_in: int, log2K: int, V: int) -> int:
    n = ctypes.c_size_t(0)
    _check("sage_packed_bytes", lib().sage_packed_bytes(d_out, d_in, log2K, V, ctypes.byref(n)))
    return n.value


def pack(signs, idx, rcode, mu, delta, codebook, pi, log2K: int, V: int, stream=None) -> Packed:
    """Pack device field tensors (uint8 [d_out, d_in/8] x3, fp16 [d_out, d_in/128] x2) and keep
    the codebook (fp16 [K, 8]) and permutation (int32 [d_in] or None) alongside."""
    torch = _torch()
    _require_cuda(signs, idx, rcode, mu, delta, codebook, pi)
    d_out, m = signs.shape
    d_in = m * 8
    for name, t in (("signs", signs), ("idx", idx), ("rcode", rcode)):
        if tuple(t.shape) != (d_out, m) or str(t.dtype) != "torch.uint8" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 [{d_out}, {m}] tensor")
    for name, t in (("mu", mu), ("delta", delta)):
        if (tuple(t.shape) != (d_out, d_in // 128) or str(t.dtype) != "torch.float16"
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float16 [{d_out}, {d_in // 128}] tensor")
    buf = torch.empty(packed_bytes(d_out, d_in, log2K, V), dtype=torch.uint8, device=signs.device)
    _check("sage_pack", lib().sage_pack(_ptr(signs), _ptr(idx), _ptr(rcode), _ptr(mu), _ptr(delta),
                                        d_out, d_in, log2K, V, _ptr(buf), _stream(stream)))
    return Packed(d_out, d_in, log2K, V, buf, codebook, pi)


def unpack(p: Packed, stream=None):
    torch = _torch()
    dev = p.packed.device
    m, ng = p.d_in // 8, p.d_in // 128
    signs = torch.empty((p.d_out, m), dtype=torch.uint8, device=dev)
    idx = torch.empty_like(signs)
    rcode = torch.empty_like(signs)
    mu = torch.empty((p.d_out, ng), dtype=torch.float16, device=dev)
    delta = torch.empty_like(mu)
    _check("sage_unpack", lib().sage_unpack(_ptr(p.packed), p.d_out, p.d_in, p.log2K, p.V,
                                            _ptr(signs), _ptr(idx), _ptr(rcode), _ptr(mu),
                                            _ptr(delta), _stream(stream)))
    return signs, idx, rcode, mu, delta


def encode_fields(W, pi, omega, codebook, log2K: int, V: int, overflow=None, stream=None):
    """Code fields of W (fp32 [d_out, d_in], original order) for a given fp16 codebook [K, 8],
    permutation (int32 [d_in] or None) and float64 position weights [d_in] in permuted order.
    Returns (signs, idx, rcode, mu, delta) as device tensors in sage_pack's layout; `overflow`,
    if given, is a uint32 device counter incremented for every group outside the fp16 range."""
    torch = _torch()
    _require_cuda(W, pi, omega, codebook, overflow)
    d_out, d_in = W.shape
    dev = W.device
    m, ng = d_in // 8, d_in // 128
    signs = torch.empty((d_out, m), dtype=torch.uint8, device=dev)
    idx = torch.empty_like(signs)
    rcode = torch.empty_like(signs)
    mu = torch.empty((d_out, ng), dtype=torch.float16, device=dev)
    delta = torch.empty_like(mu)
    _check("sage_encode_fields",
           lib().sage_encode_fields(_ptr(W), d_out, d_in, W.stride(0), _ptr(pi), _ptr(omega),
                                    _ptr(codebook), log2K, V, _ptr(signs), _ptr(idx),
                                    _ptr(rcode), _ptr(mu), _ptr(delta), _ptr(overflow),
                                    _stream(stream)))
    return signs, idx, rcode, mu, delta


def abs_score(W, e, fields, codebook, log2K: int, V: int, pi, stream=None):
    """Eq. (8) score of an encoding: a float64 device tensor [numerator, denominator, ratio].
    `fields` is (signs, idx, rcode, mu, delta) as encode_fields returns them; e holds the float64
    channel energies in original order."""
    torch = _torch()
    signs, idx, rcode, mu, delta = fields
    _require_cuda(W, e, signs, idx, rcode, mu, delta, codebook, pi)
    d_out, d_in = W.shape
    n = ctypes.c_size_t(0)
    _check("sage_abs_score_workspace_bytes",
           lib().sage_abs_score_workspace_bytes(d_out, d_in, ctypes.byref(n)))
    ws = torch.empty(max(n.value, 8), dtype=torch.uint8, device=W.device)
    out = torch.empty(3, dtype=torch.float64, device=W.device)
    _check("sage_abs_score",
           lib().sage_abs_score(_ptr(W), d_out, d_in, W.stride(0), _ptr(e), _ptr(signs), _ptr(idx),
                                _ptr(rcode), _ptr(mu), _ptr(delta), _ptr(codebook), log2K, V,
                                _ptr(pi), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def _rows(t):
    return (1, t.shape[0], t.shape[0]) if t.dim() == 1 else (t.shape[0], t.shape[1], t.stride(0))


def rmsnorm_permute(X, gamma, eps: float, pi=None, out=None, stream=None):
    """fp16 RMSNorm of the rows of X ([M, d] or [d]) with weight gamma, written in the order of
    pi (a matrix's permutation) or unpermuted when pi is None."""
    torch = _torch()
    _require_cuda(X, gamma, pi, out)
    M, d, ld = _rows(X)
    if out is None:
        out = torch.empty(X.shape, dtype=torch.float16, device=X.device)
    _check("sage_rmsnorm_permute",
           lib().sage_rmsnorm_permute(_ptr(X), M, d, ld, _ptr(gamma), float(eps), _ptr(pi),
                                      _ptr(out), _rows(out)[2], _stream(stream)))
    return out


def silu_mul_permute(G, U, pi=None, out=None, stream=None):
    """fp16 silu(G) * U ([M, d] or [d], same strides), written in the order of pi."""
    torch = _torch()
    _require_cuda(G, U, pi, out)
    M, d, ld = _rows(G)
    if _rows(U)[2] != ld:
        raise ValueError("G and U must share their row stride")
    if out is None:
        out = torch.empty(G.shape, dtype=torch.float16, device=G.device)
    _check("sage_silu_mul_permute",
           lib().sage_silu_mul_permute(_ptr(G), _ptr(U), M, d, ld, _ptr(pi), _ptr(out),
                                       _rows(out)[2], _stream(stream)))
    return out


def dequant(p: Packed, out=None, stream=None):
    """Dense fp16 copy of the decoded weights in original column order (see sage_dequant)."""
    torch = _torch()
    _check_packed(p)
    w = torch.empty((p.d_out, p.d_in), dtype=torch.float16, device=p.packed.device) \
        if out is None else out
    _require_vec("out", w, p.d_out * p.d_in)
    d = p.desc()
    _check("sage_dequant", lib().sage_dequant(ctypes.byref(d), _ptr(w), _stream(stream)))
    return w


def gemv_workspace_bytes(p: Packed) -> int:
    n = ctypes.c_size_t(0)
    d = p.desc()
    _check("sage_gemv_workspace_bytes", lib().sage_gemv_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def workspace(nbytes: int, device):
    """A zero-filled workspace (libsage keeps it zero-ready between calls)."""
    torch = _torch()
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def gemv(p: Packed, x, y=None, ws=None, stream=None):
    """y = W_hat x (batch one). x in original channel order, or in stored order when p.pi is
    None (see sage_gemv in include/sage.h)."""
    torch = _torch()
    _check_packed(p)
    _require_vec("x", x, p.d_in)
    if y is None:
        y = torch.empty(p.d_out, dtype=torch.float16, device=x.device)
    _require_vec("y", y, p.d_out)
    d = p.desc()
    _check("sage_gemv", lib().sage_gemv(ctypes.byref(d), _ptr(x), _ptr(y), _ptr(ws),
                                        0 if ws is None else ws.numel(), _stream(stream)))
    return y


def _mat_array(ps: Sequence[Packed]):
    arr = (SageMatrix * len(ps))()
    for i, p in enumerate(ps):
        arr[i] = p.desc()
    return arr


def gemv_multi_workspace_bytes(ps: Sequence[Packed]) -> int:
    n = ctypes.c_size_t(0)
    arr = _mat_array(ps)
    _check("sage_gemv_multi_workspace_bytes",
           lib().sage_gemv_multi_workspace_bytes(arr, len(ps), ctypes.byref(n)))
    return n.value


def gemv_multi(ps: Sequence[Packed], xs, ys=None, ws=None, stream=None):
    """Several independent products y_j = W_j x_j in one launch (see sage_gemv_multi)."""
    torch = _torch()
    if len(xs) != len(ps):
        raise ValueError("one input per matrix")
    if ys is None:
        ys = [torch.empty(p.d_out, dtype=torch.float16, device=x.device) for p, x in zip(ps, xs)]
    for p, x, y in zip(ps, xs, ys):
        _check_packed(p)
        _require_vec("x", x, p.d_in)
        _require_vec("y", y, p.d_out)
    arr = _mat_array(ps)
    xa = (ctypes.c_void_p * len(ps))(*[_ptr(x) for x in xs])
    ya = (ctypes.c_void_p * len(ps))(*[_ptr(y) for y in ys])
    _check("sage_gemv_multi", lib().sage_gemv_multi(arr, xa, ya, len(ps), _ptr(ws),
                                                    0 if ws is None else ws.numel(),
                                                    _stream(stream)))
    return ys


def gemm_small_workspace_bytes(p: Packed, M: int) -> int:
    n = ctypes.c_size_t(0)
    d = p.desc()
    _check("sage_gemm_small_workspace_bytes",
           lib().sage_gemm_small_workspace_bytes(ctypes.byref(d), M, ctypes.byref(n)))
    return n.value


def gemm_small(p: Packed, X, Y=None, ws=None, stream=None):
    """Y = X W_hat^T for M activation rows (see sage_gemm_small)."""
    torch = _torch()
    _check_packed(p)
    _require_cuda(X)
    if X.dim() != 2 or str(X.dtype) != "torch.float16" or X.stride(1) != 1:
        raise ValueError("X must be a 2-D float16 tensor with unit column stride")
    M = X.shape[0]
    if X.shape[1] < p.d_in:
        raise ValueError(f"X rows hold {X.shape[1]} values, need d_in = {p.d_in}")
    if Y is None:
        Y = torch.empty((M, p.d_out), dtype=torch.float16, device=X.device)
    if (Y.dim() != 2 or str(Y.dtype) != "torch.float16" or Y.stride(1) != 1
            or Y.shape[0] < M or Y.shape[1] < p.d_out):
        raise ValueError("Y must be a float16 [M, >= d_out] tensor with unit column stride")
    if ws is None:
        ws = workspace(gemm_small_workspace_bytes(p, M), X.device)
    d = p.desc()
    _check("sage_gemm_small", lib().sage_gemm_small(ctypes.byref(d), _ptr(X), M, X.stride(0),
                                                    _ptr(Y), Y.stride(0), _ptr(ws), ws.numel(),
                                                    _stream(stream)))
    return Y


# Size of sage_gemm_small_noalloc's fixed device workspace (SAGE_NOALLOC_SCRATCH_BYTES in sage.h).
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024


def gemm_small_noalloc(p: Packed, X, Y, stream=None):
    """Y = X W_hat^T like gemm_small, through sage_gemm_small_noalloc: the library's fixed
    per-device workspace instead of a caller's, so the call allocates no device memory (Y is the
    caller's). Calls that overlap in time on one device race on that workspace."""
    _check_packed(p)
    _require_cuda(X)
    _require_cuda(Y)
    if X.dim() != 2 or str(X.dtype) != "torch.float16" or X.stride(1) != 1:
        raise ValueError("X must be a 2-D float16 tensor with unit column stride")
    M = X.shape[0]
    if X.shape[1] < p.d_in:
        raise ValueError(f"X rows hold {X.shape[1]} values, need d_in = {p.d_in}")
    if (Y.dim() != 2 or str(Y.dtype) != "torch.float16" or Y.stride(1) != 1
            or Y.shape[0] < M or Y.shape[1] < p.d_out):
        raise ValueError("Y must be a float16 [M, >= d_out] tensor with unit column stride")
    d = p.desc()
    _check("sage_gemm_small_noalloc",
           lib().sage_gemm_small_noalloc(ctypes.byref(d), _ptr(X), M, X.stride(0), _ptr(Y),
                                         Y.stride(0), _stream(stream)))
    return Y


def expert_table(experts: Sequence, device):
    """Device array of descriptors for moe_gemv / moe_gemv_grouped.

    `experts` is a sequence of Packed (one matrix per expert) or of sequences of Packed (expert
    e's matrix j at e*n_mats + j). The returned tensor keeps references to the Packed matrices it
    points at, so their device buffers stay allocated for as long as the table is alive."""
    torch = _torch()
    if len(experts) == 0:
        raise ValueError("no experts")
    nested = not isinstance(experts[0], Packed)
    n_mats = len(experts[0]) if nested else 1
    flat = [m for ex in experts for m in ex] if nested else list(experts)
    if nested and any(len(ex) != n_mats for ex in experts):
        raise ValueError("every expert needs the same number of matrices")
    for m in flat:
        _check_packed(m)
    arr = _mat_array(flat)
    raw = bytes(arr)
    host = torch.frombuffer(bytearray(raw), dtype=torch.uint8)
    table = host.to(device)
    table._sage_matrices = flat
    table._sage_n_mats = n_mats
    return table, n_mats


def _table_mats(table):
    mats = getattr(table, "_sage_matrices", None)
    if mats is None:
        raise ValueError("use a table made by expert_table()")
    return mats


def _check_moe_slots(mats, n_mats, j, ids, x, x_stride, y, y_stride):
    """Every expert's matrix j fits the slot strides and the x / y tensors for n_sel slots."""
    n_sel = ids.numel()
    d_in = max(mats[e * n_mats + j].d_in for e in range(len(mats) // n_mats))
    d_out = max(mats[e * n_mats + j].d_out for e in range(len(mats) // n_mats))
    if x_stride < 0 or x_stride % 2 or y_stride < 0:
        raise ValueError("strides must be non-negative (x_stride even)")
    if x_stride and x_stride < d_in:
        raise ValueError("x_stride shorter than an expert's d_in")
    if n_sel > 1 and y_stride < d_out:
        raise ValueError("y_stride shorter than an expert's d_out")
    _require_vec("x", x, (n_sel - 1) * x_stride + d_in)
    _require_vec("y", y, (n_sel - 1) * y_stride + d_out)


def moe_gemv(table, ids, x, x_stride: int, y, y_stride: int, stream=None):
    """Batch-one products of the routed experts ids (int32 device tensor) in one launch: slot s
    reads x[s*x_stride:] and writes y[s*y_stride:] (see sage_moe_gemv in include/sage.h)."""
    mats = _table_mats(table)
    if getattr(table, "_sage_n_mats", 1) != 1:
        raise ValueError("moe_gemv takes a table with one matrix per expert")
    _require_vec("ids", ids, 1, "int32")
    _check_moe_slots(mats, 1, 0, ids, x, x_stride, y, y_stride)
    _check("sage_moe_gemv", lib().sage_moe_gemv(
        ctypes.cast(_ptr(table), _PM), len(mats), _ptr(ids), ids.numel(), _ptr(x), x_stride,
        _ptr(y), y_stride, _stream(stream)))
    return y


def moe_gemv_grouped(table, ids, xs, x_strides, ys, y_strides, stream=None):
    """moe_gemv over the n_mats matrices of every routed expert in one launch (see
    sage_moe_gemv_grouped in include/sage.h)."""
    mats = _table_mats(table)
    n_mats = getattr(table, "_sage_n_mats", 1)
    if not (len(xs) == len(ys) == len(x_strides) == len(y_strides) == n_mats):
        raise ValueError("one x, y and stride pair per matrix of an expert")
    _require_vec("ids", ids, 1, "int32")
    for j in range(n_mats):
        _check_moe_slots(mats, n_mats, j, ids, xs[j], x_strides[j], ys[j], y_strides[j])
    xa = (ctypes.c_void_p * n_mats)(*[_ptr(x) for x in xs])
    ya = (ctypes.c_void_p * n_mats)(*[_ptr(y) for y in ys])
    xsa = (ctypes.c_int64 * n_mats)(*x_strides)
    ysa = (ctypes.c_int64 * n_mats)(*y_strides)
    _check("sage_moe_gemv_grouped", lib().sage_moe_gemv_grouped(
        ctypes.cast(_ptr(table), _PM), len(mats) // n_mats, n_mats, _ptr(ids), ids.numel(), xa,
        xsa, ya, ysa, _stream(stream)))
    return ys


def stream_read(buf, nbytes: Optional[int] = None, sink=None, stream=None):
    """Measurement helper: one launch that reads `nbytes` (default: all) bytes of a device tensor
    once (see sage_stream_read in include/sage.h)."""
    torch = _torch()
    _require_cuda(buf)
    total = buf.numel() * buf.element_size()
    n = total if nbytes is None else nbytes
    if n > total:
        raise ValueError("nbytes exceeds the buffer")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check("sage_stream_read", lib().sage_stream_read(_ptr(buf), n, _ptr(sink), _stream(stream)))
    return sink
