"""The C ABI library on the host (no GPU needed): it loads, exports every function declared in
include/sage.h, and rejects invalid arguments with the documented status codes before queueing
any device work."""
import ctypes

import pytest

import bit_vector_quantized_amd as sage
from bit_vector_quantized_amd import SageMatrix

OK, NULL, SHAPE, SPLIT, ALIGN, WS, HIP, ARG = range(8)


@pytest.fixture(scope="module")
def L():
    return sage.lib()


def test_exports_every_declared_function(L):
    names = sage.header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert L.sage_format_version() >= 1 and L.sage_version() >= 10000


def test_status_strings(L):
    for st in range(8):
        assert len(sage.status_string(st)) >= 2
    assert sage.status_string(99) == "unknown status"


@pytest.mark.parametrize("K,V", [(16, 6), (32, 5), (64, 4), (128, 3), (256, 2)])
def test_packed_bytes_is_2p5_bits_per_weight(K, V):
    L2 = K.bit_length() - 1
    # 18 payload bits per 8 weights + 32 grid bits per 128 weights, rows padded to 64
    assert sage.packed_bytes(9728, 2560, L2, V) == 9728 * 2560 * 2.5 / 8
    assert sage.packed_bytes(65, 128, L2, V) == 2 * 64 * 128 * 2.5 / 8


@pytest.mark.parametrize("d_out,d_in,l2k,V,st", [
    (0, 128, 6, 4, SHAPE), (16, 100, 6, 4, SHAPE), (16, 0, 6, 4, SHAPE),
    (16, 128, 3, 7, SPLIT), (16, 128, 9, 1, SPLIT), (16, 128, 6, 5, SPLIT)])
def test_packed_bytes_rejects(L, d_out, d_in, l2k, V, st):
    n = ctypes.c_size_t(0)
    assert L.sage_packed_bytes(d_out, d_in, l2k, V, ctypes.byref(n)) == st
    assert L.sage_packed_bytes(16, 128, 6, 4, None) == NULL


def test_pack_rejects_null_and_misaligned(L):
    a = ctypes.c_void_p(4096)
    assert L.sage_pack(None, a, a, a, a, 16, 128, 6, 4, a, None) == NULL
    assert L.sage_pack(a, a, a, a, a, 16, 128, 6, 4, None, None) == NULL
    assert L.sage_pack(ctypes.c_void_p(4097), a, a, a, a, 16, 128, 6, 4, a, None) == ALIGN
    assert L.sage_pack(a, a, a, a, a, 16, 128, 6, 4, ctypes.c_void_p(4096 + 128), None) == ALIGN
    assert L.sage_unpack(a, 16, 128, 7, 4, a, a, a, a, a, None) == SPLIT


def _desc(**kw):
    d = dict(d_out=64, d_in=256, log2K=6, V=4, packed=4096, codebook=8192, pi=None)
    d.update(kw)
    return SageMatrix(d["d_out"], d["d_in"], d["log2K"], d["V"], d["packed"], d["codebook"], d["pi"])


def test_gemv_validation(L):
    x = ctypes.c_void_p(1 << 20)
    y = ctypes.c_void_p(1 << 21)
    assert L.sage_gemv(None, x, y, None, 0, None) == NULL
    assert L.sage_gemv(ctypes.byref(_desc(log2K=5, V=4)), x, y, None, 0, None) == SPLIT
    assert L.sage_gemv(ctypes.byref(_desc(d_in=200)), x, y, None, 0, None) == SHAPE
    assert L.sage_gemv(ctypes.byref(_desc(packed=None)), x, y, None, 0, None) == NULL
    assert L.sage_gemv(ctypes.byref(_desc(packed=4096 + 64)), x, y, None, 0, None) == ALIGN
    assert L.sage_gemv(ctypes.byref(_desc(codebook=8194)), x, y, None, 0, None) == ALIGN
    assert L.sage_gemv(ctypes.byref(_desc()), None, y, None, 0, None) == NULL
    assert L.sage_gemv(ctypes.byref(_desc()), ctypes.c_void_p((1 << 20) + 2), y, None, 0, None) == ALIGN
    # a large matrix needs split-K partials: without a workspace the call is refused
    big = _desc(d_out=2560, d_in=9728)
    n = ctypes.c_size_t(0)
    assert L.sage_gemv_workspace_bytes(ctypes.byref(big), ctypes.byref(n)) == OK
    assert n.value > 0
    assert L.sage_gemv(ctypes.byref(big), x, y, None, 0, None) == WS
    assert L.sage_gemv(ctypes.byref(big), x, y, ctypes.c_void_p(1 << 24), n.value - 1, None) == WS


def test_gemm_and_multi_validation(L):
    X = ctypes.c_void_p(1 << 20)
    Y = ctypes.c_void_p(1 << 21)
    d = _desc()
    assert L.sage_gemm_small(ctypes.byref(d), X, 0, 256, Y, 64, None, 0, None) == SHAPE
    assert L.sage_gemm_small(ctypes.byref(d), X, 4, 255, Y, 64, None, 0, None) == SHAPE
    assert L.sage_gemm_small(ctypes.byref(d), X, 4, 256, Y, 63, None, 0, None) == SHAPE
    assert L.sage_gemm_small(ctypes.byref(d), X, 4, 257, Y, 64, None, 0, None) == ALIGN
    arr = (SageMatrix * 2)(_desc(), _desc(log2K=9, V=1))
    xs = (ctypes.c_void_p * 2)(1 << 20, 1 << 20)
    ys = (ctypes.c_void_p * 2)(1 << 21, 1 << 22)
    assert L.sage_gemv_multi(arr, xs, ys, 2, None, 0, None) == SPLIT
    assert L.sage_gemv_multi(arr, xs, ys, 0, None, 0, None) == ARG
    assert L.sage_gemv_multi(arr, xs, ys, 17, None, 0, None) == ARG


def test_moe_validation(L):
    shapes = (SageMatrix * 3)(_desc(d_out=768, d_in=2048), _desc(d_out=768, d_in=2048),
                              _desc(d_out=2048, d_in=768))
    xs = (ctypes.c_void_p * 3)(1 << 20, 1 << 20, 1 << 22)
    ys = (ctypes.c_void_p * 3)(1 << 23, 1 << 24, 1 << 25)
    xst = (ctypes.c_int64 * 3)(0, 0, 768)
    yst = (ctypes.c_int64 * 3)(768, 768, 2048)
    tab = ctypes.cast(ctypes.c_void_p(1 << 26), ctypes.POINTER(SageMatrix))
    ids = ctypes.c_void_p(1 << 27)
    assert L.sage_moe_gemv(tab, 128, shapes, 3, ids, 0, xs, xst, ys, yst, None, 0, None) == ARG
    assert L.sage_moe_gemv(tab, 4, shapes, 3, ids, 8, xs, xst, ys, yst, None, 0, None) == ARG
    bad = (ctypes.c_int64 * 3)(0, 0, 767)
    assert L.sage_moe_gemv(tab, 128, shapes, 3, ids, 8, xs, bad, ys, yst, None, 0, None) == ARG
    small_y = (ctypes.c_int64 * 3)(100, 768, 2048)
    assert L.sage_moe_gemv(tab, 128, shapes, 3, ids, 8, xs, xst, ys, small_y, None, 0, None) == ARG
    n = ctypes.c_size_t(0)
    assert L.sage_moe_gemv_workspace_bytes(shapes, 3, 8, ctypes.byref(n)) == OK


def test_stream_read_validation(L):
    sink = ctypes.c_void_p(1 << 20)
    assert L.sage_stream_read(None, 16, sink, None) == NULL
    assert L.sage_stream_read(ctypes.c_void_p(1 << 21), 16, None, None) == NULL
    assert L.sage_stream_read(ctypes.c_void_p((1 << 21) + 8), 16, sink, None) == ALIGN
    assert L.sage_stream_read(ctypes.c_void_p(1 << 21), 24, sink, None) == ALIGN
    assert L.sage_stream_read(ctypes.c_void_p(1 << 21), 0, sink, None) == OK


def test_encode_and_abs_validation(L):
    a = ctypes.c_void_p(4096)
    args = [a, 16, 256, 256, a, a, a, 6, 4, a, a, a, a, a, None, None]

    def enc(**kw):
        v = list(args)
        names = ["W", "d_out", "d_in", "ldw", "pi", "omega", "codebook", "log2K", "V", "signs",
                 "idx", "rcode", "mu", "delta", "overflow", "stream"]
        for k, x in kw.items():
            v[names.index(k)] = x
        return L.sage_encode_fields(*v)

    assert enc(W=None) == NULL and enc(omega=None) == NULL and enc(delta=None) == NULL
    assert enc(d_in=200) == SHAPE and enc(d_out=0) == SHAPE and enc(ldw=255) == SHAPE
    assert enc(log2K=6, V=5) == SPLIT and enc(log2K=9, V=1) == SPLIT
    assert enc(W=ctypes.c_void_p(4098)) == ALIGN and enc(omega=ctypes.c_void_p(4100)) == ALIGN
    assert enc(pi=ctypes.c_void_p(4104)) == ALIGN
    n = ctypes.c_size_t(0)
    assert L.sage_abs_score_workspace_bytes(16, 256, ctypes.byref(n)) == OK and n.value >= 16
    assert L.sage_abs_score_workspace_bytes(16, 100, ctypes.byref(n)) == SHAPE
    sargs = [a, 16, 256, 256, a, a, a, a, a, a, a, 6, 4, None, a, a, n.value, None]
    assert L.sage_abs_score(*sargs[:14], None, *sargs[15:]) == NULL
    assert L.sage_abs_score(*sargs[:15], None, *sargs[16:]) == WS
    assert L.sage_abs_score(*sargs[:16], n.value - 1, None) == WS
    assert L.sage_abs_score(*sargs[:11], 6, 5, *sargs[13:]) == SPLIT
    assert L.sage_abs_score(*sargs[:4], ctypes.c_void_p(4100), *sargs[5:]) == ALIGN


def test_producer_validation(L):
    a = ctypes.c_void_p(4096)
    assert L.sage_rmsnorm_permute(None, 1, 128, 128, a, 1e-6, None, a, 128, None) == NULL
    assert L.sage_rmsnorm_permute(a, 0, 128, 128, a, 1e-6, None, a, 128, None) == SHAPE
    assert L.sage_rmsnorm_permute(a, 1, 124, 128, a, 1e-6, None, a, 128, None) == SHAPE
    assert L.sage_rmsnorm_permute(a, 1, 128, 127, a, 1e-6, None, a, 128, None) == SHAPE
    assert L.sage_rmsnorm_permute(a, 1, 128, 128, a, -1.0, None, a, 128, None) == ARG
    assert L.sage_rmsnorm_permute(ctypes.c_void_p(4097), 1, 128, 128, a, 1e-6, None, a, 128, None) == ALIGN
    assert L.sage_rmsnorm_permute(a, 1, 128, 128, a, 1e-6, ctypes.c_void_p(4098), a, 128, None) == ALIGN
    assert L.sage_silu_mul_permute(a, None, 1, 128, 128, None, a, 128, None) == NULL
    assert L.sage_silu_mul_permute(a, a, 70000, 128, 128, None, a, 128, None) == SHAPE
    assert L.sage_silu_mul_permute(a, a, 1, 128, 128, None, ctypes.c_void_p(4097), 128, None) == ALIGN
