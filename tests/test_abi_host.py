"""The C ABI library on the host (no GPU needed): it loads, exports every function declared in
include/sage.h, and rejects invalid arguments with the documented status codes before queueing
any device work."""
import ctypes

import pytest

import bit_vector_quantized_amd as sage
from bit_vector_quantized_amd import SageMatrix

OK, NULL, SHAPE, SPLIT, ALIGN, WS, HIP, ARG, SCRATCH = range(9)


@pytest.fixture(scope="module")
def L():
    return sage.lib()


def test_exports_every_declared_function(L):
    names = sage.header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert L.sage_format_version() == 3 and L.sage_version() >= 20000
    assert len(sage.source_digest()) == 16


def test_status_strings(L):
    for st in range(9):
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
    # the product needs no workspace
    n = ctypes.c_size_t(7)
    big = _desc(d_out=2560, d_in=9728)
    assert L.sage_gemv_workspace_bytes(ctypes.byref(big), ctypes.byref(n)) == OK and n.value == 0
    # inputs wider than the workgroup stages in LDS are refused before any launch
    assert L.sage_gemv(ctypes.byref(_desc(d_in=33792)), x, y, None, 0, None) == SHAPE
    assert L.sage_gemv(ctypes.byref(_desc(d_in=12288, log2K=8, V=2, pi=1 << 23)), x, y, None, 0,
                       None) == SHAPE


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


def test_gemm_noalloc_validation(L):
    """The no-allocation variant checks its arguments like sage_gemm_small and refuses, before
    any device call, a problem whose workspace exceeds its fixed 16 MiB."""
    X = ctypes.c_void_p(1 << 20)
    Y = ctypes.c_void_p(1 << 21)
    d = _desc()
    assert sage.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert L.sage_gemm_small_noalloc(None, X, 4, 256, Y, 64, None) == NULL
    assert L.sage_gemm_small_noalloc(ctypes.byref(d), None, 4, 256, Y, 64, None) == NULL
    assert L.sage_gemm_small_noalloc(ctypes.byref(d), X, 0, 256, Y, 64, None) == SHAPE
    assert L.sage_gemm_small_noalloc(ctypes.byref(d), X, 4, 257, Y, 64, None) == ALIGN
    assert L.sage_gemm_small_noalloc(ctypes.byref(_desc(log2K=9, V=1)), X, 4, 256, Y, 64,
                                     None) == SPLIT
    big = _desc(d_out=2560, d_in=9728)
    n = ctypes.c_size_t(0)
    assert L.sage_gemm_small_workspace_bytes(ctypes.byref(big), 128, ctypes.byref(n)) == OK
    assert n.value > sage.NOALLOC_SCRATCH_BYTES
    assert L.sage_gemm_small_noalloc(ctypes.byref(big), X, 128, 9728, Y, 2560, None) == SCRATCH
    assert "16 MiB" in sage.status_string(SCRATCH)


def test_moe_validation(L):
    tab = ctypes.cast(ctypes.c_void_p(1 << 26), ctypes.POINTER(SageMatrix))
    ids = ctypes.c_void_p(1 << 27)
    x = ctypes.c_void_p(1 << 20)
    y = ctypes.c_void_p(1 << 21)
    assert L.sage_moe_gemv(None, 128, ids, 8, x, 0, y, 2048, None) == NULL
    assert L.sage_moe_gemv(tab, 128, None, 8, x, 0, y, 2048, None) == NULL
    assert L.sage_moe_gemv(tab, 128, ids, 8, None, 0, y, 2048, None) == NULL
    assert L.sage_moe_gemv(tab, 0, ids, 8, x, 0, y, 2048, None) == ARG
    assert L.sage_moe_gemv(tab, 128, ids, 0, x, 0, y, 2048, None) == ARG
    assert L.sage_moe_gemv(tab, 128, ids, 8, x, 767, y, 2048, None) == ARG
    assert L.sage_moe_gemv(tab, 128, ids, 8, x, -2, y, 2048, None) == ARG
    assert L.sage_moe_gemv(tab, 128, ids, 8, x, 0, y, 0, None) == ARG
    assert L.sage_moe_gemv(ctypes.cast(ctypes.c_void_p((1 << 26) + 4), ctypes.POINTER(SageMatrix)),
                           128, ids, 8, x, 0, y, 2048, None) == ALIGN
    assert L.sage_moe_gemv(tab, 128, ctypes.c_void_p((1 << 27) + 2), 8, x, 0, y, 2048, None) == ALIGN
    assert L.sage_moe_gemv(tab, 128, ids, 8, ctypes.c_void_p((1 << 20) + 2), 0, y, 2048, None) == ALIGN
    xs = (ctypes.c_void_p * 2)(1 << 20, 1 << 20)
    ys = (ctypes.c_void_p * 2)(1 << 21, 1 << 22)
    st = (ctypes.c_int64 * 2)(0, 0)
    yst = (ctypes.c_int64 * 2)(768, 768)
    assert L.sage_moe_gemv_grouped(tab, 128, 0, ids, 8, xs, st, ys, yst, None) == ARG
    assert L.sage_moe_gemv_grouped(tab, 128, 5, ids, 8, xs, st, ys, yst, None) == ARG
    assert L.sage_moe_gemv_grouped(tab, 128, 2, ids, 8, xs, None, ys, yst, None) == NULL
    bad = (ctypes.c_void_p * 2)(1 << 20, None)
    assert L.sage_moe_gemv_grouped(tab, 128, 2, ids, 8, bad, st, ys, yst, None) == NULL


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


# ------------------------------------------------------------------------------------------------
# The binding's own checks (argument marshalling only, no device work). Stand-in tensors expose the
# attributes the checks read, so these run without a GPU.
# ------------------------------------------------------------------------------------------------

class _FakeT:
    def __init__(self, n, dtype="float16", cuda=True, contiguous=True, ptr=1 << 20, esize=2):
        import torch
        self._n, self.dtype, self.is_cuda = n, getattr(torch, dtype), cuda
        self._c, self._p, self._e = contiguous, ptr, esize

    def numel(self):
        return self._n

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return self._p

    def element_size(self):
        return self._e


def _fake_packed(d_out=64, d_in=256, log2K=6, V=4, cb=None, pi="ok", packed_bytes=None):
    nbytes = sage.packed_bytes(d_out, d_in, log2K, V) if packed_bytes is None else packed_bytes
    return sage.Packed(d_out, d_in, log2K, V, _FakeT(nbytes, "uint8", esize=1),
                       _FakeT(8 << log2K) if cb is None else cb,
                       _FakeT(d_in, "int32", esize=4) if pi == "ok" else pi)


def test_binding_rejects_wrong_vectors():
    p = _fake_packed()
    with pytest.raises(ValueError, match="at least 256"):
        sage.gemv(p, _FakeT(255))
    with pytest.raises(ValueError, match="float16"):
        sage.gemv(p, _FakeT(256, "float32"))
    with pytest.raises(ValueError, match="contiguous"):
        sage.gemv(p, _FakeT(256, contiguous=False))
    with pytest.raises(ValueError, match="device"):
        sage.gemv(p, _FakeT(256, cuda=False))
    with pytest.raises(ValueError, match="y has"):
        sage.gemv(p, _FakeT(256), y=_FakeT(63))


def test_binding_rejects_mismatched_matrix_buffers():
    with pytest.raises(ValueError, match="codebook"):
        sage.gemv(_fake_packed(cb=_FakeT(8 * 32)), _FakeT(256))
    with pytest.raises(ValueError, match="pi"):
        sage.gemv(_fake_packed(pi=_FakeT(255, "int32", esize=4)), _FakeT(256))
    with pytest.raises(ValueError, match="packed"):
        sage.gemv(_fake_packed(packed_bytes=100), _FakeT(256))
    with pytest.raises(ValueError, match="out has"):
        sage.dequant(_fake_packed(), out=_FakeT(64 * 256 - 1))


def test_expert_table_keeps_its_matrices_alive():
    """The device descriptor table holds references to the matrices it points at: dropping the
    caller's list must not free them while the table lives (the cause of a past GPU fault)."""
    import gc
    import weakref
    mats = [_fake_packed() for _ in range(3)]
    table, n_mats = sage.expert_table(mats, "cpu")
    assert n_mats == 1
    refs = [weakref.ref(m) for m in mats]
    del mats
    gc.collect()
    assert all(r() is not None for r in refs)
    assert [m.packed.data_ptr() for m in table._sage_matrices] == [1 << 20] * 3
    del table
    gc.collect()
    assert all(r() is None for r in refs)


def test_expert_table_grouped_layout():
    mats = [[_fake_packed(), _fake_packed(d_out=128)] for _ in range(2)]
    table, n_mats = sage.expert_table(mats, "cpu")
    assert n_mats == 2 and table.numel() == 4 * ctypes.sizeof(SageMatrix)
    with pytest.raises(ValueError, match="same number"):
        sage.expert_table([[_fake_packed()], [_fake_packed(), _fake_packed()]], "cpu")
