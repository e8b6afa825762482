"""sage_gemm_small_noalloc (the small-batch product on the library's fixed per-device workspace)
against sage_gemm_small (the same product on a caller's workspace), through the C ABI.

Both run the same kernels in the same order, so their outputs must agree bit for bit; the first
call of each sequence is also checked against the oracle on sampled activation rows (the bound of
the MFMA kernels, SAGE paper §3.5 and App. A.1). Each sequence makes two calls in a row, the
second with a smaller input: the second call's split-K arrival counters then lie where the first
call left partial sums, so a call that did not zero them would give wrong sums or never finish its
reduction. Problems larger than the fixed workspace are refused before anything is queued.
"""
import numpy as np
import pytest

import workloads as W
from sage_testlib import log, rounded_weight_bounds, upload_pack

import bit_vector_quantized_amd as sage

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "these tests need the GPU"
    sage.lib()
    yield
    torch.cuda.synchronize()


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def _noalloc(p, Xd):
    import torch
    Y = torch.full((Xd.shape[0], p.d_out), float("nan"), dtype=torch.float16, device=Xd.device)
    return sage.gemm_small_noalloc(p, Xd, Y)


def _check_oracle(name, c, X, Y, rows):
    ref, tight, contract = rounded_weight_bounds(c, X[rows])
    got = _np(Y)[rows].astype(np.float64)
    err = np.abs(got - ref)
    log(f"[noalloc] {name}: err/tight={float(np.max(err / tight)):.3f}")
    assert np.all(err <= contract)
    assert np.all(err <= tight)


def _same(name, Y_noalloc, Y_ws):
    a, b = _np(Y_noalloc).view(np.uint16), _np(Y_ws).view(np.uint16)
    log(f"[noalloc] {name}: {a.shape} differing={int(np.count_nonzero(a != b))}")
    assert np.array_equal(a, b), name


@pytest.mark.parametrize("shape,M1,M2", [
    ((4096, 2560), 64, 24),    # split-K small-batch kernel, then a smaller split-K plan
    ((9728, 2560), 64, 17),    # every column group in one workgroup (no split-K), twice
    ((2560, 9728), 48, 17),    # gathered through pi in the workspace, split-K
    ((1024, 2560), 96, 8),     # a prefill-kernel plan, then one 1 x 4 split
])
def test_two_calls_match_workspace_entry(shape, M1, M2):
    d_out, d_in = shape
    c, X = W.small_batch(d_out, d_in, M1)
    p = upload_pack(c)
    for M, seq in ((M1, "first"), (M2, "second")):
        need = sage.gemm_small_workspace_bytes(p, M)
        assert need <= sage.NOALLOC_SCRATCH_BYTES
        Xm = X[:M] if M == M1 else W.draw_x(W.rng_for(181, d_out, M), (M, d_in))
        Xd = _dev(Xm)
        log(f"[noalloc] {d_out}x{d_in} {seq} call M={M} workspace={need} B")
        Y_na = _noalloc(p, Xd)
        Y_ws = sage.gemm_small(p, Xd)
        _same(f"{d_out}x{d_in} M={M}", Y_na, Y_ws)
        if seq == "first":
            _check_oracle(f"{d_out}x{d_in} M={M}", c, Xm, Y_na, [0, M // 2, M - 1])


def test_stored_order_input_and_single_row():
    """pi = NULL with 16-byte aligned rows reads X in place; M = 1 runs the batch-one kernel."""
    c, X = W.small_batch(9728, 2560, 32)
    p = upload_pack(c)
    q = sage.Packed(p.d_out, p.d_in, p.log2K, p.V, p.packed, p.codebook, None)
    Xp = _dev(X[:, np.asarray(c.pi, np.int64)])
    log("[noalloc] 9728x2560 pi=NULL M=32, then M=1")
    _same("pi=NULL M=32", _noalloc(q, Xp), sage.gemm_small(q, Xp))
    _same("pi=NULL M=1", _noalloc(q, Xp[:1]), sage.gemm_small(q, Xp[:1]))


def test_oversized_problem_is_refused():
    """2560 x 9728 at 128 rows needs more than the fixed workspace: SAGE_ERR_SCRATCH, nothing
    queued (the output keeps its contents)."""
    import torch
    c, X = W.small_batch(2560, 9728, 128)
    p = upload_pack(c)
    assert sage.gemm_small_workspace_bytes(p, 128) > sage.NOALLOC_SCRATCH_BYTES
    Y = torch.zeros((128, 2560), dtype=torch.float16, device="cuda")
    with pytest.raises(sage.SageError) as e:
        sage.gemm_small_noalloc(p, _dev(X), Y)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(Y)) == 0
    # the entry point still works after the refusal
    _same("after refusal M=16", _noalloc(p, _dev(X[:16])), sage.gemm_small(p, _dev(X[:16])))
