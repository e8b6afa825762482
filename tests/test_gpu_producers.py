"""Permuting producers (sage_rmsnorm_permute, sage_silu_mul_permute) against the float64 oracle,
and chains that feed their output to the product kernels with pi = NULL.

Bars:
  producer output  within 1 fp16 ulp of the correctly rounded float64 value (the kernels compute
                   in fp32 and round once; their fp32 error is far below half an fp16 ulp, so the
                   result is the correct rounding or its neighbour).
  chains           the product bound of the other parity tests (2e-3 * max_r sum |W_hat||x|),
                   against the oracle product of the producer's own fp16 output in original order.
Compiled-decoding mode of SAGE §3.5: the permutation is fused into the preceding normalization or
activation. Inputs are seeded synthetic (workloads/).
"""
import numpy as np
import pytest

import workloads as W
from oracle import decoder
from sage_testlib import log, ulp_distance, upload_pack

import bit_vector_quantized_amd as sage

pytestmark = pytest.mark.gpu
TOL_REL = 2e-3


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


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint16)


def _check_ulp(name, got_bits, ref64):
    ref_bits = ref64.astype(np.float16).view(np.uint16)
    d = ulp_distance(got_bits, ref_bits)
    log(f"[producer] {name}: max ulp {int(d.max())}, exact {float(np.mean(d == 0)) * 100:.2f} %")
    assert int(d.max()) <= 1, name


@pytest.mark.parametrize("M,d", [(1, 128), (3, 2560), (64, 9728), (2, 32768)])
@pytest.mark.parametrize("permuted", [True, False])
def test_rmsnorm_permute(M, d, permuted):
    rng = W.rng_for(170, M, d)
    X = W.draw_x(rng, (M, d)) * np.float16(3.0)
    gamma = (1.0 + 0.25 * rng.standard_normal(d)).astype(np.float16)
    pi = W.draw_perm(rng, d) if permuted else None
    out = sage.rmsnorm_permute(_dev(X), _dev(gamma), 1e-6, None if pi is None else _dev(pi))
    ref = decoder.rmsnorm_permute(X.astype(np.float64), gamma.astype(np.float64), 1e-6, pi)
    _check_ulp(f"rmsnorm M={M} d={d} pi={permuted}", _bits(out), ref)


@pytest.mark.parametrize("M,d", [(1, 768), (5, 9728), (130, 2048)])
@pytest.mark.parametrize("permuted", [True, False])
def test_silu_mul_permute(M, d, permuted):
    rng = W.rng_for(171, M, d)
    G = W.draw_x(rng, (M, d)) * np.float16(4.0)
    U = W.draw_x(rng, (M, d))
    pi = W.draw_perm(rng, d) if permuted else None
    out = sage.silu_mul_permute(_dev(G), _dev(U), None if pi is None else _dev(pi))
    ref = decoder.silu_mul_permute(G.astype(np.float64), U.astype(np.float64), pi)
    _check_ulp(f"silu*mul M={M} d={d} pi={permuted}", _bits(out), ref)


@pytest.mark.parametrize("pad", [40, 41])
def test_producers_strided_rows_and_scalar_stores(pad):
    """Input rows wider than d (16-byte aligned rows with pad 40, 2-byte aligned with 41); output
    rows of odd stride (no vector stores)."""
    import torch
    rng = W.rng_for(172, pad)
    M, d = 4, 1024
    Xw = W.draw_x(rng, (M, d + pad))
    gamma = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float16)
    pi = W.draw_perm(rng, d)
    Xd = _dev(Xw)[:, :d]
    out = torch.full((M, d + 3), 5.0, dtype=torch.float16, device="cuda")
    sage.rmsnorm_permute(Xd, _dev(gamma), 1e-5, _dev(pi), out=out[:, :d])
    ref = decoder.rmsnorm_permute(Xw[:, :d].astype(np.float64), gamma.astype(np.float64), 1e-5, pi)
    ob = _bits(out)
    _check_ulp("rmsnorm strided", np.ascontiguousarray(ob[:, :d]), ref)
    assert np.all(ob[:, d:] == np.float16(5.0).view(np.uint16))
    G = _dev(Xw)[:, :d]
    U = _dev(Xw[::-1].copy())[:, :d]
    out2 = torch.full((M, d + 3), 5.0, dtype=torch.float16, device="cuda")
    sage.silu_mul_permute(G, U, _dev(pi), out=out2[:, :d])
    ref2 = decoder.silu_mul_permute(Xw[:, :d].astype(np.float64), Xw[::-1, :d].astype(np.float64), pi)
    _check_ulp("silu*mul strided", np.ascontiguousarray(_bits(out2)[:, :d]), ref2)


def _chain_check(name, c, x_orig16, y_dev):
    Wh = decoder.decode(c)
    xf = np.asarray(x_orig16, np.float64)
    ref = xf @ Wh.T
    got = y_dev.detach().cpu().numpy().astype(np.float64)
    tol = TOL_REL * np.max(np.abs(xf) @ np.abs(Wh).T, axis=-1)
    err = np.max(np.abs(got - ref), axis=-1)
    log(f"[chain] {name}: worst err/tol={float(np.max(err / tol)):.3f}")
    assert np.all(err <= tol), name


@pytest.mark.parametrize("M", [1, 16, 300])
def test_rmsnorm_permute_feeds_product_without_gather(M):
    """x -> RMSNorm written in q's stored order -> q with pi = NULL; checked against the oracle
    product of the same normalised values in original order."""
    import torch
    rng = W.rng_for(173, M)
    c = W.draw_codes(rng, 4096, 2560, 64, 4)
    X = W.draw_x(rng, (M, 2560))
    gamma = (1.0 + 0.2 * rng.standard_normal(2560)).astype(np.float16)
    xp = sage.rmsnorm_permute(_dev(X), _dev(gamma), 1e-6, _dev(c.pi))
    x_plain = sage.rmsnorm_permute(_dev(X), _dev(gamma), 1e-6, None)
    # the permuted output is the plain one gathered through pi, bit for bit
    assert np.array_equal(_bits(xp), _bits(x_plain)[:, c.pi])
    p = upload_pack(c, identity_pi=True)
    if M == 1:
        y = sage.gemv(p, xp[0])[None]
    else:
        y = sage.gemm_small(p, xp)
    torch.cuda.synchronize()
    _chain_check(f"rmsnorm -> q M={M}", c, _bits(x_plain).view(np.float16), y)


def test_silu_mul_permute_feeds_down_projection():
    """gate/up outputs -> silu*mul written in down's stored order -> down with pi = NULL."""
    import torch
    rng = W.rng_for(174)
    c = W.draw_codes(rng, 2560, 9728, 64, 4)
    G = W.draw_x(rng, (9728,)) * np.float16(3.0)
    U = W.draw_x(rng, (9728,))
    hp = sage.silu_mul_permute(_dev(G), _dev(U), _dev(c.pi))
    h = sage.silu_mul_permute(_dev(G), _dev(U), None)
    assert np.array_equal(_bits(hp), _bits(h)[c.pi])
    p = upload_pack(c, identity_pi=True)
    y = sage.gemv(p, hp)
    torch.cuda.synchronize()
    _chain_check("silu*mul -> down", c, _bits(h).view(np.float16)[None], y[None])
