"""GPU encoder for a given codebook (sage_encode_fields, sage_abs_score) against the float64 oracle.

Bars:
  fields     bit-exact (signs, idx, rcode, fp16 mu and delta) against oracle.encoder.encode_fields:
             every argmax and rounding decision is taken in float64 on both sides with the same
             evaluation order (SAGE paper §3.2 Eq. (6), §3.1 Eq. (2), App. A.6 Eq. (14)).
  ABS score  |E_gpu - E_oracle| <= 1e-10 E_oracle (§3.3 Eq. (8); both are float64 sums of
             nonnegative terms in different orders), and the split chosen by Eq. (9) is the same.
Inputs: seeded synthetic weights and energies (workloads/); the permutation and position weights
are the oracle's ESG order and Eq. (4) weights of those energies.
"""
import numpy as np
import pytest

import workloads as W
from oracle import decoder, encoder
from sage_testlib import log

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
    return t.detach().cpu().numpy()


def _inputs(d_out, d_in, K, seed, gamma=0.75, esg=True):
    rng = W.rng_for(150, d_out, d_in, K, seed)
    Wm, e = W.encoder_matrix(rng, d_out, d_in)
    pi = encoder.esg_permutation(e) if esg else np.arange(d_in)
    omega = encoder.position_weights(e[pi], gamma).reshape(-1)
    cb = W.draw_codebook(rng, K)
    return Wm, e, pi.astype(np.int32), omega, cb


def _gpu_fields(Wm, pi, omega, cb, K, V, overflow=None, identity=False):
    fields = sage.encode_fields(_dev(Wm), None if identity else _dev(pi), _dev(omega), _dev(cb),
                                K.bit_length() - 1, V, overflow=overflow)
    return [(_np(f)) for f in fields]


def _check_fields(name, got, ref, rows=None):
    keys = ("signs", "idx", "rcode", "mu", "delta")
    for k, g in zip(keys, got):
        r = ref[k]
        g = g.view(np.uint16) if k in ("mu", "delta") else g
        if rows is not None:
            g = g[rows]
        mism = int(np.sum(g != r))
        log(f"[encode] {name} {k}: {mism} of {r.size} differ")
        assert mism == 0, f"{name}: {k}"


@pytest.mark.parametrize("K,V", W.SPLITS_FIVE)
@pytest.mark.parametrize("d_out,d_in", [(1, 128), (37, 256), (130, 1152)])
def test_encode_fields_bit_exact(d_out, d_in, K, V):
    Wm, e, pi, omega, cb = _inputs(d_out, d_in, K, 1)
    got = _gpu_fields(Wm, pi, omega, cb, K, V)
    ref = encoder.encode_fields(Wm, pi, omega, cb, V)
    _check_fields(f"{d_out}x{d_in} K={K}", got, ref)


def test_encode_fields_identity_and_uniform_weights():
    """pi = NULL and gamma = 0 (omega = 1: the cosine rule of Eq. (6), §3.2)."""
    Wm, e, pi, omega, cb = _inputs(64, 512, 64, 2, gamma=0.0, esg=False)
    assert np.all(omega == 1.0)
    got = _gpu_fields(Wm, pi, omega, cb, 64, 4, identity=True)
    ref = encoder.encode_fields(Wm, pi, omega, cb, 4)
    _check_fields("identity, uniform weights", got, ref)


def test_encode_fields_zeros_and_signed_zeros():
    """Zero weights are positive (sign bit 0) whatever their sign bit in fp32; an all-zero group
    has mu = delta = 0 and codes 0."""
    Wm, e, pi, omega, cb = _inputs(8, 256, 32, 3)
    Wm[0, :] = 0.0
    Wm[1, ::3] = -0.0
    Wm[2, pi[:8]] = [-1.0, 0.5, -0.25, 0.0, -0.0, 2.0, -3.0, 1.0]
    got = _gpu_fields(Wm, pi, omega, cb, 32, 5)
    ref = encoder.encode_fields(Wm, pi, omega, cb, 5)
    _check_fields("zeros", got, ref)
    assert np.all(got[0][0] == 0) and np.all(got[2][0] == 0) and np.all(got[3][0] == 0)
    assert got[0][2, 0] == 0b01000101


@pytest.mark.parametrize("K,V", [(16, 6), (64, 4), (256, 2)])
def test_encode_fields_planted_exact_recovery(K, V):
    """A matrix built exactly from a codebook, fp16 grids and codes (all exact in fp32) is
    encoded back to the planted fields, and its decode equals it bit for bit."""
    from test_oracle_encoder import planted_matrix
    rng = W.rng_for(151, K)
    d_out, d_in = 40, 512
    e = rng.lognormal(size=d_in)
    pi = encoder.esg_permutation(e)
    Wm, parts = planted_matrix(d_out, d_in, K, V, pi, seed=K + 7)
    assert np.array_equal(Wm.astype(np.float32).astype(np.float64), Wm)
    omega = encoder.position_weights(e[pi], 0.75).reshape(-1)
    cb = parts["C"].astype(np.float16).view(np.uint16)
    got = _gpu_fields(Wm.astype(np.float32), pi.astype(np.int32), omega, cb, K, V)
    assert np.array_equal(got[1], parts["z"])
    assert np.array_equal(got[2], parts["q"])
    assert np.array_equal(got[3].astype(np.float64), parts["mu"])
    assert np.array_equal(got[4].astype(np.float64), parts["delta"])
    enc = dict(signs=got[0], idx=got[1], rcode=got[2], mu=got[3].view(np.uint16),
               delta=got[4].view(np.uint16), codebook=cb, pi=pi, K=K, V=V, d_out=d_out, d_in=d_in)
    assert np.array_equal(decoder.decode(enc), Wm)


@pytest.mark.parametrize("K,V", [(64, 4), (256, 2)])
def test_encode_fields_full_size_sampled_rows(K, V):
    """9728x2560 encoded whole on the GPU; 384 sampled rows (first, last, spread) checked bit for
    bit against the oracle, which encodes rows independently."""
    Wm, e, pi, omega, cb = _inputs(9728, 2560, K, 4)
    got = _gpu_fields(Wm, pi, omega, cb, K, V)
    rows = np.unique(np.concatenate([[0, 1, 9727], W.rng_for(152).choice(9728, 381, replace=False)]))
    ref = encoder.encode_fields(Wm[rows], pi, omega, cb, V)
    _check_fields(f"9728x2560 K={K} sampled", got, ref, rows=rows)


def test_encode_fields_calibrated_matrix_matches_full_encoder():
    """The single calibrated matrix: the oracle's full encoder (k-means codebook) and the GPU,
    given that codebook, the ESG order and the Eq. (4) weights, give the same fields."""
    sm = W.single_matrix_calib()
    e = encoder.channel_energy(sm.X_cal)
    full = encoder.encode_matrix(sm.W.astype(np.float64), e, 64, 4, gamma=0.75, iters=20, seed=0)
    omega = encoder.position_weights(e[full["pi"]], 0.75).reshape(-1)
    got = _gpu_fields(sm.W, full["pi"], omega, full["codebook"], 64, 4)
    ref = encoder.encode_fields(sm.W, full["pi"], omega, full["codebook"], 4)
    _check_fields("calibrated 256x1024", got, ref)
    for k, g in zip(("signs", "idx", "rcode"), got[:3]):
        assert np.array_equal(g, full[k]), k


@pytest.mark.filterwarnings("ignore:overflow encountered in cast")
def test_encode_fields_overflow_counted():
    """Weights beyond the fp16 range make the grid non-finite: the oracle refuses, the device
    counts the groups."""
    import torch
    Wm, e, pi, omega, cb = _inputs(4, 256, 64, 5)
    Wm[1, :] *= 1e7
    with pytest.raises(OverflowError):
        encoder.encode_fields(Wm, pi, omega, cb, 4)
    ovf = torch.zeros(1, dtype=torch.int32, device="cuda")
    _gpu_fields(Wm, pi, omega, cb, 64, 4, overflow=ovf)
    n = int(_np(ovf)[0])
    log(f"[encode] overflow groups: {n}")
    assert n == 2       # both groups of row 1


@pytest.mark.parametrize("K,V", [(64, 4), (256, 2)])
@pytest.mark.parametrize("d_out,d_in", [(37, 256), (300, 2560)])
def test_abs_score_matches_oracle(d_out, d_in, K, V):
    Wm, e, pi, omega, cb = _inputs(d_out, d_in, K, 6)
    ref_f = encoder.encode_fields(Wm, pi, omega, cb, V)
    fields = sage.encode_fields(_dev(Wm), _dev(pi), _dev(omega), _dev(cb), K.bit_length() - 1, V)
    out = _np(sage.abs_score(_dev(Wm), _dev(e), fields, _dev(cb), K.bit_length() - 1, V, _dev(pi)))
    E = encoder.abs_score(Wm, decoder.decode(ref_f), e)
    num = np.sum(e * np.sum((Wm.astype(np.float64) - decoder.decode(ref_f)) ** 2, axis=0))
    log(f"[abs] {d_out}x{d_in} K={K}: gpu {out[2]:.15e} oracle {E:.15e}")
    assert abs(out[2] - E) <= 1e-10 * E
    assert abs(out[0] - num) <= 1e-10 * num


def test_abs_selection_matches_oracle():
    """Eq. (9): encode with each of the five splits (each with its own codebook) and keep the
    first minimum of Eq. (8); GPU scores pick the same split as the oracle's."""
    Wm, e, pi, omega, _ = _inputs(64, 1024, 16, 7)
    rng = W.rng_for(153)
    scores_gpu, scores_ref = [], []
    for K, V in W.SPLITS_FIVE:
        cb = W.draw_codebook(rng, K)
        fields = sage.encode_fields(_dev(Wm), _dev(pi), _dev(omega), _dev(cb), K.bit_length() - 1, V)
        scores_gpu.append(float(_np(sage.abs_score(_dev(Wm), _dev(e), fields, _dev(cb),
                                                   K.bit_length() - 1, V, _dev(pi)))[2]))
        scores_ref.append(encoder.abs_score(Wm, decoder.decode(encoder.encode_fields(Wm, pi, omega, cb, V)), e))
    log(f"[abs] scores gpu {np.round(scores_gpu, 6)} oracle {np.round(scores_ref, 6)}")
    assert int(np.argmin(scores_gpu)) == int(np.argmin(scores_ref))
    assert np.allclose(scores_gpu, scores_ref, rtol=1e-10, atol=0)
