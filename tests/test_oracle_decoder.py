"""Pins for the oracle's decoder and products (SAGE paper §3.1 Eq. (1)-(2), §3.2, App. A.6), CPU.

The decoder is checked against a hand-worked example, exact rational arithmetic, unit-vector probes
of the permutation direction, the equal-radii special case, and a brute-force loop product.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import budget, decoder
from workloads import draw_codes, draw_x, rng_for


def _fp16_bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def worked_example(golden_dir):
    with open(os.path.join(golden_dir, "decode_worked_example.json")) as f:
        g = json.load(f)
    d_out, d_in, K, V = g["d_out"], g["d_in"], g["K"], g["V"]
    m = d_in // 8
    cb = np.zeros((K, 8))
    for k in range(K):
        row = g["codebook_rows"].get(str(k))
        if row is None:
            cb[k, k % 8] = 1.0
        else:
            cb[k] = row
    signs = np.zeros((d_out, m), np.uint8)
    idx = np.zeros((d_out, m), np.uint8)
    rcode = np.zeros((d_out, m), np.uint8)
    for c in g["codes"]:
        signs[c["row"], c["subvector"]] = c["signs"]
        idx[c["row"], c["subvector"]] = c["idx"]
        rcode[c["row"], c["subvector"]] = c["rcode"]
    codes = dict(K=K, V=V, signs=signs, idx=idx, rcode=rcode, mu=_fp16_bits(g["mu"]),
                 delta=_fp16_bits(g["delta"]), codebook=_fp16_bits(cb),
                 pi=np.arange(d_in - 1, -1, -1, dtype=np.int32))
    expected = np.zeros((d_out, d_in))
    listed = {(c["row"], c["subvector"]) for c in g["codes"]}
    for r in range(d_out):
        for j in range(m):
            if (r, j) not in listed:
                expected[r, 255 - 8 * j] = g["mu"][r][j // 16]
    for r, col, val in g["expected_nonzero"]:
        expected[r, col] = val
    return codes, expected


def test_decode_worked_example(golden_dir):
    codes, expected = worked_example(golden_dir)
    W = decoder.decode(codes)
    assert np.array_equal(W, expected)
    # compared as values: a negative sign on a zero codeword component gives -0.0, equal to +0.0
    assert np.array_equal(decoder.dequant_fp16(codes).view(np.float16), expected.astype(np.float16))


def test_decode_is_exact_rational():
    """Every decoded weight equals the exact rational mu + q*delta times the signed component."""
    c = draw_codes(rng_for(1), 3, 256, 32, 5)
    W = decoder.decode(c)
    cb = c.codebook.view(np.float16)
    mu = c.mu.view(np.float16)
    de = c.delta.view(np.float16)
    inv = np.argsort(c.pi)
    for r in range(3):
        for col in range(0, 256, 7):
            p = int(inv[col])
            j, i = divmod(p, 8)
            q = int(c.rcode[r, j])
            rr = Fraction(float(mu[r, j // 16])) + q * Fraction(float(de[r, j // 16]))
            sgn = -1 if (int(c.signs[r, j]) >> i) & 1 else 1
            w = rr * sgn * Fraction(float(cb[int(c.idx[r, j]), i]))
            assert Fraction(W[r, col]) == w
            assert np.float16(float(w)) == W[r, col].astype(np.float16)


def test_permutation_direction_unit_probe():
    """With x = e_c in original channel order, y is column c of W_hat; column pi[p] of W_hat is
    permuted column p of the stored matrix (§3.2: inputs are gathered by pi at inference)."""
    c = draw_codes(rng_for(2), 5, 128, 16, 6)
    Wp = decoder.decode_permuted(c)
    for p in (0, 1, 9, 77, 127):
        x = np.zeros(128, np.float16)
        x[c.pi[p]] = 1.0
        assert np.array_equal(decoder.gemv(c, x), Wp[:, p])


def test_equal_radii_group_reconstructs_common_value():
    """Appendix A.6: with a zero step every radius in the group is the offset."""
    c = draw_codes(rng_for(3), 4, 256, 64, 4)
    c.delta[:] = 0
    r = decoder.radii(c)
    mu = c.mu.view(np.float16).astype(np.float64)
    assert np.array_equal(r, mu[:, np.arange(32) // 16])


@pytest.mark.parametrize("d_out,d_in", [(1, 128), (5, 128), (16, 256)])
def test_gemv_brute_force_loop(d_out, d_in):
    c = draw_codes(rng_for(4, d_out, d_in), d_out, d_in, 128, 3)
    x = rng_for(5).standard_normal(d_in).astype(np.float16)
    cb = c.codebook.view(np.float16).astype(float)
    mu = c.mu.view(np.float16).astype(float)
    de = c.delta.view(np.float16).astype(float)
    y = np.zeros(d_out)
    for r in range(d_out):
        acc = 0.0
        for p in range(d_in):
            j, i = divmod(p, 8)
            rad = mu[r, j // 16] + int(c.rcode[r, j]) * de[r, j // 16]
            s = -1.0 if (int(c.signs[r, j]) >> i) & 1 else 1.0
            acc += rad * s * cb[int(c.idx[r, j]), i] * float(x[int(c.pi[p])])
        y[r] = acc
    ref = decoder.gemv(c, x)
    assert np.allclose(ref, y, rtol=1e-12, atol=1e-12)


def test_gemm_and_moe_agree_with_gemv():
    c = draw_codes(rng_for(6), 32, 256, 64, 4)
    X = rng_for(7).standard_normal((4, 256)).astype(np.float16)
    Y = decoder.gemm(c, X)
    for m in range(4):
        assert np.allclose(Y[m], decoder.gemv(c, X[m]), rtol=1e-13, atol=1e-13)
    experts = [{"gate": draw_codes(rng_for(10, e), 16, 128, 16, 6),
                "up": draw_codes(rng_for(11, e), 16, 128, 16, 6),
                "down": draw_codes(rng_for(12, e), 128, 16 * 8, 16, 6)} for e in range(4)]
    ids = np.array([2, 0])
    x = rng_for(8).standard_normal(128).astype(np.float16)
    h = rng_for(9).standard_normal((2, 128)).astype(np.float16)
    out = decoder.moe_gemv(experts, ids, x, h)
    assert np.array_equal(out["gate"][0], decoder.gemv(experts[2]["gate"], x))
    assert np.array_equal(out["down"][1], decoder.gemv(experts[0]["down"], h[1]))


def test_tolerance_definition():
    c = draw_codes(rng_for(13), 8, 128, 64, 4)
    x = rng_for(14).standard_normal(128).astype(np.float16)
    t = decoder.tolerance(c, x)
    W = decoder.decode(c)
    assert t == pytest.approx(2e-3 * np.max(np.abs(W) @ np.abs(x.astype(float))), rel=1e-15)


def test_decode_rejects_bad_fields():
    c = draw_codes(rng_for(15), 2, 128, 16, 6)
    c.idx[0, 0] = 16
    with pytest.raises(ValueError):
        decoder.decode(c)
    c = draw_codes(rng_for(15), 2, 128, 16, 6)
    c.pi[0] = c.pi[1]
    with pytest.raises(ValueError):
        decoder.decode(c)


# ------------------------------------------------------------------------------ Eq. (3), Eq. (15)

@pytest.mark.parametrize("K,V", [(16, 6), (32, 5), (64, 4), (128, 3), (256, 2)])
def test_bit_budget_18_bits(K, V):
    assert budget.bits_per_subvector(K, V) == 18
    assert budget.bits_per_subvector(K, V) / 8 == 2.25


def test_storage_figures_from_the_paper():
    # App. A.6: fp16 grids add 0.25 bits per weight at G = 128, giving 2.50 before the codebook.
    N = 4096 * 4096
    bpw = budget.bpw_matrix(4096, 4096, 64, 4)
    assert bpw - 64 * 8 * 16 / N == 2.50
    # §1: a 64-entry fp16 codebook occupies 1 KiB.
    assert budget.codebook_bytes(64) == 1024
    assert budget.payload_bytes(9728, 2560, 64, 4) == 9728 * 2560 * 18 / 64
    assert budget.grid_bytes(9728, 2560) == 9728 * 20 * 4


# ------------------------------------------------------------------------------ SwiGLU block

def test_silu_closed_forms():
    e = np.e
    assert decoder.silu(0.0) == 0.0
    assert abs(decoder.silu(1.0) - 1.0 / (1.0 + 1.0 / e)) < 1e-15
    assert abs(decoder.silu(-1.0) - (-1.0) / (1.0 + e)) < 1e-15
    assert abs(decoder.silu(2.0) - 2.0 * e * e / (1.0 + e * e)) < 1e-15
    assert abs(decoder.silu(40.0) - 40.0) < 1e-12 and abs(decoder.silu(-40.0)) < 1e-15
    t = np.random.default_rng(7).normal(0, 3, 1000)
    assert np.allclose(decoder.silu(t) - decoder.silu(-t), t, rtol=0, atol=1e-12)


def _mlp_codes(seed, hidden=256, inter=384, out=128):
    rng = rng_for(seed)
    gate = draw_codes(rng, inter, hidden, 32, 5)
    up = draw_codes(rng, inter, hidden, 64, 4)
    down = draw_codes(rng, out, inter, 16, 6)
    x = draw_x(rng, (hidden,))
    return gate, up, down, x


def test_swiglu_zero_gate_or_up_gives_zero():
    for which in ("gate", "up"):
        gate, up, down, x = _mlp_codes(901)
        c = gate if which == "gate" else up
        c.mu[:] = 0
        c.delta[:] = 0
        h, y = decoder.swiglu_mlp(gate, up, down, x)
        assert np.all(h == 0) and np.all(y == 0), which


def test_swiglu_intermediate_is_fp16_and_follows_gate_sign():
    gate, up, down, x = _mlp_codes(902)
    h, y = decoder.swiglu_mlp(gate, up, down, x)
    assert np.array_equal(h, h.astype(np.float16).astype(np.float64))
    g = decoder.gemv(gate, x)
    u = decoder.gemv(up, x)
    # silu(t) = t * sigmoid(t) keeps the sign of t, so h has the sign of g * u
    big = (np.abs(g) > 0.5) & (np.abs(u) > 0.05)
    assert big.sum() > 10
    assert np.all(np.sign(h[big]) == np.sign(g[big]) * np.sign(u[big]))
    assert y.shape == (down.d_out,)


# ------------------------------------------------------------------------------ producers (§3.5)

def test_rmsnorm_unit_rms_scale_invariance_and_worked_vector():
    rng = np.random.default_rng(31)
    X = rng.standard_normal((5, 64)) * 3.0
    ones = np.ones(64)
    Y = decoder.rmsnorm_permute(X, ones, 0.0)
    assert np.allclose(np.sqrt(np.mean(Y * Y, axis=1)), 1.0, rtol=1e-15, atol=0)
    assert np.allclose(decoder.rmsnorm_permute(7.5 * X, ones, 0.0), Y, rtol=1e-14, atol=0)
    # x = (3, 4, 0, 0): mean square 25/4, so x / 2.5; gamma doubles the second entry
    y = decoder.rmsnorm_permute(np.array([3.0, 4.0, 0.0, 0.0]), np.array([1.0, 2.0, 1.0, 1.0]), 0.0)
    assert np.array_equal(y, np.array([1.2, 3.2, 0.0, 0.0]))
    # eps enters under the root: x = (1, 1), eps = 3 -> x / 2
    assert np.array_equal(decoder.rmsnorm_permute(np.ones(2), np.ones(2), 3.0), np.full(2, 0.5))


def test_producers_gather_through_pi():
    """Column p of the permuted output is column pi[p] of the unpermuted one (unit probes)."""
    rng = np.random.default_rng(32)
    d = 16
    pi = rng.permutation(d)
    g = rng.lognormal(size=d)
    for c in range(d):
        x = np.zeros(d)
        x[c] = 4.0
        out = decoder.rmsnorm_permute(x, g, 0.0, pi)
        p = int(np.nonzero(pi == c)[0][0])
        assert np.nonzero(out)[0].tolist() == [p] and out[p] == 4.0 * g[c]
        G = np.zeros(d)
        G[c] = 2.0
        U = np.full(d, 3.0)
        h = decoder.silu_mul_permute(G, U, pi)
        assert np.nonzero(h)[0].tolist() == [p]
        assert h[p] == 3.0 * 2.0 / (1.0 + np.exp(-2.0))
