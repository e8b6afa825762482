"""Pins for the oracle's encoder (SAGE paper §3.1-§3.3, Appendix A.6/A.7), CPU only.

Each test checks the oracle against something other than itself: a hand-worked example of Eq. (5),
properties the paper states (one channel per energy tier, unit-mean weights, the reduction of
Eq. (6) to the cosine rule under uniform weights), brute-force minimisation, closed-form grid
bounds and exact recovery of planted matrices.
"""
import itertools
import os

import numpy as np
import pytest

from oracle import decoder, encoder


# ------------------------------------------------------------------------------ helpers

def dyadic_unit_vectors():
    """Nonnegative 8-vectors with entries a/4 and sum of squares exactly 1 (exact in fp16)."""
    out = set()
    for pattern in ((4,), (2, 2, 2, 2), (3, 2, 1, 1, 1), (2, 2, 2, 1, 1, 1, 1)):
        base = list(pattern) + [0] * (8 - len(pattern))
        for perm in set(itertools.permutations(base)):
            out.add(perm)
    vecs = np.array(sorted(out), dtype=np.float64) / 4.0
    assert np.all(np.sum(vecs ** 2, axis=1) == 1.0)
    return vecs


def planted_matrix(d_out, d_in, K, V, pi, seed):
    """A matrix exactly representable in split (K, V): K dyadic unit codewords (each used), exact
    fp16 grids whose groups contain both code 0 and code 2^V - 1, random signs; returned in
    original column order together with the planted permuted-order pieces."""
    rng = np.random.default_rng(seed)
    allv = dyadic_unit_vectors()
    C = allv[rng.choice(allv.shape[0], size=K, replace=False)]
    m = d_in // 8
    ng = d_in // 128
    n = d_out * m
    z = rng.permutation(np.arange(n) % K).reshape(d_out, m)
    qmax = (1 << V) - 1
    q = rng.integers(0, qmax + 1, size=(d_out, m))
    q[:, 0::16] = 0
    q[:, 1::16] = qmax
    mu = rng.integers(1, 64, size=(d_out, ng)) / 64.0
    delta = rng.integers(1, 32, size=(d_out, ng)) / 256.0
    r = mu[:, np.arange(m) // 16] + q * delta[:, np.arange(m) // 16]
    sign = np.where(rng.integers(0, 2, size=(d_out, m, 8)) == 1, -1.0, 1.0)
    Wp = (r[..., None] * (sign * C[z])).reshape(d_out, d_in)
    W = np.empty_like(Wp)
    W[:, pi] = Wp
    return W, dict(C=C, z=z, q=q, mu=mu, delta=delta)


# ------------------------------------------------------------------------------ §3.2 energy

def test_channel_energy_mean_square():
    X = np.array([[1.0, -2.0, 0.0], [3.0, 2.0, 0.5]])
    assert np.array_equal(encoder.channel_energy(X), np.array([5.0, 4.0, 0.125]))


# ------------------------------------------------------------------------------ §3.2 Eq. (5)

def _read_golden(path):
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            vals[k.strip()] = v.split()
    return vals


def test_esg_worked_example(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "esg_pi_d16.txt"))
    e = np.array([float(t) for t in g["energies"]])
    pi = encoder.esg_permutation(e)
    assert pi.tolist() == [int(t) for t in g["pi"]]


@pytest.mark.parametrize("d_in", [16, 128, 1024, 2560])
def test_esg_one_channel_per_tier(d_in):
    rng = np.random.default_rng(d_in)
    e = rng.lognormal(size=d_in)
    pi = encoder.esg_permutation(e)
    m = d_in // 8
    assert np.array_equal(np.sort(pi), np.arange(d_in))          # bijective
    rank = np.empty(d_in, dtype=np.int64)
    rank[np.argsort(-e, kind="stable")] = np.arange(d_in)          # 0 = highest energy
    tiers = rank[pi].reshape(m, 8) // m
    assert np.array_equal(tiers, np.broadcast_to(np.arange(8), (m, 8)))
    # positions inside each subvector run from higher to lower energy
    ep = e[pi].reshape(m, 8)
    assert np.all(np.diff(ep, axis=1) <= 0)
    # subvector j holds the j-th member of every tier
    assert np.array_equal(rank[pi].reshape(m, 8) % m,
                          np.broadcast_to(np.arange(m)[:, None], (m, 8)))


def test_esg_ties_keep_channel_order():
    e = np.ones(16)
    pi = encoder.esg_permutation(e)
    # sigma is the identity, so pi[8j + t] = 2t + j
    assert pi.tolist() == [0, 2, 4, 6, 8, 10, 12, 14, 1, 3, 5, 7, 9, 11, 13, 15]


# ------------------------------------------------------------------------------ §3.2 Eq. (4)

def test_position_weights_unit_mean_and_ratios():
    rng = np.random.default_rng(1)
    e = rng.lognormal(size=64)
    for gamma in (0.5, 0.75, 1.0):
        om = encoder.position_weights(e, gamma)
        assert np.allclose(om.mean(axis=1), 1.0, rtol=0, atol=1e-14)
        ee = e.reshape(-1, 8)
        assert np.allclose(om[:, 0] / om[:, 3], (ee[:, 0] / ee[:, 3]) ** gamma, rtol=1e-12)


def test_position_weights_equal_energy_and_gamma_zero():
    assert np.array_equal(encoder.position_weights(np.full(32, 3.7), 0.75), np.ones((4, 8)))
    rng = np.random.default_rng(2)
    assert np.array_equal(encoder.position_weights(rng.lognormal(size=32), 0.0), np.ones((4, 8)))
    assert np.array_equal(encoder.position_weights(np.zeros(16), 0.75), np.ones((2, 8)))


# ------------------------------------------------------------------------------ §3.2 Eq. (6)

def test_assign_uniform_weights_is_cosine_rule():
    rng = np.random.default_rng(3)
    P = np.abs(rng.standard_normal((500, 8)))
    C = np.abs(rng.standard_normal((64, 8)))
    C /= np.linalg.norm(C, axis=1, keepdims=True)
    z, r = encoder.assign(P, np.ones_like(P), C)
    d = P / np.linalg.norm(P, axis=1, keepdims=True)
    cos = d @ C.T
    assert np.array_equal(z, np.argmax(cos, axis=1))
    assert np.allclose(r, np.sum(P * C[z], axis=1), rtol=1e-13)   # r_tilde = |w|^T c_z


def test_assign_matches_brute_force_minimisation():
    """Eq. (6) must pick the codeword whose best radius gives the smallest weighted error."""
    rng = np.random.default_rng(4)
    for _ in range(40):
        p = np.abs(rng.standard_normal(8))
        w = rng.uniform(0.1, 3.0, size=8)
        C = np.abs(rng.standard_normal((6, 8)))
        C /= np.linalg.norm(C, axis=1, keepdims=True)
        rs = np.linspace(0.0, 2.0 * np.linalg.norm(p), 200001)
        best = []
        for k in range(6):
            loss = ((p[None, :] - rs[:, None] * C[k][None, :]) ** 2 * w[None, :]).sum(axis=1)
            i = np.argmin(loss)
            best.append((loss[i], rs[i]))
        kstar = int(np.argmin([b[0] for b in best]))
        z, r = encoder.assign(p[None], w[None], C)
        losses = sorted(b[0] for b in best)
        if losses[1] - losses[0] > 1e-6:       # skip near-ties the grid cannot separate
            assert z[0] == kstar
        assert abs(r[0] - best[z[0]][1]) <= 2.0 * (rs[1] - rs[0])


def test_assign_exact_recovery():
    rng = np.random.default_rng(5)
    C = dyadic_unit_vectors()[:40]
    z0 = rng.integers(0, 40, size=300)
    r0 = rng.integers(1, 200, size=300) / 64.0
    P = r0[:, None] * C[z0]
    w = rng.uniform(0.2, 2.0, size=P.shape)
    z, r = encoder.assign(P, w, C)
    assert np.array_equal(z, z0)
    assert np.allclose(r, r0, rtol=1e-14, atol=0)


def test_assign_zero_subvector():
    C = dyadic_unit_vectors()[:8]
    z, r = encoder.assign(np.zeros((3, 8)), np.ones((3, 8)), C)
    assert np.array_equal(z, [0, 0, 0]) and np.array_equal(r, [0, 0, 0])


def test_error_decomposition_identity():
    """Appendix A.6 Eq. (11): ||p - r c||^2 = ||p||^2 - (p.c)^2 + (r - p.c)^2 for unit c."""
    rng = np.random.default_rng(6)
    for _ in range(100):
        p = np.abs(rng.standard_normal(8))
        c = np.abs(rng.standard_normal(8))
        c /= np.linalg.norm(c)
        rhat = rng.uniform(0, 3)
        lhs = np.sum((p - rhat * c) ** 2)
        pc = p @ c
        rhs = p @ p - pc ** 2 + (rhat - pc) ** 2
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
        z, r = encoder.assign(p[None], np.ones((1, 8)), c[None])
        assert abs(r[0] - pc) <= 1e-14 * pc  # the continuous optimum is p.c


# ------------------------------------------------------------------------------ k-means

def test_kmeans_invariants():
    rng = np.random.default_rng(7)
    P = np.abs(rng.standard_normal((4000, 8)) * rng.lognormal(size=8))
    w = np.broadcast_to(rng.uniform(0.3, 2.0, size=8), P.shape).copy()
    w /= w.mean(axis=1, keepdims=True)
    C, hist = encoder.kmeans(P, w, 32, 12, np.random.default_rng(0))
    assert np.all(C >= 0)
    assert np.allclose(np.linalg.norm(C, axis=1), 1.0, atol=1e-12)
    assert np.all(np.diff(hist) <= 1e-9 * hist[0])


def test_kmeans_planted_fixed_point():
    rng = np.random.default_rng(8)
    allv = dyadic_unit_vectors()
    C0 = allv[rng.choice(allv.shape[0], size=16, replace=False)]
    z0 = np.arange(800) % 16
    P = rng.uniform(0.5, 2.0, size=800)[:, None] * C0[z0]
    C, hist = encoder.kmeans(P, np.ones_like(P), 16, 5, np.random.default_rng(1))
    assert sorted(map(tuple, np.round(C, 12))) == sorted(map(tuple, C0))
    assert hist[-1] <= 1e-20


# ------------------------------------------------------------------------------ Eq. (2), Eq. (14)

@pytest.mark.parametrize("V", [2, 3, 4, 5, 6])
def test_radius_grid_bounds(V):
    rng = np.random.default_rng(V)
    r = rng.uniform(0.0, 2.0, size=(7, 64))
    mu, delta, q = encoder.radius_grid(r, V, store_fp16=False)
    qmax = (1 << V) - 1
    assert q.min() >= 0 and q.max() <= qmax
    g = np.arange(64) // 16
    rhat = mu[:, g] + q * delta[:, g]
    assert np.all(np.abs(rhat - r) <= delta[:, g] / 2 * (1 + 1e-12))
    rg = r.reshape(7, 4, 16)
    qg = q.reshape(7, 4, 16)
    assert np.all(qg[np.arange(7)[:, None], np.arange(4)[None], rg.argmin(axis=2)] == 0)
    assert np.all(qg[np.arange(7)[:, None], np.arange(4)[None], rg.argmax(axis=2)] == qmax)
    # stored grids: q is computed against the fp16 values and stays within range
    mu16, d16, q16 = encoder.radius_grid(r, V)
    assert np.array_equal(mu16, mu16.astype(np.float16).astype(np.float64))
    assert q16.min() >= 0 and q16.max() <= qmax
    rhat16 = mu16[:, g] + q16 * d16[:, g]
    slack = np.abs(mu16 - mu)[:, g] + qmax * np.abs(d16 - delta)[:, g]
    assert np.all(np.abs(rhat16 - r) <= d16[:, g] * 0.5 + slack + 1e-12)


def test_radius_grid_equal_radii_reconstruct_common_value():
    """Appendix A.6: coinciding radii in a group reconstruct to their common value."""
    r = np.full((2, 32), 0.7071)
    mu, delta, q = encoder.radius_grid(r, 4, store_fp16=False)
    assert np.all(delta == 0) and np.all(q == 0) and np.all(mu == 0.7071)
    mu16, d16, q16 = encoder.radius_grid(r, 4)
    assert np.all(q16 == 0) and np.all(mu16 == np.float64(np.float16(0.7071)))


# ------------------------------------------------------------------------------ encode / ABS

@pytest.mark.parametrize("K,V", [(16, 6), (64, 4), (256, 2)])
def test_encode_exact_recovery_planted(K, V):
    rng = np.random.default_rng(K)
    d_out, d_in = 48, 256
    e = rng.lognormal(size=d_in)
    pi = encoder.esg_permutation(e)
    W, parts = planted_matrix(d_out, d_in, K, V, pi, seed=K + V)
    enc = encoder.encode_matrix(W, e, K, V, gamma=0.75, iters=4, seed=3)
    assert np.array_equal(enc["pi"], pi)
    assert np.array_equal(decoder.decode(enc), W)          # bit-exact in float64
    # the encoder sees the planted structure in the permuted order
    assert np.array_equal(decoder.radii(enc), parts["mu"][:, np.arange(32) // 16]
                          + parts["q"] * parts["delta"][:, np.arange(32) // 16])


def test_encode_fields_ranges_and_signs():
    rng = np.random.default_rng(11)
    W = rng.standard_normal((16, 128)) * 0.02
    W[0, :8] = [-1, 2, -3, 4, -5, 6, -7, 0]
    enc = encoder.encode_matrix(W, None, 32, 5, esg=False, iters=3)
    assert enc["signs"][0, 0] == 0b01010101
    assert enc["idx"].max() < 32 and enc["rcode"].max() < 32
    assert enc["codebook"].shape == (32, 8) and enc["mu"].shape == (16, 1)


def test_abs_score_basic():
    rng = np.random.default_rng(12)
    W = rng.standard_normal((8, 128))
    e = rng.lognormal(size=128)
    assert encoder.abs_score(W, W, e) == 0.0
    Wn = W.copy()
    Wn[:, 5] = 0.0
    s = encoder.abs_score(W, Wn, e)
    assert abs(s - e[5] * np.sum(W[:, 5] ** 2) / np.sum(e * np.sum(W ** 2, axis=0))) < 1e-15


@pytest.mark.parametrize("planted", [(256, 2), (64, 4)])
def test_abs_selects_planted_split(planted):
    K0, V0 = planted
    rng = np.random.default_rng(K0)
    d_out, d_in = 32, 512
    e = rng.lognormal(size=d_in)
    pi = encoder.esg_permutation(e)
    W, _ = planted_matrix(d_out, d_in, K0, V0, pi, seed=21)
    best, scores, enc = encoder.abs_select(W, e, [(64, 4), (128, 3), (256, 2)],
                                           gamma=0.75, iters=3, seed=5)
    assert best == planted
    assert scores[planted] == 0.0
    assert all(s > 0 for k, s in scores.items() if k != planted)


@pytest.mark.slow
def test_single_matrix_calibration_encode():
    from workloads import single_matrix_calib
    cfg = single_matrix_calib()
    e = encoder.channel_energy(cfg.X_cal)
    enc = encoder.encode_matrix(cfg.W, e, cfg.K, cfg.V, gamma=cfg.gamma, iters=cfg.kmeans_iters,
                                samples=cfg.kmeans_samples, seed=cfg.seed)
    hist = enc["_kmeans_history"]
    assert np.all(np.diff(hist) <= 1e-9 * hist[0])
    assert enc["idx"].max() < 64 and enc["rcode"].max() < 16
    cb = enc["codebook"].view(np.float16).astype(np.float64)
    assert np.all(cb >= 0)
    assert np.all(np.abs(np.linalg.norm(cb, axis=1) - 1.0) <= 2.0 ** -10)
    s = encoder.abs_score(cfg.W, decoder.decode(enc), e)
    assert 0.0 < s < 0.5


# ------------------------------------------------------------------------------ fixed-order Eq. (6)

def _assign_python(P, omega, C):
    """Eq. (6) by plain Python float loops in the order assign_ordered states (left to right)."""
    z_out, r_out = [], []
    for p, w in zip(P.tolist(), omega.tolist()):
        t = [w[i] * p[i] for i in range(8)]
        best, bz, bnum, bden = None, 0, 0.0, 0.0
        for k, c in enumerate(C.tolist()):
            num = t[0] * c[0]
            den = w[0] * (c[0] * c[0])
            for i in range(1, 8):
                num = num + t[i] * c[i]
                den = den + w[i] * (c[i] * c[i])
            score = (num * num) / den if den > 0 else 0.0
            if best is None or score > best:
                best, bz, bnum, bden = score, k, num, den
        z_out.append(bz)
        r_out.append(bnum / bden if bden > 0 else 0.0)
    return np.array(z_out), np.array(r_out)


def test_assign_ordered_matches_python_loop_bit_for_bit():
    rng = np.random.default_rng(21)
    n, K = 60, 16
    P = np.abs(rng.standard_normal((n, 8)))
    P[3] = 0.0                                   # zero subvector
    omega = rng.lognormal(size=(n, 8))
    omega[5, :4] = 0.0                           # weights that vanish on part of the subvector
    C = np.abs(rng.standard_normal((K, 8)))
    C /= np.linalg.norm(C, axis=1, keepdims=True)
    C[2, 4:] = 0.0                               # a codeword with zero weighted norm for row 5
    C = C.astype(np.float16).astype(np.float64)
    omega[5, 4:] = rng.lognormal(size=4)
    z, r = encoder.assign_ordered(P, omega, C)
    zp, rp = _assign_python(P, omega, C)
    assert np.array_equal(z, zp)
    assert np.array_equal(r.view(np.uint64), rp.view(np.uint64))
    assert z[3] == 0 and r[3] == 0.0


def test_assign_ordered_agrees_with_assign():
    rng = np.random.default_rng(22)
    n, K = 20000, 64
    P = np.abs(rng.standard_normal((n, 8)))
    omega = rng.lognormal(size=(n, 8))
    C = np.abs(rng.standard_normal((K, 8)))
    C = (C / np.linalg.norm(C, axis=1, keepdims=True)).astype(np.float16).astype(np.float64)
    z1, r1 = encoder.assign(P, omega, C)
    z2, r2 = encoder.assign_ordered(P, omega, C)
    num = (omega * P) @ C.T
    den = omega @ (C * C).T
    score = num * num / den
    rows = np.arange(n)
    differ = z1 != z2
    # a different choice is only allowed between scores equal to rounding
    assert np.all(np.abs(score[rows, z1] - score[rows, z2])[differ]
                  <= 1e-12 * score[rows, z1][differ])
    same = ~differ
    assert np.all(np.abs(r1 - r2)[same] <= 1e-14 * np.abs(r1)[same])


@pytest.mark.parametrize("K,V", [(16, 6), (64, 4), (256, 2)])
def test_encode_fields_exact_recovery_planted(K, V):
    rng = np.random.default_rng(K + 100)
    d_out, d_in = 24, 384
    e = rng.lognormal(size=d_in)
    pi = encoder.esg_permutation(e)
    W, parts = planted_matrix(d_out, d_in, K, V, pi, seed=K + V + 1)
    omega = encoder.position_weights(e[pi], 0.75).reshape(-1)
    enc = encoder.encode_fields(W, pi, omega, parts["C"].astype(np.float16), V)
    assert np.array_equal(enc["idx"], parts["z"])
    assert np.array_equal(enc["rcode"], parts["q"])
    assert np.array_equal(enc["mu"].view(np.float16).astype(np.float64), parts["mu"])
    assert np.array_equal(enc["delta"].view(np.float16).astype(np.float64), parts["delta"])
    assert np.array_equal(decoder.decode(enc), W)          # bit-exact in float64
    Wp = W[:, pi].reshape(d_out, -1, 8)
    assert np.array_equal(enc["signs"], encoder.sign_bytes(Wp))


def test_encode_fields_reproduces_encode_matrix_with_its_codebook():
    """With the codebook, permutation and weights the full encoder produced, the fixed-codebook
    encoder gives the same fields (the two differ only in the summation order of Eq. (6))."""
    rng = np.random.default_rng(23)
    d_out, d_in = 32, 256
    W = rng.standard_normal((d_out, d_in)) * 0.02
    e = rng.lognormal(size=d_in)
    full = encoder.encode_matrix(W, e, 64, 4, gamma=0.75, iters=5, seed=4)
    omega = encoder.position_weights(e[full["pi"]], 0.75).reshape(-1)
    fixed = encoder.encode_fields(W, full["pi"], omega, full["codebook"], 4)
    for key in ("signs", "idx", "rcode", "mu", "delta"):
        assert np.array_equal(fixed[key], full[key]), key
