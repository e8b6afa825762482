"""Encoder side of the SAGE quantiser in float64 (TEST INFRASTRUCTURE ONLY; see oracle/__init__).

Written from "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World Usability":
  channel_energy      §3.2: the energy of input channel c is the mean of x_c^2 over calibration tokens.
  esg_permutation     §3.2, Eq. (5): sort channels by decreasing energy, cut the sorted list into 8
                      tiers of m = d_in/8, and let subvector j take the j-th channel of every tier,
                      tier 1 first.
  position_weights    §3.2, Eq. (4): omega_i = e_{a_i}^gamma divided by the subvector's mean of
                      e^gamma, so the eight weights average to one.
  assign              §3.2, Eq. (6): weighted closed-form radius and argmax of the substituted score.
  assign_ordered      the same, with every 8-term sum taken left to right (i = 0..7) and no fused
                      operations, so that a second implementation can reproduce each rounding and
                      therefore each argmax decision exactly.
  encode_fields       §3.2 Eq. (6) with §3.1 Eq. (2) / Appendix A.6 Eq. (14): the final assignment
                      and radius grid of one matrix for a given fp16 codebook, permutation and
                      position weights (no codebook fit), built on assign_ordered.
  kmeans              §3.2 + §4.1: activation-weighted spherical k-means (20 iterations on up to
                      65,536 sampled subvectors by default).
  radius_grid         §3.1 Eq. (2) with Appendix A.6 Eq. (14): per 128-weight group, offset = min
                      fitted radius, step = range / (2^V - 1), code = clip(round((r - mu)/delta)).
  encode_matrix       Appendix A.7, the per-matrix body for one (K, V).
  abs_score           §3.3, Eq. (8): energy-weighted relative column error in original order.
  abs_select          §3.3, Eq. (9): argmin of the score over the candidate splits.

Readings where the paper is silent (each one also listed in the design notes):
  sign(0)          a zero weight gets sign bit 0 (positive); it contributes nothing either way.
  sign bits        bit i of the sign byte belongs to position i of the subvector; 1 means negative.
  energy ties      equal energies keep ascending channel order in the sort.
  pi direction     gather form: pi[p] is the original channel placed at permuted position p, so the
                   permuted matrix is W[:, pi] and the permuted input is x[pi].
  zero energies    a subvector whose e^gamma values are all zero gets omega = 1 everywhere.
  k-means init     the first K distinct nonzero directions met in a seeded random order of the
                   sampled subvectors (random |N| directions fill up if fewer exist).
  k-means update   with assignments and radii fixed, each coordinate of the cluster centre is set
                   to its exact weighted least-squares value sum(w r p_i) / sum(w r^2) (unweighted
                   if that denominator is zero), then the centre is scaled to unit length; an
                   empty cluster keeps its previous codeword.
  argmax ties      the lowest index wins (codeword) / the first listed split wins (ABS).
  rounding         round half to even.
  grid precision   mu and delta are stored in fp16 and the codes are computed against the stored
                   fp16 values; a zero stored step gives code 0.
  codebook         stored in fp16; the final assignment uses the fp16 codebook.

Parity status:
  channel_energy, esg_permutation, position_weights, assign, radius_grid, abs_score: pinned by the
    CPU tests (worked example of Eq. (5), closed forms, brute-force minimisation, special cases).
  assign_ordered: pinned bit for bit by a pure-Python loop over the same operations, and against
    assign (same decisions away from near-ties, radii within a few ulps).
  encode_fields: pinned by exact recovery of planted matrices for a given codebook.
  kmeans: PARITY UNPINNED. The paper gives neither its initialisation nor its update rule, so only
    invariants are checked (nonnegative unit codewords, non-increasing objective, planted fixed
    point).
  encode_matrix, abs_select: pinned by exact recovery of planted matrices; on generic data they
    inherit the unpinned k-means.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import decoder

V_SUB = 8          # subvector length v (§3.1)
G_WEIGHTS = 128    # weights per radius group (§3.1, Appendix A.6)


# ---------------------------------------------------------------------------------------------
# §3.2: energies, ESG permutation, position weights
# ---------------------------------------------------------------------------------------------

def channel_energy(X_cal: np.ndarray) -> np.ndarray:
    """e_c = mean over calibration tokens of x_c^2. X_cal is [tokens, d_in]."""
    X = np.asarray(X_cal, dtype=np.float64)
    return np.mean(X * X, axis=0)


def esg_permutation(e: np.ndarray, v: int = V_SUB) -> np.ndarray:
    """Eq. (5) in 0-based form: pi[j*v + t] = sigma[t*m + j] for j < m = d_in/v and t < v, where
    sigma lists channels by decreasing energy (ties: lower channel index first)."""
    e = np.asarray(e, dtype=np.float64)
    d = e.size
    if d % v:
        raise ValueError("d_in must be a multiple of v")
    m = d // v
    sigma = sorted(range(d), key=lambda c: (-e[c], c))
    pi = np.empty(d, dtype=np.int64)
    for j in range(m):
        for t in range(v):
            pi[j * v + t] = sigma[t * m + j]
    return pi


def position_weights(e_perm: np.ndarray, gamma: float, v: int = V_SUB) -> np.ndarray:
    """Eq. (4) weights for every column subvector of the permuted order: [d_in/v, v]."""
    a = np.asarray(e_perm, dtype=np.float64).reshape(-1, v) ** gamma
    mean = a.mean(axis=1)
    omega = np.ones_like(a)
    ok = mean > 0
    omega[ok] = a[ok] / mean[ok, None]
    return omega


# ---------------------------------------------------------------------------------------------
# §3.2 Eq. (6): assignment with a continuous radius
# ---------------------------------------------------------------------------------------------

def assign(P: np.ndarray, omega: np.ndarray, C: np.ndarray,
           chunk: int = 8192) -> Tuple[np.ndarray, np.ndarray]:
    """For each magnitude vector p (rows of P) with weights omega (same shape), pick
    z = argmax_k (sum_i w_i p_i c_ki)^2 / sum_i w_i c_ki^2 and return it with
    r_tilde = sum_i w_i p_i c_zi / sum_i w_i c_zi^2. A codeword whose weighted norm is zero scores 0.
    """
    P = np.asarray(P, dtype=np.float64)
    W = np.asarray(omega, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    n = P.shape[0]
    z = np.empty(n, dtype=np.int64)
    r = np.empty(n, dtype=np.float64)
    C2 = C * C
    for s in range(0, n, chunk):
        p, w = P[s:s + chunk], W[s:s + chunk]
        num = (w * p) @ C.T            # [n, K]
        den = w @ C2.T                 # [n, K]
        score = np.zeros_like(num)
        pos = den > 0
        score[pos] = num[pos] * num[pos] / den[pos]
        zz = np.argmax(score, axis=1)  # first maximum on ties
        rows = np.arange(zz.size)
        nz, dz = num[rows, zz], den[rows, zz]
        rr = np.zeros_like(nz)
        ok = dz > 0
        rr[ok] = nz[ok] / dz[ok]
        z[s:s + chunk] = zz
        r[s:s + chunk] = rr
    return z, r


def assign_ordered(P: np.ndarray, omega: np.ndarray, C: np.ndarray,
                   chunk: int = 4096) -> Tuple[np.ndarray, np.ndarray]:
    """Eq. (6) like `assign`, with a fixed evaluation order: t_i = w_i p_i; num_k = t_0 c_k0, then
    num_k = num_k + t_i c_ki for i = 1..7; den_k likewise from w_i (c_ki c_ki); score_k =
    (num_k num_k) / den_k (0 where den_k is 0); z = first maximum; r = num_z / den_z (0 where
    den_z is 0). Every step is one IEEE double operation (numpy element-wise ops do not fuse)."""
    P = np.asarray(P, dtype=np.float64)
    W = np.asarray(omega, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    C2 = C * C
    n, v = P.shape
    z = np.empty(n, dtype=np.int64)
    r = np.empty(n, dtype=np.float64)
    for s in range(0, n, chunk):
        t = W[s:s + chunk] * P[s:s + chunk]
        w = W[s:s + chunk]
        num = t[:, 0:1] * C[None, :, 0]
        den = w[:, 0:1] * C2[None, :, 0]
        for i in range(1, v):
            num = num + t[:, i:i + 1] * C[None, :, i]
            den = den + w[:, i:i + 1] * C2[None, :, i]
        pos = den > 0
        score = np.where(pos, (num * num) / np.where(pos, den, 1.0), 0.0)
        zz = np.argmax(score, axis=1)
        rows = np.arange(zz.size)
        nz, dz = num[rows, zz], den[rows, zz]
        z[s:s + chunk] = zz
        r[s:s + chunk] = np.where(dz > 0, nz / np.where(dz > 0, dz, 1.0), 0.0)
    return z, r


def weighted_objective(P, omega, C, z, r) -> float:
    """Sum over subvectors of Eq. (4)'s loss with the given assignment and radii."""
    rec = r[:, None] * np.asarray(C, dtype=np.float64)[z]
    return float(np.sum(omega * (P - rec) ** 2))


# ---------------------------------------------------------------------------------------------
# §3.2 / §4.1: activation-weighted spherical k-means
# ---------------------------------------------------------------------------------------------

def _init_codebook(P: np.ndarray, K: int, rng: np.random.Generator) -> np.ndarray:
    chosen: List[np.ndarray] = []
    for i in rng.permutation(P.shape[0]):
        nrm = np.linalg.norm(P[i])
        if nrm == 0:
            continue
        d = P[i] / nrm
        if chosen and np.min(np.linalg.norm(np.asarray(chosen) - d, axis=1)) < 1e-9:
            continue
        chosen.append(d)
        if len(chosen) == K:
            break
    while len(chosen) < K:
        g = np.abs(rng.standard_normal(P.shape[1]))
        chosen.append(g / np.linalg.norm(g))
    return np.asarray(chosen, dtype=np.float64)


def kmeans(P: np.ndarray, omega: np.ndarray, K: int, iters: int,
           rng: np.random.Generator) -> Tuple[np.ndarray, List[float]]:
    """Returns the fitted float64 codebook [K, v] and the objective after each assignment step
    (iters + 1 values: one per iteration, then one with the final codebook)."""
    P = np.asarray(P, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    C = _init_codebook(P, K, rng)
    history: List[float] = []
    for _ in range(iters):
        z, r = assign(P, omega, C)
        history.append(weighted_objective(P, omega, C, z, r))
        for k in range(K):
            mem = z == k
            if not np.any(mem):
                continue
            w, p, rr = omega[mem], P[mem], r[mem][:, None]
            num_w = np.sum(w * rr * p, axis=0)
            den_w = np.sum(w * rr * rr, axis=0)
            num_u = np.sum(rr * p, axis=0)
            den_u = np.sum(rr * rr, axis=0)
            u = np.zeros(P.shape[1])
            for i in range(P.shape[1]):
                if den_w[i] > 0:
                    u[i] = num_w[i] / den_w[i]
                elif den_u[i] > 0:
                    u[i] = num_u[i] / den_u[i]
            nrm = np.linalg.norm(u)
            if nrm > 0:
                C[k] = u / nrm
    z, r = assign(P, omega, C)
    history.append(weighted_objective(P, omega, C, z, r))
    return C, history


# ---------------------------------------------------------------------------------------------
# §3.1 Eq. (2) and Appendix A.6 Eq. (14): the shared radius grid
# ---------------------------------------------------------------------------------------------

def radius_grid(r_tilde: np.ndarray, V: int, subvecs_per_group: int = G_WEIGHTS // V_SUB,
                store_fp16: bool = True) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """r_tilde is [d_out, d_in/8]. Per group of 16 consecutive subvectors of a row:
    mu = min, delta = (max - mu)/(2^V - 1), then (optionally) both rounded to fp16, then
    q = clip(rint((r - mu)/delta), 0, 2^V - 1), with q = 0 where delta is zero.
    Returns mu, delta (float64 values of what is stored) of shape [d_out, groups] and q."""
    r = np.asarray(r_tilde, dtype=np.float64)
    d_out, m = r.shape
    if m % subvecs_per_group:
        raise ValueError("row length must be a whole number of groups")
    rg = r.reshape(d_out, m // subvecs_per_group, subvecs_per_group)
    qmax = (1 << V) - 1
    mu = rg.min(axis=2)
    delta = (rg.max(axis=2) - mu) / qmax
    if store_fp16:
        mu = mu.astype(np.float16).astype(np.float64)
        delta = delta.astype(np.float16).astype(np.float64)
    if not (np.all(np.isfinite(mu)) and np.all(np.isfinite(delta))):
        raise OverflowError("radius grid does not fit the storage precision")
    q = np.zeros(rg.shape, dtype=np.int64)
    ok = delta > 0
    t = (rg - mu[..., None]) / np.where(ok, delta, 1.0)[..., None]
    q = np.where(ok[..., None], np.clip(np.rint(t), 0, qmax), 0).astype(np.int64)
    return mu, delta, q.reshape(d_out, m)


# ---------------------------------------------------------------------------------------------
# Appendix A.7: one matrix, one (K, V)
# ---------------------------------------------------------------------------------------------

def sign_bytes(Wsub: np.ndarray) -> np.ndarray:
    """Wsub [..., 8] -> uint8 whose bit i is 1 iff element i is negative."""
    neg = (np.asarray(Wsub) < 0).astype(np.uint16)
    out = np.zeros(neg.shape[:-1], dtype=np.uint16)
    for i in range(neg.shape[-1]):
        out |= neg[..., i] << i
    return out.astype(np.uint8)


def encode_matrix(W: np.ndarray, e: Optional[np.ndarray], K: int, V: int, gamma: float = 0.75,
                  esg: bool = True, iters: int = 20, samples: int = 65536,
                  seed: int = 0, pi: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Encode W [d_out, d_in] for split (K, V). `e` are the calibration energies (None means equal
    energies). Returns the stored fields (see workloads' field conventions) plus float64
    intermediates under keys starting with an underscore."""
    W = np.asarray(W, dtype=np.float64)
    d_out, d_in = W.shape
    if d_in % G_WEIGHTS:
        raise ValueError("d_in must be a multiple of 128")
    e = np.ones(d_in) if e is None else np.asarray(e, dtype=np.float64)
    if pi is None:
        pi = esg_permutation(e) if esg else np.arange(d_in)
    pi = np.asarray(pi, dtype=np.int64)
    Wp = W[:, pi]
    ep = e[pi]
    m = d_in // V_SUB
    Wsub = Wp.reshape(d_out, m, V_SUB)
    P = np.abs(Wsub)
    omega = np.broadcast_to(position_weights(ep, gamma)[None], (d_out, m, V_SUB))
    Pf = P.reshape(-1, V_SUB)
    Of = omega.reshape(-1, V_SUB)
    rng = np.random.default_rng(seed)
    n = Pf.shape[0]
    take = rng.choice(n, size=min(samples, n), replace=False)
    C64, hist = kmeans(Pf[take], Of[take], K, iters, rng)
    C16 = C64.astype(np.float16)
    z, r = assign(Pf, Of, C16.astype(np.float64))
    mu, delta, q = radius_grid(r.reshape(d_out, m), V)
    return {
        "signs": sign_bytes(Wsub),
        "idx": z.reshape(d_out, m).astype(np.uint8),
        "rcode": q.astype(np.uint8),
        "mu": mu.astype(np.float16).view(np.uint16),
        "delta": delta.astype(np.float16).view(np.uint16),
        "codebook": C16.view(np.uint16),
        "pi": pi.astype(np.int32),
        "K": K, "V": V, "d_out": d_out, "d_in": d_in,
        "_r_tilde": r.reshape(d_out, m), "_kmeans_history": np.asarray(hist),
        "_codebook64": C64,
    }


def encode_fields(W: np.ndarray, pi: np.ndarray, omega: np.ndarray, codebook16: np.ndarray,
                  V: int) -> Dict[str, np.ndarray]:
    """The stored fields of W [d_out, d_in] (original column order) for a given fp16 codebook
    [K, 8] (uint16 bits or float16 values), permutation pi (gather form) and position weights
    omega [d_in] in permuted order: signs, idx = z and rcode = q from Eq. (6) evaluated with
    `assign_ordered` on the fp16 codebook, then the per-group fp16 grid of Eq. (2) / Eq. (14)."""
    W = np.asarray(W, dtype=np.float64)
    d_out, d_in = W.shape
    if d_in % G_WEIGHTS:
        raise ValueError("d_in must be a multiple of 128")
    C16 = np.asarray(codebook16)
    C16 = C16.view(np.float16) if C16.dtype == np.uint16 else C16.astype(np.float16)
    C = C16.astype(np.float64).reshape(-1, V_SUB)
    pi = np.asarray(pi, dtype=np.int64)
    m = d_in // V_SUB
    Wsub = W[:, pi].reshape(d_out, m, V_SUB)
    P = np.abs(Wsub).reshape(-1, V_SUB)
    om = np.broadcast_to(np.asarray(omega, dtype=np.float64).reshape(1, m, V_SUB),
                         (d_out, m, V_SUB)).reshape(-1, V_SUB)
    z, r = assign_ordered(P, om, C)
    mu, delta, q = radius_grid(r.reshape(d_out, m), V)
    return {
        "signs": sign_bytes(Wsub),
        "idx": z.reshape(d_out, m).astype(np.uint8),
        "rcode": q.astype(np.uint8),
        "mu": mu.astype(np.float16).view(np.uint16),
        "delta": delta.astype(np.float16).view(np.uint16),
        "codebook": C16.reshape(-1, V_SUB).view(np.uint16),
        "pi": pi.astype(np.int32),
        "K": C.shape[0], "V": V, "d_out": d_out, "d_in": d_in,
        "_r_tilde": r.reshape(d_out, m),
    }


# ---------------------------------------------------------------------------------------------
# §3.3: Adaptive Bit Split
# ---------------------------------------------------------------------------------------------

def abs_score(W: np.ndarray, W_hat: np.ndarray, e: np.ndarray) -> float:
    """Eq. (8): sum_c e_c ||W_:,c - What_:,c||^2 / sum_c e_c ||W_:,c||^2 (original column order)."""
    W = np.asarray(W, dtype=np.float64)
    Wh = np.asarray(W_hat, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    num = np.sum(e * np.sum((W - Wh) ** 2, axis=0))
    den = np.sum(e * np.sum(W ** 2, axis=0))
    return float(num / den)


def abs_select(W: np.ndarray, e: np.ndarray, splits: Sequence[Tuple[int, int]],
               **kw) -> Tuple[Tuple[int, int], Dict[Tuple[int, int], float], Dict]:
    """Eq. (9): encode W with every split, score each decode, keep the first minimum."""
    scores: Dict[Tuple[int, int], float] = {}
    encs: Dict[Tuple[int, int], Dict] = {}
    for (K, V) in splits:
        enc = encode_matrix(W, e, K, V, **kw)
        scores[(K, V)] = abs_score(W, decoder.decode(enc), e)
        encs[(K, V)] = enc
    best = None
    for s in splits:
        if best is None or scores[s] < scores[best]:
            best = s
    return best, scores, encs[best]
