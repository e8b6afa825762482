"""Seeded synthetic inputs for the SAGE decode path.

This module only draws random inputs. It is shared by the tests, the benchmark and the scripts that
write stored expected values, and it holds none of the quantiser's arithmetic: no channel energies,
no permutation built from energies, no codeword assignment, no radius-grid fitting, no decoding and
no products. Every draw is seeded, so a configuration always yields the same bytes.

Method background (SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World Usability, §3.1):
each 8-weight subvector along a row's input axis carries 8 sign bits, a log2(K)-bit index into a
per-matrix codebook of nonnegative unit directions, and a V-bit radius code on a uniform grid
(offset mu, step delta) shared by every 128 weights of a row, with 8 + log2(K) + V = 18.

Field conventions (permuted column order, as stored):
  signs  uint8 [d_out, d_in/8]   bit i set <=> weight at position i of the subvector is negative
  idx    uint8 [d_out, d_in/8]   codeword index z in [0, K)
  rcode  uint8 [d_out, d_in/8]   radius code q in [0, 2^V)
  mu     uint16 [d_out, d_in/128]  fp16 bit patterns of the group offsets
  delta  uint16 [d_out, d_in/128]  fp16 bit patterns of the group steps
  codebook uint16 [K, 8]         fp16 bit patterns, codeword k is row k
  pi     int32 [d_in]            pi[p] = original input channel found at permuted position p
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

SUBVEC = 8
GROUP = 128

# (K, V) pairs drawn by the synthetic workloads. The three-split set is the one the paper
# searches (its §3.3, Eq. (7)); the five-split sweep adds (16,6) and (32,5), which keep
# log2(K) + V = 10.
SPLITS_THREE: Tuple[Tuple[int, int], ...] = ((64, 4), (128, 3), (256, 2))
SPLITS_FIVE: Tuple[Tuple[int, int], ...] = ((16, 6), (32, 5), (64, 4), (128, 3), (256, 2))

BASE_SEED = 42


def rng_for(*key: int) -> np.random.Generator:
    """A PCG64 generator keyed by a tuple of non-negative integers."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


@dataclass
class Codes:
    """One quantised matrix as separate fields (see the module docstring for layouts)."""

    d_out: int
    d_in: int
    K: int
    V: int
    signs: np.ndarray
    idx: np.ndarray
    rcode: np.ndarray
    mu: np.ndarray
    delta: np.ndarray
    codebook: np.ndarray
    pi: np.ndarray
    name: str = ""

    @property
    def log2K(self) -> int:
        return int(self.K).bit_length() - 1

    def nbytes_fields(self) -> int:
        return sum(a.nbytes for a in (self.signs, self.idx, self.rcode, self.mu, self.delta,
                                      self.codebook, self.pi))


def _fp16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a.astype(np.float16)).view(np.uint16)


def draw_codebook(rng: np.random.Generator, K: int) -> np.ndarray:
    """K directions drawn as |N(0, I_8)| scaled to unit length, stored as fp16 bit patterns."""
    g = np.abs(rng.standard_normal((K, SUBVEC)))
    g /= np.linalg.norm(g, axis=1, keepdims=True)
    return _fp16_bits(g)


def draw_grid(rng: np.random.Generator, d_out: int, d_in: int,
              mu_range=(0.0, 0.5), delta_range=(0.01, 0.1)) -> Tuple[np.ndarray, np.ndarray]:
    ng = d_in // GROUP
    mu = rng.uniform(mu_range[0], mu_range[1], size=(d_out, ng))
    delta = rng.uniform(delta_range[0], delta_range[1], size=(d_out, ng))
    return _fp16_bits(mu), _fp16_bits(delta)


def draw_perm(rng: np.random.Generator, d_in: int) -> np.ndarray:
    return rng.permutation(d_in).astype(np.int32)


def draw_codes(rng: np.random.Generator, d_out: int, d_in: int, K: int, V: int,
               pi: Optional[np.ndarray] = None, name: str = "") -> Codes:
    """Codes drawn directly: uniform idx and rcode, 8 independent fair sign bits per subvector,
    uniform grid offsets/steps, an |N| unit codebook and (unless given) a uniform random pi."""
    assert d_in % GROUP == 0
    ns = d_in // SUBVEC
    signs = rng.integers(0, 256, size=(d_out, ns), dtype=np.uint8)
    assert 1 <= K <= 256
    idx = rng.integers(0, K, size=(d_out, ns), dtype=np.uint8)
    rcode = rng.integers(0, 1 << V, size=(d_out, ns), dtype=np.uint8)
    mu, delta = draw_grid(rng, d_out, d_in)
    codebook = draw_codebook(rng, K)
    if pi is None:
        pi = draw_perm(rng, d_in)
    return Codes(d_out, d_in, K, V, signs, idx, rcode, mu, delta, codebook,
                 np.ascontiguousarray(pi, dtype=np.int32), name)


def draw_x(rng: np.random.Generator, shape) -> np.ndarray:
    """fp16 activations drawn from N(0, 1), returned as np.float16."""
    return rng.standard_normal(shape).astype(np.float16)


# ----------------------------------------------------------------------------------------------
# The five synthetic workloads
# ----------------------------------------------------------------------------------------------

@dataclass
class SingleMatrixCalib:
    """A 256x1024 fp32 weight with N(0, 0.02^2) entries, and 512 calibration rows whose channel c
    is N(0,1) times a per-channel LogNormal(0,1) scale; 8 distinct channels get their scale
    multiplied by sqrt(10), i.e. ten times the energy. x is one fp16 N(0,1) input row."""

    W: np.ndarray
    X_cal: np.ndarray
    x: np.ndarray
    hot_channels: np.ndarray
    K: int = 64
    V: int = 4
    gamma: float = 0.75
    kmeans_iters: int = 20
    kmeans_samples: int = 65536
    seed: int = BASE_SEED + 1


def encoder_matrix(rng: np.random.Generator, d_out: int, d_in: int) -> Tuple[np.ndarray, np.ndarray]:
    """Encoder inputs: W ~ N(0, 0.02^2) as fp32 [d_out, d_in] and channel energies e = s^2 with
    s ~ LogNormal(0, 1) per channel (the energy of x_c = z s_c, z ~ N(0, 1)), float64 [d_in]."""
    Wm = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    e = rng.lognormal(0.0, 1.0, size=d_in) ** 2
    return Wm, e


def single_matrix_calib(d_out: int = 256, d_in: int = 1024, tokens: int = 512,
                        n_hot: int = 8, seed: int = BASE_SEED + 1) -> SingleMatrixCalib:
    rng = rng_for(seed)
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    scale = rng.lognormal(0.0, 1.0, size=d_in)
    hot = np.sort(rng.choice(d_in, size=n_hot, replace=False))
    scale[hot] *= np.sqrt(10.0)
    X_cal = (rng.standard_normal((tokens, d_in)) * scale[None, :]).astype(np.float32)
    x = draw_x(rng, (d_in,))
    return SingleMatrixCalib(W=W, X_cal=X_cal, x=x, hot_channels=hot, seed=seed)


# Qwen3-4B-shaped decoder layer: hidden 2560, 32 query heads and 8 KV heads of width 128,
# MLP width 9728.
QWEN3_4B_SHAPES: Dict[str, Tuple[int, int]] = {
    "q": (4096, 2560),
    "k": (1024, 2560),
    "v": (1024, 2560),
    "o": (2560, 4096),
    "gate": (9728, 2560),
    "up": (9728, 2560),
    "down": (2560, 9728),
}
# Projections that read the same input share its permutation and its activation vector.
QWEN3_4B_INPUTS: Dict[str, Tuple[str, ...]] = {
    "attn_in": ("q", "k", "v"),
    "attn_out": ("o",),
    "mlp_in": ("gate", "up"),
    "mlp_mid": ("down",),
}


@dataclass
class Layer:
    mats: Dict[str, Codes]
    xs: Dict[str, np.ndarray]           # input name -> fp16 [d_in]
    input_of: Dict[str, str]            # matrix name -> input name


def decoder_layer(K: int = 64, V: int = 4, seed: int = BASE_SEED + 2,
                  shapes: Dict[str, Tuple[int, int]] = QWEN3_4B_SHAPES) -> Layer:
    rng = rng_for(seed)
    mats: Dict[str, Codes] = {}
    xs: Dict[str, np.ndarray] = {}
    input_of: Dict[str, str] = {}
    for inp, names in QWEN3_4B_INPUTS.items():
        d_in = shapes[names[0]][1]
        pi = draw_perm(rng, d_in)
        xs[inp] = draw_x(rng, (d_in,))
        for nm in names:
            d_out, d_in2 = shapes[nm]
            assert d_in2 == d_in
            mats[nm] = draw_codes(rng, d_out, d_in, K, V, pi=pi, name=nm)
            input_of[nm] = inp
    return Layer(mats, xs, input_of)


def split_sweep_matrix(K: int, V: int, d_out: int = 9728, d_in: int = 2560,
                       seed: int = BASE_SEED + 3) -> Tuple[Codes, np.ndarray]:
    rng = rng_for(seed, K, V)
    c = draw_codes(rng, d_out, d_in, K, V, name=f"sweep_K{K}_V{V}")
    x = draw_x(rng, (d_in,))
    return c, x


def small_batch(d_out: int, d_in: int, M: int, K: int = 64, V: int = 4,
                seed: int = BASE_SEED + 4) -> Tuple[Codes, np.ndarray]:
    rng = rng_for(seed, d_out, d_in)
    c = draw_codes(rng, d_out, d_in, K, V, name=f"gemm_{d_out}x{d_in}")
    X = draw_x(rng_for(seed, d_out, d_in, M), (M, d_in))
    return c, X


@dataclass
class MoE:
    n_experts: int
    experts: List[Dict[str, Codes]]     # per expert: gate, up, down
    ids: np.ndarray                     # int32 [top_k], distinct
    x: np.ndarray                       # fp16 [hidden]  shared input of gate/up
    h: np.ndarray                       # fp16 [top_k, inter]  per selected expert input of down


MOE_HIDDEN = 2048
MOE_INTER = 768


def moe_expert(e: int, splits: Sequence[Tuple[int, int]] = SPLITS_THREE,
               hidden: int = MOE_HIDDEN, inter: int = MOE_INTER,
               seed: int = BASE_SEED + 5) -> Dict[str, Codes]:
    """Expert e's three matrices; its (K, V) is drawn uniformly from `splits`, and gate/up share a
    permutation of the hidden input."""
    rng = rng_for(seed, 1000 + e)
    K, V = splits[int(rng.integers(0, len(splits)))]
    pi_h = draw_perm(rng, hidden)
    gate = draw_codes(rng, inter, hidden, K, V, pi=pi_h, name=f"e{e}.gate")
    up = draw_codes(rng, inter, hidden, K, V, pi=pi_h, name=f"e{e}.up")
    down = draw_codes(rng, hidden, inter, K, V, name=f"e{e}.down")
    return {"gate": gate, "up": up, "down": down}


def moe_layer(n_experts: int = 128, top_k: int = 8, splits=SPLITS_THREE,
              hidden: int = MOE_HIDDEN, inter: int = MOE_INTER, seed: int = BASE_SEED + 5,
              experts_to_build: Optional[Sequence[int]] = None) -> MoE:
    """Routing picks top_k distinct experts uniformly. Only the experts listed in
    `experts_to_build` (default: the routed ones) are materialised; the rest are None."""
    rng = rng_for(seed)
    ids = np.sort(rng.choice(n_experts, size=top_k, replace=False)).astype(np.int32)
    x = draw_x(rng, (hidden,))
    h = draw_x(rng, (top_k, inter))
    build = set(int(i) for i in (ids if experts_to_build is None else experts_to_build))
    experts = [moe_expert(e, splits, hidden, inter, seed) if e in build else None
               for e in range(n_experts)]
    return MoE(n_experts, experts, ids, x, h)
