"""Bit budget and storage cost (TEST INFRASTRUCTURE ONLY; see oracle/__init__).

Written from "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World Usability":
  bits_per_subvector  §3.1, Eq. (3): v sign bits + log2(K) index bits + V radius bits.
  bpw_matrix          Appendix A.6, Eq. (15): B/v + 2*b_g/G + K*v*b_c/N bits per weight for an
                      N-weight matrix (grid parameters of b_g bits per G weights, codebook entries
                      of b_c bits), excluding permutation and format metadata.
  codebook_bytes      K codewords of v components of b_c bits.

Parity status: pinned against the paper's own figures (18 bits and 2.25 bits per weight at
(64,4); 0.25 extra bits per weight from fp16 grids at G = 128, 2.50 in total; a 64-entry fp16
codebook occupying 1 KiB).
"""
from __future__ import annotations

import math


def bits_per_subvector(K: int, V: int, v: int = 8) -> int:
    lk = math.log2(K)
    if lk != int(lk):
        raise ValueError("K must be a power of two")
    return v + int(lk) + V


def bpw_matrix(d_out: int, d_in: int, K: int, V: int, v: int = 8, G: int = 128,
               b_g: int = 16, b_c: int = 16) -> float:
    N = d_out * d_in
    return bits_per_subvector(K, V, v) / v + 2.0 * b_g / G + K * v * b_c / N


def codebook_bytes(K: int, v: int = 8, b_c: int = 16) -> int:
    return K * v * b_c // 8


def payload_bytes(d_out: int, d_in: int, K: int, V: int, v: int = 8) -> float:
    """Bytes of sign/index/radius-code payload for a matrix."""
    return d_out * d_in / v * bits_per_subvector(K, V, v) / 8.0


def grid_bytes(d_out: int, d_in: int, G: int = 128, b_g: int = 16) -> float:
    return d_out * d_in / G * 2 * b_g / 8.0
