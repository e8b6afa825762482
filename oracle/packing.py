"""Our packed storage layout, written from its format description (TEST INFRASTRUCTURE ONLY; see
oracle/__init__).

The SAGE paper fixes what a subvector stores (§3.1, Eq. (3): 8 sign bits, a log2(K)-bit codeword
index and a V-bit radius code, 18 bits) and that every 128 weights of a row share an fp16 grid
(App. A.6), and says its own kernels keep "a 16-bit main word plus two auxiliary bits" per
subvector (§3.5); it gives no bit positions. The layout below is this repository's own (format
version 3), restated here from its description so the library's packer can be compared byte for
byte against an implementation that shares nothing with it:

  The matrix is cut into blocks of 64 rows (a row tile; the last tile is padded with zero rows)
  by 128 columns (a grid group). Block (rt, g) is 2560 bytes at (rt * n_groups + g) * 2560:
    bytes    0..1023  plane A, row 64 rt + l at bytes 16 l .. 16 l + 15: dwords P0, P1, P2, P3
    bytes 1024..2047  plane B, the same for P4, P5, P6, P7
    bytes 2048..2559  side plane, row 64 rt + l at bytes 8 l .. 8 l + 7: dword X, then dword G
  Dwords are little-endian. With L = log2 K, V = 10 - L, and for subvector j (0..15) of the group
  its sign byte s_j, index z_j and radius code q_j, dword P_i holds the pair a = 2i, b = 2i + 1:
    bits  0..2        s_b >> 5
    bits  3..2+L      z_a
    bits  3+L..6+L    s_a & 15
    bits  7+L..16     q_a
    bits  17..16+L    z_b
    bits  17+L..20+L  s_b & 15
    bits  21+L..30    q_b
    bit   31          (s_b >> 4) & 1
  X holds (s_{2i} >> 4) at bits 4i .. 4i + 3 for i = 0..7, and G = mu | delta << 16 (the fp16
  bit patterns of the group's grid offset and step).

Parity status: pinned by the CPU tests (every one of the 18 x 16 + 32 bits of a row's group lands
at its documented position when set alone; pack then unpack returns the fields for all five splits
and ragged row counts; the byte count is 2.5 bits per weight).
"""
from __future__ import annotations

from typing import Any, Dict

import numpy as np

TILE = 64
GROUP = 128
SUBVEC = 8
BLOCK_BYTES = 2560


def _get(c: Any, name: str):
    return c[name] if isinstance(c, dict) else getattr(c, name)


def packed_nbytes(d_out: int, d_in: int) -> int:
    tiles = -(-d_out // TILE)
    return tiles * (d_in // GROUP) * BLOCK_BYTES


def pack(c: Any) -> np.ndarray:
    """The packed bytes (uint8 [packed_nbytes]) of a matrix given as fields (signs, idx, rcode
    uint8 [d_out, d_in/8]; mu, delta fp16 bit patterns [d_out, d_in/128]; K, V)."""
    signs = np.asarray(_get(c, "signs"), dtype=np.uint32)
    idx = np.asarray(_get(c, "idx"), dtype=np.uint32)
    rcode = np.asarray(_get(c, "rcode"), dtype=np.uint32)
    mu = np.asarray(_get(c, "mu"), dtype=np.uint16).astype(np.uint32)
    delta = np.asarray(_get(c, "delta"), dtype=np.uint16).astype(np.uint32)
    K, V = int(_get(c, "K")), int(_get(c, "V"))
    L = K.bit_length() - 1
    assert (1 << L) == K and L + V == 10
    d_out, m = signs.shape
    d_in = m * SUBVEC
    ng = d_in // GROUP
    tiles = -(-d_out // TILE)
    rows = tiles * TILE

    def padded(a):
        out = np.zeros((rows,) + a.shape[1:], dtype=np.uint32)
        out[:d_out] = a
        return out

    # [tiles, 64 rows, groups, 16 subvectors]
    s = padded(signs).reshape(tiles, TILE, ng, 16)
    z = padded(idx & ((1 << L) - 1)).reshape(tiles, TILE, ng, 16)
    q = padded(rcode & ((1 << V) - 1)).reshape(tiles, TILE, ng, 16)
    sa, sb = s[..., 0::2], s[..., 1::2]
    za, zb = z[..., 0::2], z[..., 1::2]
    qa, qb = q[..., 0::2], q[..., 1::2]
    P = ((sb >> 5)
         | (za << 3)
         | ((sa & 15) << (3 + L))
         | (qa << (7 + L))
         | (zb << 17)
         | ((sb & 15) << (17 + L))
         | (qb << (21 + L))
         | (((sb >> 4) & 1) << 31))                      # [tiles, 64, ng, 8]
    X = np.zeros((tiles, TILE, ng), dtype=np.uint32)
    for i in range(8):
        X |= (sa[..., i] >> 4) << (4 * i)
    G = (padded(mu).reshape(tiles, TILE, ng) | (padded(delta).reshape(tiles, TILE, ng) << 16))

    P = P.transpose(0, 2, 1, 3)                           # [tiles, ng, 64 lanes, 8]
    plane_a = P[..., 0:4].reshape(tiles, ng, TILE * 4)
    plane_b = P[..., 4:8].reshape(tiles, ng, TILE * 4)
    side = np.stack([X.transpose(0, 2, 1), G.transpose(0, 2, 1)], axis=-1).reshape(tiles, ng, TILE * 2)
    blocks = np.concatenate([plane_a, plane_b, side], axis=-1).astype("<u4")
    return np.ascontiguousarray(blocks).reshape(-1).view(np.uint8)


def unpack(packed: np.ndarray, d_out: int, d_in: int, K: int, V: int) -> Dict[str, np.ndarray]:
    """The fields (signs, idx, rcode uint8; mu, delta uint16 bit patterns) of packed bytes."""
    L = K.bit_length() - 1
    ng = d_in // GROUP
    tiles = -(-d_out // TILE)
    w = np.ascontiguousarray(packed, dtype=np.uint8)[: packed_nbytes(d_out, d_in)]
    w = w.view("<u4").astype(np.uint32).reshape(tiles, ng, BLOCK_BYTES // 4)
    plane_a = w[..., 0:256].reshape(tiles, ng, TILE, 4)
    plane_b = w[..., 256:512].reshape(tiles, ng, TILE, 4)
    side = w[..., 512:640].reshape(tiles, ng, TILE, 2)
    P = np.concatenate([plane_a, plane_b], axis=-1)      # [tiles, ng, 64, 8]
    X, G = side[..., 0], side[..., 1]
    kmask, vmask = (1 << L) - 1, (1 << V) - 1
    za = (P >> 3) & kmask
    qa = (P >> (7 + L)) & vmask
    sa_lo = (P >> (3 + L)) & 15
    zb = (P >> 17) & kmask
    qb = (P >> (21 + L)) & vmask
    sb = ((P >> (17 + L)) & 15) | ((P >> 31) << 4) | ((P & 7) << 5)
    sa_hi = np.stack([(X >> (4 * i)) & 15 for i in range(8)], axis=-1)
    sa = sa_lo | (sa_hi << 4)

    def interleave(a, b):
        out = np.empty(a.shape[:-1] + (16,), dtype=np.uint32)
        out[..., 0::2] = a
        out[..., 1::2] = b
        return out.transpose(0, 2, 1, 3).reshape(tiles * TILE, ng * 16)[:d_out]

    def per_row(g):
        return g.transpose(0, 2, 1).reshape(tiles * TILE, ng)[:d_out]

    return dict(
        signs=interleave(sa, sb).astype(np.uint8),
        idx=interleave(za, zb).astype(np.uint8),
        rcode=interleave(qa, qb).astype(np.uint8),
        mu=per_row(G & 0xFFFF).astype(np.uint16),
        delta=per_row(G >> 16).astype(np.uint16),
    )
