"""Pins of the oracle's packer (oracle/packing.py) against the layout's own definition.

The paper fixes the 18 bits a subvector stores (§3.1 Eq. (3)) and the fp16 grid of every 128
weights (App. A.6); the bit positions are this repository's format (version 3). These tests pin
the packer to that definition independently of how it is written: every single field bit, set
alone, must land at the one packed bit the format assigns to it (positions written out below as
literals), the 288 field bits and 32 grid bits of a row's group must fill the row's 10 dwords of
the block exactly once, and unpack must invert pack.
"""
import numpy as np
import pytest

import workloads as W
from oracle import packing

SPLITS = W.SPLITS_FIVE


def _empty(d_out, d_in, K, V):
    m, ng = d_in // 8, d_in // 128
    z8 = lambda: np.zeros((d_out, m), np.uint8)  # noqa: E731
    z16 = lambda: np.zeros((d_out, ng), np.uint16)  # noqa: E731
    return dict(signs=z8(), idx=z8(), rcode=z8(), mu=z16(), delta=z16(), K=K, V=V)


def _set_bits(buf):
    """(byte offset, bit) of every set bit."""
    out = []
    for off in np.flatnonzero(buf):
        for b in range(8):
            if (int(buf[off]) >> b) & 1:
                out.append((int(off), b))
    return out


def _dword_bits(byte0, bits):
    """Packed (byte, bit) positions of bits `bits` of the little-endian dword at byte0."""
    return sorted((byte0 + b // 8, b % 8) for b in bits)


# where lane l's dwords live inside its block
def _p_byte(lane, i):
    return (0 if i < 4 else 1024) + 16 * lane + 4 * (i % 4)


def _x_byte(lane):
    return 2048 + 8 * lane


def _g_byte(lane):
    return 2048 + 8 * lane + 4


@pytest.mark.parametrize("K,V", SPLITS)
def test_each_field_bit_lands_where_the_format_puts_it(K, V):
    L = K.bit_length() - 1
    d_out, d_in = 70, 256           # rows 64..69 are in the second tile; two groups per row
    ng = 2
    for row, g, j in [(0, 0, 0), (0, 0, 1), (5, 1, 14), (66, 1, 15), (69, 0, 7), (63, 1, 8)]:
        rt, lane = divmod(row, 64)
        blk = (rt * ng + g) * packing.BLOCK_BYTES
        i = j // 2
        for name, width in (("signs", 8), ("idx", L), ("rcode", V)):
            for b in range(width):
                c = _empty(d_out, d_in, K, V)
                c[name][row, 16 * g + j] = 1 << b
                got = _set_bits(packing.pack(c))
                # the format's position of bit b of this field (see oracle/packing.py)
                if j % 2 == 0:  # subvector a of pair i
                    if name == "idx":
                        want = _dword_bits(blk + _p_byte(lane, i), [3 + b])
                    elif name == "rcode":
                        want = _dword_bits(blk + _p_byte(lane, i), [7 + L + b])
                    elif b < 4:
                        want = _dword_bits(blk + _p_byte(lane, i), [3 + L + b])
                    else:
                        want = _dword_bits(blk + _x_byte(lane), [4 * i + b - 4])
                else:           # subvector b of pair i
                    if name == "idx":
                        want = _dword_bits(blk + _p_byte(lane, i), [17 + b])
                    elif name == "rcode":
                        want = _dword_bits(blk + _p_byte(lane, i), [21 + L + b])
                    elif b < 4:
                        want = _dword_bits(blk + _p_byte(lane, i), [17 + L + b])
                    elif b == 4:
                        want = _dword_bits(blk + _p_byte(lane, i), [31])
                    else:
                        want = _dword_bits(blk + _p_byte(lane, i), [b - 5])
                assert got == want, (name, b, row, g, j)
        for name, byte in (("mu", _g_byte(lane)), ("delta", _g_byte(lane) + 2)):
            for b in range(16):
                c = _empty(d_out, d_in, K, V)
                c[name][row, g] = 1 << b
                assert _set_bits(packing.pack(c)) == [(blk + byte + b // 8, b % 8)], (name, b)


@pytest.mark.parametrize("K,V", SPLITS)
def test_field_bits_fill_the_block_exactly_once(K, V):
    """The 16 x 18 payload bits and 32 grid bits of one row's group map one-to-one onto the
    row's 10 dwords (P0..P7, X, G): 2.5 bits per weight with no bit unused or shared."""
    L = K.bit_length() - 1
    seen = set()
    row, lane, g = 3, 3, 0
    for j in range(16):
        for name, width in (("signs", 8), ("idx", L), ("rcode", V)):
            for b in range(width):
                c = _empty(64, 128, K, V)
                c[name][row, j] = 1 << b
                bits = _set_bits(packing.pack(c))
                assert len(bits) == 1
                seen.add(bits[0])
    for name in ("mu", "delta"):
        for b in range(16):
            c = _empty(64, 128, K, V)
            c[name][row, g] = 1 << b
            seen.add(_set_bits(packing.pack(c))[0])
    assert len(seen) == 16 * 18 + 32
    lane_bytes = set()
    for i in range(8):
        lane_bytes |= {_p_byte(lane, i) + k for k in range(4)}
    lane_bytes |= {_x_byte(lane) + k for k in range(8)}
    assert {byte for byte, _ in seen} == lane_bytes


@pytest.mark.parametrize("K,V", SPLITS)
@pytest.mark.parametrize("d_out,d_in", [(1, 128), (7, 256), (64, 128), (65, 384), (130, 1152)])
def test_pack_then_unpack_returns_the_fields(d_out, d_in, K, V):
    c = W.draw_codes(W.rng_for(200, d_out, d_in, K), d_out, d_in, K, V)
    buf = packing.pack(c)
    assert buf.size == packing.packed_nbytes(d_out, d_in)
    assert buf.size * 8 == -(-d_out // 64) * 64 * d_in * 2.5
    f = packing.unpack(buf, d_out, d_in, K, V)
    for name in ("signs", "idx", "rcode", "mu", "delta"):
        assert np.array_equal(f[name], getattr(c, name)), name


def test_padded_rows_are_zero():
    c = W.draw_codes(W.rng_for(201), 65, 256, 64, 4)
    buf = packing.pack(c).reshape(2, 2, packing.BLOCK_BYTES)   # [tile, group, bytes]
    second = buf[1]
    for lane in range(1, 64):
        for i in range(8):
            assert not np.any(second[:, _p_byte(lane, i):_p_byte(lane, i) + 4])
        assert not np.any(second[:, _x_byte(lane):_x_byte(lane) + 8])
