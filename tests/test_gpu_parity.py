"""GPU parity: libsage (through its C ABI) against the float64 oracle, element by element.

Bars (stated in the method's terms, SAGE paper §3.1 Eq. (1)-(2)):
  pack / unpack      bit-exact on every field; the packed bytes equal the oracle's own packer
                     (oracle/packing.py, written from the format description).
  dequant            within 1 fp16 ulp of the correctly rounded decode (+0 == -0); the fp64 device
                     decode is expected to be exact.
  products           the contract bound, max |y - y_ref| <= 2e-3 * max_r sum_c |W_hat||x|
                     per output vector, AND a tight per-element bound derived from the arithmetic
                     (see sage_testlib: one fp16 rounding of the output, the fp32 accumulation and,
                     for the batch-one kernel, its radius arithmetic) that one wrong subvector
                     exceeds; the planted-corruption tests below show that it does. Following the
                     paper's App. A.3 / Table 4 practice the relative L2 error against the
                     independent decode is logged as well.
Inputs are the seeded synthetic workloads (see workloads/); sizes span several row tiles, column
groups and ragged tails, up to the full benchmark shapes.
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from oracle import decoder, encoder, packing
from sage_testlib import (batch_one_bounds, log, log2k, rounded_weight_bounds, ulp_distance,
                          upload, upload_pack)

import bit_vector_quantized_amd as sage

pytestmark = pytest.mark.gpu

SPLITS = W.SPLITS_FIVE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "these tests need the GPU"
    sage.lib()
    log(f"[lib] sources {sage.source_digest()}")
    yield
    torch.cuda.synchronize()


def _np(t):
    return t.detach().cpu().numpy()


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gemv_errors(c, x, y_dev, stored_order=False):
    """(worst err / tight bound, rows over the tight bound, worst err / contract bound)."""
    import torch
    torch.cuda.synchronize()
    ref, tight, contract = batch_one_bounds(c, x, stored_order)
    got = _np(y_dev).astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    return err, tight, contract, ref, got


def check_gemv(name, c, x, y_dev, stored_order=False):
    err, tight, contract, ref, got = gemv_errors(c, x, y_dev, stored_order)
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    log(f"[gemv] {name}: max_err={err.max():.3e} err/tight={float(np.max(err / tight)):.3f} "
        f"contract={contract:.3e} rel_l2={rel_l2:.2e}")
    assert float(err.max()) <= contract, f"{name}: contract bound"
    bad = np.flatnonzero(err > tight)
    assert bad.size == 0, f"{name}: rows {bad[:8].tolist()} over the tight bound"


def check_gemm(name, c, X, Y_dev, rounded=True):
    """Rows of Y against the oracle. rounded: the kernel decodes weights to fp16 (MFMA paths);
    M = 1 runs the batch-one kernel and is checked as such."""
    import torch
    torch.cuda.synchronize()
    got = _np(Y_dev).astype(np.float64)
    assert np.all(np.isfinite(got))
    if not rounded:
        for m in range(X.shape[0]):
            check_gemv(f"{name} row {m}", c, X[m], torch.from_numpy(got[m].astype(np.float16)))
        return
    ref, tight, contract = rounded_weight_bounds(c, X)
    err = np.abs(got - ref)
    log(f"[gemm] {name}: err/tight={float(np.max(err / tight)):.3f} "
        f"err/contract={float(np.max(err / contract)):.4f}")
    assert np.all(err <= contract), f"{name}: contract bound"
    bad = np.argwhere(err > tight)
    assert bad.shape[0] == 0, f"{name}: (row, output) {bad[:8].tolist()} over the tight bound"


# ------------------------------------------------------------------------------ pack / unpack

SMALL_SHAPES = [(1, 128), (7, 256), (64, 128), (65, 384), (130, 1152), (256, 1024)]


@pytest.mark.parametrize("K,V", SPLITS)
@pytest.mark.parametrize("d_out,d_in", SMALL_SHAPES)
def test_pack_unpack_roundtrip_and_oracle_bytes(d_out, d_in, K, V):
    import torch
    c = W.draw_codes(W.rng_for(100, d_out, d_in, K), d_out, d_in, K, V)
    log(f"[pack] {d_out}x{d_in} K={K} V={V}")
    p = upload_pack(c)
    s, i, q, mu, de = sage.unpack(p)
    torch.cuda.synchronize()
    assert np.array_equal(_np(s), c.signs)
    assert np.array_equal(_np(i), c.idx)
    assert np.array_equal(_np(q), c.rcode)
    assert np.array_equal(_np(mu).view(np.uint16), c.mu)
    assert np.array_equal(_np(de).view(np.uint16), c.delta)
    raw = _np(p.packed)
    assert raw.size == sage.packed_bytes(d_out, d_in, log2k(c), V)
    assert np.array_equal(raw, packing.pack(c)), "packed bytes differ from the oracle's packer"


def test_pack_ignores_bits_above_field_width():
    import torch
    c = W.draw_codes(W.rng_for(101), 70, 256, 32, 5)
    d = upload(c)
    noisy_i = d["idx"] | torch.tensor(0xE0, dtype=torch.uint8, device="cuda")
    noisy_q = d["rcode"] | torch.tensor(0xE0, dtype=torch.uint8, device="cuda")
    p = sage.pack(d["signs"], noisy_i, noisy_q, d["mu"], d["delta"], d["codebook"], d["pi"], 5, 5)
    s, i, q, mu, de = sage.unpack(p)
    torch.cuda.synchronize()
    assert np.array_equal(_np(i), c.idx) and np.array_equal(_np(q), c.rcode)
    assert np.array_equal(_np(p.packed), packing.pack(c))


def test_pack_unpack_full_size():
    import torch
    c = W.draw_codes(W.rng_for(102), 9728, 2560, 64, 4)
    log("[pack] 9728x2560 K=64")
    p = upload_pack(c)
    s, i, q, mu, de = sage.unpack(p)
    torch.cuda.synchronize()
    for a, b in ((s, c.signs), (i, c.idx), (q, c.rcode)):
        assert np.array_equal(_np(a), b)
    assert np.array_equal(_np(mu).view(np.uint16), c.mu)
    assert np.array_equal(_np(de).view(np.uint16), c.delta)
    assert np.array_equal(_np(p.packed), packing.pack(c))


# ------------------------------------------------------------------------------ dequant

def check_dequant(name, c, p):
    import torch
    w = sage.dequant(p)
    torch.cuda.synchronize()
    got = _np(w).view(np.uint16)
    ref = decoder.dequant_fp16(c)
    d = ulp_distance(got, ref)
    exact = float(np.mean(d == 0))
    log(f"[dequant] {name}: max_ulp={int(d.max())} exact={exact:.6f}")
    assert int(d.max()) <= 1, name
    return exact


@pytest.mark.parametrize("K,V", SPLITS)
@pytest.mark.parametrize("d_out,d_in", SMALL_SHAPES)
def test_dequant_small(d_out, d_in, K, V):
    c = W.draw_codes(W.rng_for(110, d_out, d_in, K), d_out, d_in, K, V)
    exact = check_dequant(f"{d_out}x{d_in} K={K}", c, upload_pack(c))
    assert exact == 1.0


@pytest.mark.parametrize("K,V", SPLITS)
def test_dequant_full_size_sweep(K, V):
    c, _ = W.split_sweep_matrix(K, V)
    check_dequant(f"9728x2560 K={K}", c, upload_pack(c))


def test_dequant_identity_permutation():
    c = W.draw_codes(W.rng_for(111), 96, 512, 128, 3)
    c.pi = np.arange(512, dtype=np.int32)
    check_dequant("identity pi", c, upload_pack(c, identity_pi=True))


# ------------------------------------------------------------------------------ batch-one gemv

GEMV_SMALL = [(1, 128), (7, 256), (64, 128), (65, 384), (130, 1152), (200, 2048), (700, 768)]


@pytest.mark.parametrize("K,V", SPLITS)
@pytest.mark.parametrize("d_out,d_in", GEMV_SMALL)
def test_gemv_small(d_out, d_in, K, V):
    rng = W.rng_for(120, d_out, d_in, K)
    c = W.draw_codes(rng, d_out, d_in, K, V)
    x = W.draw_x(rng, (d_in,))
    log(f"[gemv] start {d_out}x{d_in} K={K}")
    y = sage.gemv(upload_pack(c), _dev(x))
    check_gemv(f"{d_out}x{d_in} K={K}", c, x, y)


@pytest.mark.parametrize("K,V", SPLITS)
@pytest.mark.parametrize("d_out,d_in", [(130, 1152), (700, 768)])
def test_gemv_stored_order_input(d_out, d_in, K, V):
    """pi = NULL (the input's producer wrote it in stored order, §3.5 compiled decoding)."""
    rng = W.rng_for(121, d_out, d_in, K)
    c = W.draw_codes(rng, d_out, d_in, K, V)
    xp = W.draw_x(rng, (d_in,))
    p = dataclasses.replace(upload_pack(c), pi=None)
    y = sage.gemv(p, _dev(xp))
    check_gemv(f"stored order {d_out}x{d_in} K={K}", c, xp, y, stored_order=True)


def test_gemv_single_matrix_calibrated():
    """256x1024 matrix encoded by the oracle (K=64, V=4, gamma=0.75, ESG), one fp16 input."""
    cfg = W.single_matrix_calib()
    e = encoder.channel_energy(cfg.X_cal)
    enc = encoder.encode_matrix(cfg.W, e, cfg.K, cfg.V, gamma=cfg.gamma, iters=cfg.kmeans_iters,
                                samples=cfg.kmeans_samples, seed=cfg.seed)
    p = upload_pack(enc)
    check_dequant("calibrated 256x1024", enc, p)
    y = sage.gemv(p, _dev(cfg.x))
    check_gemv("calibrated 256x1024", enc, cfg.x, y)


@pytest.fixture(scope="module")
def layer():
    return W.decoder_layer()


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "gate", "up", "down"])
def test_gemv_decoder_layer(layer, name):
    c = layer.mats[name]
    x = layer.xs[layer.input_of[name]]
    p = upload_pack(c)
    y = sage.gemv(p, _dev(x))
    check_gemv(f"layer.{name} {c.d_out}x{c.d_in}", c, x, y)
    # the same matrix with its input already permuted (compiled decoding)
    xp = np.ascontiguousarray(x[c.pi])
    y2 = sage.gemv(dataclasses.replace(p, pi=None), _dev(xp))
    check_gemv(f"layer.{name} stored order", c, xp, y2, stored_order=True)


def test_gemv_multi_siblings_and_repeat(layer):
    """q/k/v in one launch and gate/up in one launch; a second call reproduces the bits."""
    import torch
    for group in (("q", "k", "v"), ("gate", "up")):
        cs = [layer.mats[n] for n in group]
        x = layer.xs[layer.input_of[group[0]]]
        ps = [upload_pack(c) for c in cs]
        xd = _dev(x)
        ys1 = sage.gemv_multi(ps, [xd] * len(ps))
        torch.cuda.synchronize()
        first = [_np(y).copy() for y in ys1]
        ys2 = sage.gemv_multi(ps, [xd] * len(ps))
        for n, c, y, f in zip(group, cs, ys2, first):
            check_gemv(f"multi.{n}", c, x, y)
            assert np.array_equal(_np(y), f), "repeat call must reproduce the same bits"


@pytest.mark.parametrize("K,V", SPLITS)
def test_gemv_split_sweep_full_size(K, V):
    c, x = W.split_sweep_matrix(K, V)
    y = sage.gemv(upload_pack(c), _dev(x))
    check_gemv(f"sweep 9728x2560 K={K}", c, x, y)


@pytest.mark.parametrize("rows,d_in", [((9728, 9731), 2560), ((12000, 11001), 2048),
                                       ((40003, 1), 1024)])
def test_gemv_multi_many_chunks(rows, d_in):
    """Products with several 16-row chunks per workgroup (up to 40003 rows: ten chunks), ragged
    row counts, two codebook sizes, lane-group ranges that cross a chunk boundary; repeat calls
    reproduce the same bits."""
    import torch
    rng = W.rng_for(135, rows[0], d_in)
    cs = [W.draw_codes(rng, rows[0], d_in, 64, 4), W.draw_codes(rng, rows[1], d_in, 128, 3)]
    x = W.draw_x(rng, (d_in,))
    ps = [upload_pack(c) for c in cs]
    xd = _dev(x)
    ys = sage.gemv_multi(ps, [xd, xd])
    torch.cuda.synchronize()
    first = [_np(y).copy() for y in ys]
    ys = sage.gemv_multi(ps, [xd, xd])
    for c, y, f in zip(cs, ys, first):
        check_gemv(f"chunks {c.d_out}x{d_in}", c, x, y)
        assert np.array_equal(_np(y), f), "repeat call must reproduce the same bits"


def test_gemv_range_padding_at_chunk_end():
    """Single-chunk products for every even half-group count mod 64 (d_in = 64 * 2..128): the 64
    lane-group ranges then differ in length by one, a range shorter than the longest in its
    wavefront steps one unit past its end, and where such a range ends exactly at the chunk's end
    that padding step must leave its sum where it is."""
    rng = W.rng_for(140)
    for d_out in (16, 9):
        for nhalf in range(2, 130, 2):
            d_in = 64 * nhalf
            c = W.draw_codes(rng, d_out, d_in, 64, 4)
            x = W.draw_x(rng, (d_in,))
            y = sage.gemv(upload_pack(c), _dev(x))
            check_gemv(f"one chunk {d_out}x{d_in}", c, x, y)


@pytest.mark.parametrize("d_in", [2560, 3968, 4224, 8320])
def test_gemv_range_padding_two_and_three_chunks(d_in):
    """8784 rows = 549 chunks: two or three chunks per workgroup on a 256-CU device, ranges that
    cross a chunk boundary next to ranges that end exactly at one. 4224 and 8320 columns (33 and
    65 groups) put more than 32 ranges on a chunk, so the final reduction takes eight sums per lane
    and, for the second and third chunks, reads past range 63 that it must leave out."""
    rng = W.rng_for(141, d_in)
    c = W.draw_codes(rng, 8784, d_in, 64, 4)
    x = W.draw_x(rng, (d_in,))
    y = sage.gemv(upload_pack(c), _dev(x))
    check_gemv(f"chunks 8784x{d_in}", c, x, y)


def test_gemv_most_chunks_per_workgroup():
    """One product with more than 64 chunks per compute unit: the planner adds workgroups (each
    takes at most 64 chunks, 1024 rows)."""
    rng = W.rng_for(139)
    c = W.draw_codes(rng, 300000, 256, 32, 5)
    x = W.draw_x(rng, (256,))
    y = sage.gemv(upload_pack(c), _dev(x))
    check_gemv("300000x256", c, x, y)


def test_gemv_zero_input_and_zero_grid():
    import torch
    c = W.draw_codes(W.rng_for(132), 300, 640, 16, 6)
    p = upload_pack(c)
    y = sage.gemv(p, torch.zeros(640, dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    assert np.all(_np(y) == 0)
    c.mu[:] = 0
    c.delta[:] = 0
    p = upload_pack(c)
    x = W.draw_x(W.rng_for(133), (640,))
    y = sage.gemv(p, _dev(x))
    torch.cuda.synchronize()
    assert np.all(_np(y) == 0)


@pytest.mark.parametrize("d_in,K,V,identity", [(17408, 64, 4, False), (11264, 256, 2, False),
                                               (32768, 64, 4, True)])
def test_gemv_widest_inputs(d_in, K, V, identity):
    """The widest inputs the workgroup stages in LDS: gathered through pi (the gather needs the
    input twice and pi once, so the width depends on the table size) and in stored order."""
    rng = W.rng_for(134, d_in)
    c = W.draw_codes(rng, 200, d_in, K, V)
    x = W.draw_x(rng, (d_in,))
    p = upload_pack(c)
    if identity:
        p = dataclasses.replace(p, pi=None)
    y = sage.gemv(p, _dev(x))
    check_gemv(f"wide 200x{d_in} K={K}", c, x, y, stored_order=identity)


def test_gemv_too_wide_is_refused():
    rng = W.rng_for(134, 1)
    c = W.draw_codes(rng, 16, 33792, 64, 4)
    p = upload_pack(c)
    with pytest.raises(sage.SageError) as ei:
        sage.gemv(dataclasses.replace(p, pi=None), _dev(W.draw_x(rng, (33792,))))
    assert ei.value.status == 2
    c2 = W.draw_codes(rng, 16, 12288, 256, 2)
    with pytest.raises(sage.SageError):
        sage.gemv(upload_pack(c2), _dev(W.draw_x(rng, (12288,))))


def test_gemv_input_not_16_byte_aligned():
    """x only 4-byte aligned (an offset view)."""
    import torch
    rng = W.rng_for(135)
    c = W.draw_codes(rng, 300, 1024, 32, 5)
    x = W.draw_x(rng, (1024,))
    buf = torch.zeros(1024 + 2, dtype=torch.float16, device="cuda")
    buf[2:] = _dev(x)
    xd = buf[2:]
    assert xd.data_ptr() % 16 != 0 and xd.data_ptr() % 4 == 0
    y = sage.gemv(upload_pack(c), xd)
    check_gemv("x at a 4-byte offset", c, x, y)


def test_gemv_multi_sixteen_mixed_products():
    """The most products one launch takes, of very different sizes, mixed splits, with and
    without a permutation."""
    rng = W.rng_for(137)
    shapes = [(64 * (1 + (i * 7) % 23) - (i % 3), 128 * (1 + i % 5)) for i in range(16)]
    splits = [(16, 6), (32, 5), (64, 4), (128, 3), (256, 2)]
    cs = [W.draw_codes(rng, d_out, d_in, *splits[i % 5]) for i, (d_out, d_in) in enumerate(shapes)]
    xs = [W.draw_x(rng, (d_in,)) for _, d_in in shapes]
    ps = [upload_pack(c) for c in cs]
    ps = [dataclasses.replace(p, pi=None) if i % 4 == 3 else p for i, p in enumerate(ps)]
    ys = sage.gemv_multi(ps, [_dev(x) for x in xs])
    for i, (c, x, y) in enumerate(zip(cs, xs, ys)):
        check_gemv(f"mixed[{i}] {c.d_out}x{c.d_in} K={c.K}", c, x, y, stored_order=(i % 4 == 3))


# ------------------------------------------------------------------------------ planted errors

def _plant(c, x, kind, seed, contract):
    """Copy of c with one subvector changed (its codeword index, or one sign bit), chosen among
    random candidates as the change with the largest effect on y that the contract bound still
    cannot see. Returns (corrupted codes, row, |delta y|)."""
    rng = W.rng_for(seed)
    xp = np.asarray(x, np.float64)[np.asarray(c.pi, np.int64)]
    C = np.asarray(c.codebook, np.uint16).view(np.float16).astype(np.float64).reshape(-1, 8)
    r_all = decoder.radii(c)
    best = None
    for _ in range(400):
        r = int(rng.integers(c.d_out))
        j = int(rng.integers(c.idx.shape[1]))
        s, z = int(c.signs[r, j]), int(c.idx[r, j])
        sgn = np.array([-1.0 if (s >> i) & 1 else 1.0 for i in range(8)])
        old = r_all[r, j] * sgn * C[z]
        if kind == "idx":
            z2 = (z + 1 + int(rng.integers(c.K - 1))) % c.K
            new, change = r_all[r, j] * sgn * C[z2], ("idx", z2)
        else:
            b = int(rng.integers(8))
            sg2 = sgn.copy()
            sg2[b] = -sg2[b]
            new, change = r_all[r, j] * sg2 * C[z], ("sign", s ^ (1 << b))
        dy = abs(float((new - old) @ xp[8 * j:8 * j + 8]))
        if dy < 0.5 * contract and (best is None or dy > best[0]):
            best = (dy, r, j, change)
    dy, r, j, (what, val) = best
    bad = dataclasses.replace(c, signs=c.signs.copy(), idx=c.idx.copy())
    (bad.idx if what == "idx" else bad.signs)[r, j] = val
    return bad, r, dy


@pytest.mark.parametrize("kind", ["idx", "sign"])
@pytest.mark.parametrize("name", ["gate", "down"])
def test_planted_error_batch_one(layer, name, kind):
    """One subvector of the 9728x2560 / 2560x9728 layer matrix is changed before sage_pack; the
    result is compared with the oracle's product of the UNCHANGED fields. The contract bound
    passes; the tight bound flags exactly the changed row (compare a fast path against an
    independent decode of the same codes: App. A.3 / Table 4)."""
    c = layer.mats[name]
    x = layer.xs[layer.input_of[name]]
    _, _, contract = batch_one_bounds(c, x)
    bad, row, dy = _plant(c, x, kind, 160 + len(name) + len(kind), contract)
    y = sage.gemv(upload_pack(bad), _dev(x))
    err, tight, contract, _, _ = gemv_errors(c, x, y)
    over = np.flatnonzero(err > tight)
    log(f"[planted] {name} {kind}: row {row} |dy|={dy:.4f} tight={tight[row]:.4f} "
        f"contract={contract:.4f} flagged={over.tolist()}")
    assert float(err.max()) <= contract, "the contract bound cannot see this change"
    assert over.tolist() == [row], "the tight bound must flag exactly the changed row"


@pytest.mark.parametrize("M,name,kind", [(16, "gate", "idx"), (64, "down", "sign"),
                                         (512, "gate", "sign")])
def test_planted_error_mfma_paths(layer, M, name, kind):
    """The same planted change through the small-batch (M = 16, 64) and prefill (M = 512)
    kernels: the tight bound flags the changed output in every activation row."""
    import torch
    c = layer.mats[name]
    X = W.draw_x(W.rng_for(165, M), (M, c.d_in))
    x0 = X[0]
    _, _, contract0 = batch_one_bounds(c, x0)
    bad, row, dy = _plant(c, x0, kind, 166 + M, contract0)
    Y = sage.gemm_small(upload_pack(bad), _dev(X))
    torch.cuda.synchronize()
    ref, tight, contract = rounded_weight_bounds(c, X)
    err = np.abs(_np(Y).astype(np.float64) - ref)
    flagged = sorted(set(np.argwhere(err > tight)[:, 1].tolist()))
    log(f"[planted] gemm M={M} {name} {kind}: output {row} |dy(row 0)|={dy:.4f} flagged={flagged}")
    assert np.all(err[0] <= contract[0]), "activation row 0: the contract bound cannot see it"
    assert flagged == [row]
    assert err[0, row] > tight[0, row]


# ------------------------------------------------------------------------------ small-batch gemm

@pytest.mark.parametrize("M", [1, 4, 5, 16, 17, 33, 64, 70])
@pytest.mark.parametrize("K,V", [(16, 6), (64, 4), (256, 2)])
def test_gemm_small_shapes(M, K, V):
    rng = W.rng_for(140, M, K)
    c = W.draw_codes(rng, 130, 1152, K, V)
    X = W.draw_x(rng, (M, 1152))
    Y = sage.gemm_small(upload_pack(c), _dev(X))
    check_gemm(f"130x1152 K={K} M={M}", c, X, Y, rounded=M > 1)


@pytest.mark.parametrize("d_in", [2560, 2688])
@pytest.mark.parametrize("M", [3, 12, 16])
def test_gemm_small_workgroup_shapes(M, d_in):
    """Up to sixteen rows with at most twenty column groups run as one split of 1 x 4 workgroups
    (d_in 2560); twenty-one groups fall back to 2 x 2 with split-K (d_in 2688). A ragged last
    row tile (70 rows) in both."""
    rng = W.rng_for(143, M, d_in)
    c = W.draw_codes(rng, 70, d_in, 64, 4)
    X = W.draw_x(rng, (M, d_in))
    Y = sage.gemm_small(upload_pack(c), _dev(X))
    check_gemm(f"70x{d_in} M={M}", c, X, Y)


@pytest.mark.parametrize("d_out,d_in,M", [
    (70, 128, 17),      # one column group: parts 1-3 idle, ragged last row tile
    (130, 256, 32),     # two groups, two row tiles
    (64, 384, 48),      # three groups over four parts
    (4160, 640, 100),   # five groups (two iterations, a part with one), two activation chunks
    (70, 2688, 33),     # 21 groups: split over the columns in the streamed plan
    (300, 2560, 64),    # 20 groups, five iterations per part, split-K on few row tiles
])
def test_gemm_streamed_activation_shapes(d_out, d_in, M):
    """From 17 rows the activations stream through LDS one column group per part and iteration:
    ragged group counts (some parts without groups), one or several iterations, one or two
    activation chunks, with and without split-K."""
    rng = W.rng_for(147, d_out, d_in, M)
    c = W.draw_codes(rng, d_out, d_in, 64, 4)
    X = W.draw_x(rng, (M, d_in))
    Y = sage.gemm_small(upload_pack(c), _dev(X))
    check_gemm(f"{d_out}x{d_in} M={M} streamed", c, X, Y)


@pytest.mark.parametrize("M", [1, 4, 16, 64])
@pytest.mark.parametrize("shape", [(9728, 2560), (2560, 9728)])
def test_gemm_small_full_size(shape, M):
    c, X = W.small_batch(shape[0], shape[1], M)
    Y = sage.gemm_small(upload_pack(c), _dev(X))
    check_gemm(f"{shape[0]}x{shape[1]} M={M}", c, X, Y, rounded=M > 1)


@pytest.mark.parametrize("M", [128, 200, 512])
@pytest.mark.parametrize("K,V", [(32, 5), (128, 3)])
def test_gemm_prefill_shapes(M, K, V):
    """Prefill-sized batches: several 64-row chunks of activations, ragged last chunk."""
    rng = W.rng_for(143, M, K)
    c = W.draw_codes(rng, 130, 1152, K, V)
    X = W.draw_x(rng, (M, 1152))
    Y = sage.gemm_small(upload_pack(c), _dev(X))
    check_gemm(f"130x1152 K={K} M={M}", c, X, Y)


def _check_sampled_rows(name, c, X, Y, rows):
    import torch
    torch.cuda.synchronize()
    assert np.all(np.isfinite(_np(Y)))
    check_gemm(name, c, X[rows], torch.from_numpy(_np(Y)[rows]))


@pytest.mark.parametrize("shape", [(9728, 2560), (2560, 9728)])
def test_gemm_prefill_full_size_sampled(shape):
    """M = 1024 at full size, checked on 48 sampled activation rows (first, last and spread)."""
    c, X = W.small_batch(shape[0], shape[1], 1024)
    Y = sage.gemm_small(upload_pack(c), _dev(X))
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 1023],
                                     W.rng_for(144).choice(1024, 43, replace=False)]))
    _check_sampled_rows(f"{shape} M=1024 sampled", c, X, Y, rows)


@pytest.mark.parametrize("d_out,d_in,M,K,V", [(4096, 1152, 1000, 64, 4), (4000, 640, 1030, 256, 2),
                                               (8192, 384, 520, 16, 6), (8192, 384, 1100, 16, 6),
                                               (8000, 640, 1030, 64, 4)])
def test_gemm_prefill_kernel(d_out, d_in, M, K, V):
    """Grids wide enough for the prefill kernel, with 128-row and (last two) 256-row activation
    blocks: ragged weight tiles, ragged last block, three to nine column groups; checked on 64
    sampled activation rows."""
    rng = W.rng_for(145, d_out, d_in, M)
    c = W.draw_codes(rng, d_out, d_in, K, V)
    X = W.draw_x(rng, (M, d_in))
    Y = sage.gemm_small(upload_pack(c), _dev(X))
    rows = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.choice(M, 60, replace=False)]))
    _check_sampled_rows(f"prefill {d_out}x{d_in} M={M} K={K}", c, X, Y, rows)


@pytest.mark.parametrize("d_out,d_in,M,K,V,ldy", [(130, 1408, 130, 32, 5, 130), (130, 1280, 300, 256, 2, 136),
                                                   (640, 9728, 128, 16, 6, 640), (200, 2432, 257, 64, 4, 203),
                                                   (640, 9728, 96, 64, 4, 640), (200, 2432, 100, 256, 2, 203)])
def test_gemm_prefill_split(d_out, d_in, M, K, V, ldy):
    """Grids too narrow for the compute units: the prefill kernel splits the column groups
    (ragged last split, 64-, 128- and 256-row activation blocks, output rows wider than d_out) and a
    second kernel adds the splits; a repeated call gives the same bits."""
    import torch
    rng = W.rng_for(146, d_out, d_in, M)
    c = W.draw_codes(rng, d_out, d_in, K, V)
    X = W.draw_x(rng, (M, d_in))
    p = upload_pack(c)
    Xd = _dev(X)
    Ybig = torch.full((M, ldy), 7.0, dtype=torch.float16, device="cuda")
    sage.gemm_small(p, Xd, Y=Ybig[:, :d_out])
    Y2 = sage.gemm_small(p, Xd)
    torch.cuda.synchronize()
    Yb = _np(Ybig)
    assert np.all(Yb[:, d_out:] == np.float16(7.0))
    Y = Yb[:, :d_out]
    assert np.array_equal(Y.view(np.uint16), _np(Y2).view(np.uint16))
    check_gemm(f"split {d_out}x{d_in} K={K} M={M}", c, X, torch.from_numpy(np.ascontiguousarray(Y)))


@pytest.mark.parametrize("d_out,d_in,M,identity", [(70, 33792, 9, False), (130, 1152, 130, True),
                                                   (64, 1024, 1030, False)])
def test_gemm_activation_reorder(d_out, d_in, M, identity):
    """The activation reorder before the GEMM: a row too wide to stage in LDS (element-wise
    gather), pi = NULL on the prefill path, and many rows per reorder workgroup."""
    rng = W.rng_for(147, d_in, M)
    c = W.draw_codes(rng, d_out, d_in, 64, 4)
    if identity:
        c.pi = np.arange(d_in, dtype=np.int32)
    X = W.draw_x(rng, (M, d_in))
    p = upload_pack(c)
    if identity:
        p = dataclasses.replace(p, pi=None)
    Y = sage.gemm_small(p, _dev(X))
    check_gemm(f"reorder {d_out}x{d_in} M={M} identity={identity}", c, X, Y)


@pytest.mark.parametrize("M", [9, 40, 96, 300])
def test_gemm_pre_permuted_strided_input(M):
    """pi = NULL and 16-byte aligned rows: the activations are read in place (no reorder), here
    with a row stride wider than d_in, on the small-batch and the prefill paths."""
    import torch
    rng = W.rng_for(148, M)
    d_out, d_in = 200, 1152
    c = W.draw_codes(rng, d_out, d_in, 64, 4)
    c.pi = np.arange(d_in, dtype=np.int32)
    X = W.draw_x(rng, (M, d_in))
    Xbig = torch.zeros((M, d_in + 24), dtype=torch.float16, device="cuda")
    Xbig[:, :d_in] = _dev(X)
    p = dataclasses.replace(upload_pack(c), pi=None)
    Y = sage.gemm_small(p, Xbig[:, :d_in])
    check_gemm(f"pre-permuted strided M={M}", c, X, Y)


def test_gemm_strided_rows():
    import torch
    c = W.draw_codes(W.rng_for(141), 200, 512, 32, 5)
    X = W.draw_x(W.rng_for(142), (6, 512))
    Xbig = torch.zeros((6, 520), dtype=torch.float16, device="cuda")
    Xbig[:, :512] = _dev(X)
    Ybig = torch.full((6, 210), 7.0, dtype=torch.float16, device="cuda")
    sage.gemm_small(upload_pack(c), Xbig[:, :512], Y=Ybig[:, :200])
    torch.cuda.synchronize()
    check_gemm("strided", c, X, Ybig[:, :200])
    assert np.all(_np(Ybig[:, 200:]) == 7.0)


# ------------------------------------------------------------------------------ routed experts

@pytest.fixture(scope="module")
def moe_packs():
    moe = W.moe_layer(splits=W.SPLITS_FIVE, experts_to_build=range(128))
    packs = [{n: upload_pack(moe.experts[e][n]) for n in ("gate", "up", "down")}
             for e in range(moe.n_experts)]
    return moe, packs


def test_moe_gemv_down_per_slot_inputs(moe_packs):
    """sage_moe_gemv in its one-matrix form: every routed expert's down projection on its own
    intermediate vector (x_stride = 768), 128 experts with mixed splits, top-8."""
    import torch
    moe, packs = moe_packs
    table, _ = sage.expert_table([packs[e]["down"] for e in range(moe.n_experts)], "cuda")
    ids = _dev(moe.ids)
    k = len(moe.ids)
    h = _dev(moe.h)
    y = torch.full((k, W.MOE_HIDDEN + 8), 5.0, dtype=torch.float16, device="cuda")
    log(f"[moe] ids={moe.ids.tolist()} splits={[moe.experts[int(e)]['down'].K for e in moe.ids]}")
    sage.moe_gemv(table, ids, h, W.MOE_INTER, y.view(-1), W.MOE_HIDDEN + 8)
    torch.cuda.synchronize()
    assert np.all(_np(y[:, W.MOE_HIDDEN:]) == 5.0)
    for s, e in enumerate(moe.ids):
        check_gemv(f"moe e{int(e)}.down", moe.experts[int(e)]["down"], moe.h[s], y[s, :W.MOE_HIDDEN])


def test_moe_gemv_grouped_gate_up_shared_input(moe_packs):
    """sage_moe_gemv_grouped: gate and up of every routed expert on the shared token (x_stride 0)
    in one launch."""
    import torch
    moe, packs = moe_packs
    table, n_mats = sage.expert_table([[packs[e]["gate"], packs[e]["up"]]
                                       for e in range(moe.n_experts)], "cuda")
    assert n_mats == 2
    ids = _dev(moe.ids)
    k = len(moe.ids)
    x = _dev(moe.x)
    yg = torch.empty((k, W.MOE_INTER), dtype=torch.float16, device="cuda")
    yu = torch.empty_like(yg)
    sage.moe_gemv_grouped(table, ids, [x, x], [0, 0], [yg.view(-1), yu.view(-1)],
                          [W.MOE_INTER, W.MOE_INTER])
    for s, e in enumerate(moe.ids):
        ex = moe.experts[int(e)]
        check_gemv(f"moe e{int(e)}.gate", ex["gate"], moe.x, yg[s])
        check_gemv(f"moe e{int(e)}.up", ex["up"], moe.x, yu[s])


def test_moe_gemv_grouped_whole_layer_and_shapes_per_expert():
    """Three matrices per expert in one launch, with shapes that differ between experts (read
    from the device descriptors) and some experts without a permutation; repeat calls give the
    same bits."""
    import torch
    rng = W.rng_for(170)
    n_exp = 12
    exps = []
    for e in range(n_exp):
        K, V = W.SPLITS_FIVE[e % 5]
        hid, inter = 256 * (1 + e % 3), 128 * (1 + e % 4)
        exps.append([W.draw_codes(rng, inter, hid, K, V), W.draw_codes(rng, inter, hid, K, V),
                     W.draw_codes(rng, hid, inter, K, V)])
    packs = [[upload_pack(c) for c in ex] for ex in exps]
    for e in range(0, n_exp, 3):
        packs[e][2] = dataclasses.replace(packs[e][2], pi=None)
    table, _ = sage.expert_table(packs, "cuda")
    ids = np.array([7, 0, 11, 4, 2], dtype=np.int32)
    x = W.draw_x(rng, (768,))
    H = W.draw_x(rng, (len(ids), 512))
    ya = torch.zeros((len(ids), 512), dtype=torch.float16, device="cuda")
    yb = torch.zeros_like(ya)
    yc = torch.zeros((len(ids), 768), dtype=torch.float16, device="cuda")
    args = (table, _dev(ids), [_dev(x), _dev(x), _dev(H).view(-1)], [0, 0, 512],
            [ya.view(-1), yb.view(-1), yc.view(-1)], [512, 512, 768])
    sage.moe_gemv_grouped(*args)
    torch.cuda.synchronize()
    first = [_np(t).copy() for t in (ya, yb, yc)]
    sage.moe_gemv_grouped(*args)
    torch.cuda.synchronize()
    for t, f in zip((ya, yb, yc), first):
        assert np.array_equal(_np(t), f)
    for s, e in enumerate(ids):
        g, u, d = exps[int(e)]
        check_gemv(f"e{e}.gate", g, x[:g.d_in], ya[s, :g.d_out])
        check_gemv(f"e{e}.up", u, x[:u.d_in], yb[s, :u.d_out])
        check_gemv(f"e{e}.down", d, H[s, :d.d_in], yc[s, :d.d_out], stored_order=(int(e) % 3 == 0))


def test_moe_gemv_invalid_id_skips_slot(moe_packs):
    """A routed id outside [0, n_experts) leaves its slot's output unwritten; the others run."""
    import torch
    moe, packs = moe_packs
    table, _ = sage.expert_table([packs[e]["down"] for e in range(moe.n_experts)], "cuda")
    ids = np.array([3, -1, 128, 5], dtype=np.int32)
    h = W.draw_x(W.rng_for(171), (4, W.MOE_INTER))
    y = torch.full((4, W.MOE_HIDDEN), 3.0, dtype=torch.float16, device="cuda")
    sage.moe_gemv(table, _dev(ids), _dev(h).view(-1), W.MOE_INTER, y.view(-1), W.MOE_HIDDEN)
    torch.cuda.synchronize()
    assert np.all(_np(y[1]) == 3.0) and np.all(_np(y[2]) == 3.0)
    check_gemv("slot 0", moe.experts[3]["down"], h[0], y[0])
    check_gemv("slot 3", moe.experts[5]["down"], h[3], y[3])


def test_stream_read_reference_runs():
    """The measurement helper reads a buffer (including a ragged last workgroup) and writes nothing."""
    import torch
    buf = torch.ones(3 * 65536 + 160, dtype=torch.uint8, device="cuda")
    sink = sage.stream_read(buf)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
