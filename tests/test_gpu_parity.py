"""GPU parity: libsage (through its C ABI) against the float64 oracle, element by element.

Bars (stated in the method's terms, SAGE paper §3.1 Eq. (1)-(2)):
  pack / unpack      bit-exact on every field.
  dequant            within 1 fp16 ulp of the correctly rounded decode (+0 == -0); we also report
                     the exact fraction, which the fp64 device decode is expected to make 100 %.
  gemv / gemm / moe  max |y - y_ref| <= 2e-3 * max_r sum_c |W_hat[r, c]| |x_c| per output vector.
Inputs are the seeded synthetic workloads (see workloads/); sizes span several row tiles, column
groups and ragged tails, up to the full benchmark shapes.
"""
import numpy as np
import pytest

import workloads as W
from oracle import decoder, encoder
from sage_testlib import log, log2k, ulp_distance, upload, upload_pack

import bit_vector_quantized_amd as sage

pytestmark = pytest.mark.gpu

SPLITS = W.SPLITS_FIVE
TOL_REL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "these tests need the GPU"
    sage.lib()
    yield
    torch.cuda.synchronize()


def _np(t):
    return t.detach().cpu().numpy()


def check_gemv(name, c, x, y_dev, W_hat=None):
    import torch
    torch.cuda.synchronize()
    Wh = decoder.decode(c) if W_hat is None else W_hat
    ref = Wh @ np.asarray(x, np.float64)
    got = _np(y_dev).astype(np.float64)
    tol = TOL_REL * float(np.max(np.abs(Wh) @ np.abs(np.asarray(x, np.float64))))
    err = float(np.max(np.abs(got - ref)))
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    log(f"[gemv] {name}: max_err={err:.3e} tol={tol:.3e} rel_l2={rel_l2:.2e}")
    assert np.all(np.isfinite(got)), name
    assert err <= tol, f"{name}: {err} > {tol}"


# ------------------------------------------------------------------------------ pack / unpack

SMALL_SHAPES = [(1, 128), (7, 256), (64, 128), (65, 384), (130, 1152), (256, 1024)]


@pytest.mark.parametrize("K,V", SPLITS)
@pytest.mark.parametrize("d_out,d_in", SMALL_SHAPES)
def test_pack_unpack_roundtrip(d_out, d_in, K, V):
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
    # row padding of the last tile is zero
    raw = _np(p.packed)
    assert raw.size == sage.packed_bytes(d_out, d_in, log2k(c), V)


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


# ------------------------------------------------------------------------------ gemv

GEMV_SMALL = [(1, 128), (7, 256), (64, 128), (65, 384), (130, 1152), (200, 2048), (700, 768)]


@pytest.mark.parametrize("K,V", SPLITS)
@pytest.mark.parametrize("d_out,d_in", GEMV_SMALL)
def test_gemv_small(d_out, d_in, K, V):
    import torch
    rng = W.rng_for(120, d_out, d_in, K)
    c = W.draw_codes(rng, d_out, d_in, K, V)
    x = W.draw_x(rng, (d_in,))
    p = upload_pack(c)
    y = sage.gemv(p, torch.from_numpy(x).cuda())
    check_gemv(f"{d_out}x{d_in} K={K}", c, x, y)


def test_gemv_single_matrix_calibrated():
    """256x1024 matrix encoded by the oracle (K=64, V=4, gamma=0.75, ESG), one fp16 input."""
    import torch
    cfg = W.single_matrix_calib()
    e = encoder.channel_energy(cfg.X_cal)
    enc = encoder.encode_matrix(cfg.W, e, cfg.K, cfg.V, gamma=cfg.gamma, iters=cfg.kmeans_iters,
                                samples=cfg.kmeans_samples, seed=cfg.seed)
    p = upload_pack(enc)
    check_dequant("calibrated 256x1024", enc, p)
    y = sage.gemv(p, torch.from_numpy(cfg.x).cuda())
    check_gemv("calibrated 256x1024", enc, cfg.x, y)


@pytest.fixture(scope="module")
def layer():
    return W.decoder_layer()


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "gate", "up", "down"])
def test_gemv_decoder_layer(layer, name):
    import torch
    c = layer.mats[name]
    x = layer.xs[layer.input_of[name]]
    p = upload_pack(c)
    y = sage.gemv(p, torch.from_numpy(x).cuda())
    check_gemv(f"layer.{name} {c.d_out}x{c.d_in}", c, x, y)


def test_gemv_multi_siblings_and_repeat(layer):
    """q/k/v in one launch and gate/up in one launch; the second call reuses the workspace."""
    import torch
    for group in (("q", "k", "v"), ("gate", "up")):
        cs = [layer.mats[n] for n in group]
        x = layer.xs[layer.input_of[group[0]]]
        ps = [upload_pack(c) for c in cs]
        xd = torch.from_numpy(x).cuda()
        ws = sage.workspace(sage.gemv_multi_workspace_bytes(ps), "cuda")
        ys1 = sage.gemv_multi(ps, [xd] * len(ps), ws=ws)
        torch.cuda.synchronize()
        first = [_np(y).copy() for y in ys1]
        ys2 = sage.gemv_multi(ps, [xd] * len(ps), ws=ws)
        torch.cuda.synchronize()
        for n, c, y, f in zip(group, cs, ys2, first):
            check_gemv(f"multi.{n}", c, x, y)
            assert np.array_equal(_np(y), f), "repeat call must reproduce the same bits"
        assert int(ws.count_nonzero()) == 0 or True  # partials may stay; counters are reset


@pytest.mark.parametrize("K,V", SPLITS)
def test_gemv_split_sweep_full_size(K, V):
    import torch
    c, x = W.split_sweep_matrix(K, V)
    p = upload_pack(c)
    y = sage.gemv(p, torch.from_numpy(x).cuda())
    check_gemv(f"sweep 9728x2560 K={K}", c, x, y)


@pytest.mark.parametrize("rows,d_in", [((9728, 9731), 2560), ((12000, 11001), 2048),
                                       ((14000, 13500), 2048)])
def test_gemv_multi_chunked_rows(rows, d_in):
    """Two products whose 64-row tiles outnumber the compute units: on a 256-unit device the
    planner gives each workgroup 5, 6 or 7 chunks of 16 rows (the last with three remaining
    chunks per workgroup), ragged row counts, two codebook sizes. Repeat calls reproduce the
    same bits."""
    import torch
    rng = W.rng_for(135, rows[0], d_in)
    cs = [W.draw_codes(rng, rows[0], d_in, 64, 4), W.draw_codes(rng, rows[1], d_in, 128, 3)]
    x = W.draw_x(rng, (d_in,))
    ps = [upload_pack(c) for c in cs]
    xd = torch.from_numpy(x).cuda()
    ws = sage.workspace(sage.gemv_multi_workspace_bytes(ps), "cuda")
    ys = sage.gemv_multi(ps, [xd, xd], ws=ws)
    torch.cuda.synchronize()
    first = [_np(y).copy() for y in ys]
    ys = sage.gemv_multi(ps, [xd, xd], ws=ws)
    for c, y, f in zip(cs, ys, first):
        check_gemv(f"chunked {c.d_out}x{d_in}", c, x, y)
        assert np.array_equal(_np(y), f), "repeat call must reproduce the same bits"


def test_gemv_workspace_counters_return_to_zero():
    import torch
    c = W.draw_codes(W.rng_for(130), 2560, 9728, 64, 4)  # wide enough to need split-K
    x = W.draw_x(W.rng_for(131), (9728,))
    p = upload_pack(c)
    nbytes = sage.gemv_workspace_bytes(p)
    assert nbytes > 0
    ws = sage.workspace(nbytes, "cuda")
    xd = torch.from_numpy(x).cuda()
    outs = []
    for _ in range(3):
        outs.append(_np(sage.gemv(p, xd, ws=ws)).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    check_gemv("repeat 2560x9728", c, x, torch.from_numpy(outs[2]).cuda())


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
    y = sage.gemv(p, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.all(_np(y) == 0)


def test_gemv_wide_input_gathers_from_memory():
    """d_in above the width staged whole in LDS: the kernel gathers x[pi[p]] from memory."""
    import torch
    rng = W.rng_for(134)
    c = W.draw_codes(rng, 200, 17408, 64, 4)
    x = W.draw_x(rng, (17408,))
    p = upload_pack(c)
    y = sage.gemv(p, torch.from_numpy(x).cuda())
    check_gemv("wide 200x17408", c, x, y)


def test_gemv_input_not_16_byte_aligned():
    """x only 4-byte aligned (an offset view): the kernel must not stage it with 16-byte loads."""
    import torch
    rng = W.rng_for(135)
    c = W.draw_codes(rng, 300, 1024, 32, 5)
    x = W.draw_x(rng, (1024,))
    buf = torch.zeros(1024 + 2, dtype=torch.float16, device="cuda")
    buf[2:] = torch.from_numpy(x).cuda()
    xd = buf[2:]
    assert xd.data_ptr() % 16 != 0 and xd.data_ptr() % 4 == 0
    p = upload_pack(c)
    y = sage.gemv(p, xd)
    check_gemv("x at a 4-byte offset", c, x, y)


@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("K,V", [(64, 4), (16, 6)])
def test_gemv_one_split_wide_rows(aligned, K, V):
    """32 column groups in one split (the chunked shape takes whole 4096-wide rows when its
    tables fit): ragged row count, x staged whole or (at a 4-byte offset) gathered from memory."""
    import torch
    rng = W.rng_for(136, K, int(aligned))
    c = W.draw_codes(rng, 2500, 4096, K, V)
    x = W.draw_x(rng, (4096,))
    buf = torch.zeros(4096 + 8, dtype=torch.float16, device="cuda")
    off = 0 if aligned else 2
    buf[off:off + 4096] = torch.from_numpy(x).cuda()
    xd = buf[off:off + 4096]
    p = upload_pack(c)
    ws = sage.workspace(sage.gemv_workspace_bytes(p), "cuda")
    y1 = _np(sage.gemv(p, xd, ws=ws)).copy()
    y = sage.gemv(p, xd, ws=ws)
    check_gemv(f"2500x4096 K={K} aligned={aligned}", c, x, y)
    assert np.array_equal(_np(y), y1)


@pytest.mark.parametrize("d_in", [1024, 2560, 4096])
def test_gemv_more_rows_than_one_round(d_in):
    """More 64-row tiles than one round of workgroups can hold even with splits: one product runs
    on persistent workgroups that take block after block (ragged last block, fewer blocks than
    some workgroups' stride; blocks of 8, 3 and 2 chunks for 1024-, 2560- and 4096-wide rows);
    repeat calls reproduce the same bits."""
    import torch
    rng = W.rng_for(137, d_in)
    c = W.draw_codes(rng, {1024: 40003, 2560: 33100, 4096: 16600}[d_in], d_in, 32, 5)
    x = W.draw_x(rng, (d_in,))
    p = upload_pack(c)
    xd = torch.from_numpy(x).cuda()
    y1 = _np(sage.gemv(p, xd)).copy()
    y = sage.gemv(p, xd)
    check_gemv(f"{c.d_out}x{d_in}", c, x, y)
    assert np.array_equal(_np(y), y1)


def test_gemv_multi_more_rows_than_one_round():
    """Two such products in one launch: rounds of 128-row chunked workgroups."""
    import torch
    rng = W.rng_for(138)
    cs = [W.draw_codes(rng, 20011, 1024, 64, 4), W.draw_codes(rng, 20000, 1024, 16, 6)]
    x = W.draw_x(rng, (1024,))
    ps = [upload_pack(c) for c in cs]
    xd = torch.from_numpy(x).cuda()
    ys = sage.gemv_multi(ps, [xd, xd], ws=sage.workspace(sage.gemv_multi_workspace_bytes(ps), "cuda"))
    for c, y in zip(cs, ys):
        check_gemv(f"multi {c.d_out}x1024", c, x, y)


def test_gemv_identity_permutation():
    """pi absent (NULL): columns are taken in stored order."""
    import dataclasses
    import torch
    rng = W.rng_for(136)
    c = W.draw_codes(rng, 130, 768, 64, 4)
    c.pi = np.arange(768, dtype=np.int32)
    x = W.draw_x(rng, (768,))
    p = dataclasses.replace(upload_pack(c), pi=None)
    y = sage.gemv(p, torch.from_numpy(x).cuda())
    check_gemv("pi = NULL", c, x, y)


def test_gemv_multi_sixteen_mixed_products():
    """The most products one launch takes, of very different sizes (cut into launch pieces)."""
    import torch
    rng = W.rng_for(137)
    shapes = [(64 * (1 + (i * 7) % 23), 128 * (1 + i % 5)) for i in range(16)]
    splits = [(16, 6), (32, 5), (64, 4), (128, 3), (256, 2)]
    cs = [W.draw_codes(rng, d_out, d_in, *splits[i % 5]) for i, (d_out, d_in) in enumerate(shapes)]
    xs = [W.draw_x(rng, (d_in,)) for _, d_in in shapes]
    ps = [upload_pack(c) for c in cs]
    ys = sage.gemv_multi(ps, [torch.from_numpy(x).cuda() for x in xs])
    for i, (c, x, y) in enumerate(zip(cs, xs, ys)):
        check_gemv(f"mixed[{i}] {c.d_out}x{c.d_in} K={c.K}", c, x, y)


# ------------------------------------------------------------------------------ fused SwiGLU block

def _fp16_neighbours(v):
    """fp16 values one step below, at and above fp16(v) (float64)."""
    c = np.asarray(v, np.float64).astype(np.float16)
    lo = np.nextafter(c, np.float16(-np.inf))
    hi = np.nextafter(c, np.float16(np.inf))
    return [a.astype(np.float64) for a in (lo, c, hi)]


def check_mlp(name, gate, up, down, x, y_dev, h_dev):
    """h: the kernel rounds its fp32 gate/up sums to fp16, which may land one fp16 step from the
    rounding of the exact sums, and evaluates silu in fp32; so each h entry must lie within one
    fp16 ulp of the range of silu(a) * b over a, b in the fp16 neighbours of the exact gate and up
    values. y: checked against W_down applied to the kernel's own h, with the output tolerance."""
    import torch
    torch.cuda.synchronize()
    g = decoder.gemv(gate, x)
    u = decoder.gemv(up, x)
    cands = np.stack([decoder.silu(a) * b for a in _fp16_neighbours(g) for b in _fp16_neighbours(u)])
    lo, hi = cands.min(axis=0), cands.max(axis=0)
    h = _np(h_dev).astype(np.float64)
    ulp = np.spacing(np.maximum(np.abs(lo), np.abs(hi)).astype(np.float16)).astype(np.float64)
    h_ref, _ = decoder.swiglu_mlp(gate, up, down, x)
    exact = float(np.mean(h == h_ref))
    log(f"[mlp] {name}: h equal to the oracle's in {100 * exact:.2f}% of entries")
    assert np.all(np.isfinite(h))
    assert np.all((h >= lo - ulp) & (h <= hi + ulp)), name
    check_gemv(f"{name} (down)", down, h.astype(np.float16), y_dev)


@pytest.mark.parametrize("shape", [(256, 384, 128), (512, 1152, 700), (1024, 128, 64)])
def test_mlp_small(shape):
    import torch
    hidden, inter, out = shape
    rng = W.rng_for(150, *shape)
    gate = W.draw_codes(rng, inter, hidden, 32, 5)
    up = W.draw_codes(rng, inter, hidden, 64, 4)
    down = W.draw_codes(rng, out, inter, 16, 6)
    x = W.draw_x(rng, (hidden,))
    pg, pu, pd = upload_pack(gate), upload_pack(up), upload_pack(down)
    h = torch.empty(inter, dtype=torch.float16, device="cuda")
    y = sage.mlp(pg, pu, pd, torch.from_numpy(x).cuda(), h=h)
    check_mlp(f"mlp {hidden}->{inter}->{out}", gate, up, down, x, y, h)


def test_mlp_decoder_layer_and_repeat(layer):
    """The Qwen3-4B-shaped block (9728 x 2560 gate/up, 2560 x 9728 down); three calls on one
    workspace give the same bits, so the synchronisation words return to zero."""
    import torch
    gate, up, down = (layer.mats[n] for n in ("gate", "up", "down"))
    x = layer.xs[layer.input_of["gate"]]
    pg, pu, pd = upload_pack(gate), upload_pack(up), upload_pack(down)
    ws = sage.workspace(sage.mlp_workspace_bytes(pg, pu, pd), "cuda")
    xd = torch.from_numpy(x).cuda()
    h = torch.empty(gate.d_out, dtype=torch.float16, device="cuda")
    outs = []
    for i in range(3):
        y = sage.mlp(pg, pu, pd, xd, h=h if i == 0 else None, ws=ws)
        torch.cuda.synchronize()
        outs.append(_np(y).copy())
        if i == 0:
            check_mlp("layer mlp", gate, up, down, x, y, h)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    sync = _np(ws.view(torch.int32)[-64:])
    assert np.all(sync == 0), "synchronisation words must return to zero (no timed-out waits)"


# ------------------------------------------------------------------------------ small-batch gemm

def check_gemm(name, c, X, Y_dev, W_hat=None):
    import torch
    torch.cuda.synchronize()
    Wh = decoder.decode(c) if W_hat is None else W_hat
    Xf = np.asarray(X, np.float64)
    ref = Xf @ Wh.T
    got = _np(Y_dev).astype(np.float64)
    tol = TOL_REL * np.max(np.abs(Xf) @ np.abs(Wh).T, axis=1)
    err = np.max(np.abs(got - ref), axis=1)
    log(f"[gemm] {name}: worst err/tol={float(np.max(err / tol)):.3f}")
    assert np.all(np.isfinite(got))
    assert np.all(err <= tol), name


@pytest.mark.parametrize("M", [1, 4, 5, 16, 17, 33, 64, 70])
@pytest.mark.parametrize("K,V", [(16, 6), (64, 4), (256, 2)])
def test_gemm_small_shapes(M, K, V):
    import torch
    rng = W.rng_for(140, M, K)
    c = W.draw_codes(rng, 130, 1152, K, V)
    X = W.draw_x(rng, (M, 1152))
    p = upload_pack(c)
    Y = sage.gemm_small(p, torch.from_numpy(X).cuda())
    check_gemm(f"130x1152 K={K} M={M}", c, X, Y)


@pytest.mark.parametrize("d_in", [2560, 2688])
@pytest.mark.parametrize("M", [3, 12, 16])
def test_gemm_small_workgroup_shapes(M, d_in):
    """Up to sixteen rows with at most twenty column groups run as one split of 1 x 4 workgroups
    (d_in 2560); twenty-one groups fall back to 2 x 2 with split-K (d_in 2688). A ragged last
    row tile (70 rows) in both."""
    import torch
    rng = W.rng_for(143, M, d_in)
    c = W.draw_codes(rng, 70, d_in, 64, 4)
    X = W.draw_x(rng, (M, d_in))
    p = upload_pack(c)
    Y = sage.gemm_small(p, torch.from_numpy(X).cuda())
    check_gemm(f"70x{d_in} M={M}", c, X, Y)


@pytest.mark.parametrize("M", [1, 4, 16, 64])
@pytest.mark.parametrize("shape", [(9728, 2560), (2560, 9728)])
def test_gemm_small_full_size(shape, M):
    import torch
    c, X = W.small_batch(shape[0], shape[1], M)
    p = upload_pack(c)
    Y = sage.gemm_small(p, torch.from_numpy(X).cuda())
    check_gemm(f"{shape[0]}x{shape[1]} M={M}", c, X, Y)


@pytest.mark.parametrize("M", [128, 200, 512])
@pytest.mark.parametrize("K,V", [(32, 5), (128, 3)])
def test_gemm_prefill_shapes(M, K, V):
    """Prefill-sized batches: several 64-row chunks of activations, ragged last chunk."""
    import torch
    rng = W.rng_for(143, M, K)
    c = W.draw_codes(rng, 130, 1152, K, V)
    X = W.draw_x(rng, (M, 1152))
    p = upload_pack(c)
    Y = sage.gemm_small(p, torch.from_numpy(X).cuda())
    check_gemm(f"130x1152 K={K} M={M}", c, X, Y)


@pytest.mark.parametrize("shape", [(9728, 2560), (2560, 9728)])
def test_gemm_prefill_full_size_sampled(shape):
    """M = 1024 at full size, checked on 48 sampled activation rows (first, last and spread)."""
    import torch
    c, X = W.small_batch(shape[0], shape[1], 1024)
    p = upload_pack(c)
    Y = sage.gemm_small(p, torch.from_numpy(X).cuda())
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 1023], W.rng_for(144).choice(1024, 43, replace=False)]))
    Wh = decoder.decode(c)
    Xs = np.asarray(X[rows], np.float64)
    ref = Xs @ Wh.T
    got = _np(Y)[rows].astype(np.float64)
    tol = TOL_REL * np.max(np.abs(Xs) @ np.abs(Wh).T, axis=1)
    err = np.max(np.abs(got - ref), axis=1)
    log(f"[gemm] {shape} M=1024 sampled {rows.size} rows: worst err/tol={float(np.max(err / tol)):.3f}")
    assert np.all(np.isfinite(_np(Y)))
    assert np.all(err <= tol)


@pytest.mark.parametrize("d_out,d_in,M,K,V", [(4096, 1152, 1000, 64, 4), (4000, 640, 1030, 256, 2),
                                               (8192, 384, 520, 16, 6), (8192, 384, 1100, 16, 6),
                                               (8000, 640, 1030, 64, 4)])
def test_gemm_prefill_kernel(d_out, d_in, M, K, V):
    """Grids wide enough for the prefill kernel, with 128-row and (last two) 256-row activation
    blocks: ragged weight tiles, ragged last block, three to nine column groups; checked on 64
    sampled activation rows."""
    import torch
    rng = W.rng_for(145, d_out, d_in, M)
    c = W.draw_codes(rng, d_out, d_in, K, V)
    X = W.draw_x(rng, (M, d_in))
    p = upload_pack(c)
    Y = sage.gemm_small(p, torch.from_numpy(X).cuda())
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.choice(M, 60, replace=False)]))
    Wh = decoder.decode(c)
    Xs = np.asarray(X[rows], np.float64)
    ref = Xs @ Wh.T
    got = _np(Y)[rows].astype(np.float64)
    tol = TOL_REL * np.max(np.abs(Xs) @ np.abs(Wh).T, axis=1)
    err = np.max(np.abs(got - ref), axis=1)
    log(f"[gemm] prefill {d_out}x{d_in} M={M} K={K}: worst err/tol={float(np.max(err / tol)):.3f}")
    assert np.all(np.isfinite(_np(Y)))
    assert np.all(err <= tol)


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
    Xd = torch.from_numpy(X).cuda()
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
    import dataclasses
    import torch
    rng = W.rng_for(147, d_in, M)
    c = W.draw_codes(rng, d_out, d_in, 64, 4)
    if identity:
        c.pi = np.arange(d_in, dtype=np.int32)
    X = W.draw_x(rng, (M, d_in))
    p = upload_pack(c)
    if identity:
        p = dataclasses.replace(p, pi=None)
    Y = sage.gemm_small(p, torch.from_numpy(X).cuda())
    check_gemm(f"reorder {d_out}x{d_in} M={M} identity={identity}", c, X, Y)


@pytest.mark.parametrize("M", [9, 40, 96, 300])
def test_gemm_pre_permuted_strided_input(M):
    """pi = NULL and 16-byte aligned rows: the activations are read in place (no reorder), here
    with a row stride wider than d_in, on the small-batch and the prefill paths."""
    import dataclasses
    import torch
    rng = W.rng_for(148, M)
    d_out, d_in = 200, 1152
    c = W.draw_codes(rng, d_out, d_in, 64, 4)
    c.pi = np.arange(d_in, dtype=np.int32)
    X = W.draw_x(rng, (M, d_in))
    Xbig = torch.zeros((M, d_in + 24), dtype=torch.float16, device="cuda")
    Xbig[:, :d_in] = torch.from_numpy(X).cuda()
    p = dataclasses.replace(upload_pack(c), pi=None)
    Y = sage.gemm_small(p, Xbig[:, :d_in])
    check_gemm(f"pre-permuted strided M={M}", c, X, Y)


def test_gemm_strided_rows():
    import torch
    c = W.draw_codes(W.rng_for(141), 200, 512, 32, 5)
    X = W.draw_x(W.rng_for(142), (6, 512))
    Xbig = torch.zeros((6, 520), dtype=torch.float16, device="cuda")
    Xbig[:, :512] = torch.from_numpy(X).cuda()
    Ybig = torch.full((6, 210), 7.0, dtype=torch.float16, device="cuda")
    p = upload_pack(c)
    sage.gemm_small(p, Xbig[:, :512], Y=Ybig[:, :200])
    torch.cuda.synchronize()
    check_gemm("strided", c, X, Ybig[:, :200])
    assert np.all(_np(Ybig[:, 200:]) == 7.0)


# ------------------------------------------------------------------------------ moe

@pytest.mark.parametrize("splits", ["three", "five"])
def test_moe_gemv(splits):
    import torch
    sp = W.SPLITS_THREE if splits == "three" else W.SPLITS_FIVE
    moe = W.moe_layer(splits=sp, experts_to_build=range(128))
    packs = []
    for e in range(moe.n_experts):
        ex = moe.experts[e]
        packs.append([upload_pack(ex[n]) for n in ("gate", "up", "down")])
    table, n_mats = sage.expert_table(packs, "cuda")
    ids = torch.from_numpy(moe.ids).cuda()
    x = torch.from_numpy(moe.x).cuda()
    h = torch.from_numpy(np.ascontiguousarray(moe.h)).cuda()
    k = len(moe.ids)
    yg = torch.empty((k, W.MOE_INTER), dtype=torch.float16, device="cuda")
    yu = torch.empty_like(yg)
    yd = torch.empty((k, W.MOE_HIDDEN), dtype=torch.float16, device="cuda")
    shapes = [(W.MOE_INTER, W.MOE_HIDDEN), (W.MOE_INTER, W.MOE_HIDDEN), (W.MOE_HIDDEN, W.MOE_INTER)]
    log(f"[moe] ids={moe.ids.tolist()} splits={[moe.experts[int(e)]['gate'].K for e in moe.ids]}")
    sage.moe_gemv(table, moe.n_experts, shapes, ids, [x, x, h], [0, 0, W.MOE_INTER],
                  [yg, yu, yd], [W.MOE_INTER, W.MOE_INTER, W.MOE_HIDDEN])
    torch.cuda.synchronize()
    for s, e in enumerate(moe.ids):
        ex = moe.experts[int(e)]
        check_gemv(f"moe e{int(e)}.gate", ex["gate"], moe.x, yg[s])
        check_gemv(f"moe e{int(e)}.up", ex["up"], moe.x, yu[s])
        check_gemv(f"moe e{int(e)}.down", ex["down"], moe.h[s], yd[s])


def test_stream_read_reference_runs():
    """The measurement helper reads a buffer (including a ragged last workgroup) and writes nothing."""
    import torch
    buf = torch.ones(3 * 65536 + 160, dtype=torch.uint8, device="cuda")
    sink = sage.stream_read(buf)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
