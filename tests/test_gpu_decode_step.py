"""The synthetic end-to-end decode step (bit_vector_quantized_amd/decode_step.py) against the
float64 oracle, stage by stage (SAGE paper §3.5 compiled decoding; App. A.2 for the step).

Each linear stage of one Qwen3-4B-shaped layer is checked on its own inputs, which are the
previous stage's fp16 outputs as the kernels produced them:
  producers (RMSNorm, silu*mul, written in the next matrix's stored order)
                 within 1 fp16 ulp of the correctly rounded float64 value;
  products       the tight per-element bound of the batch-one kernel (sage_testlib) against the
                 oracle product of the same input, and the 2e-3 relative contract bound.
The attention between the two chains is PyTorch's; the o projection that follows it gathers its
input through pi and is checked the same way. Whole steps are checked for finiteness and
bit-for-bit repetition. Weights and inputs are the seeded synthetic decoder layer (workloads/).
"""
import numpy as np
import pytest

import workloads as W
from oracle import decoder
from sage_testlib import batch_one_bounds, log, ulp_distance, upload_pack

import bit_vector_quantized_amd as sage

pytestmark = pytest.mark.gpu
EPS = 1e-6


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


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def _check_ulp(name, got, ref64):
    d = ulp_distance(got.view(np.uint16), ref64.astype(np.float16).view(np.uint16))
    log(f"[step] {name}: max ulp {int(d.max())}")
    assert int(d.max()) <= 1, name


def _check_product(name, c, x_np, y_dev, stored_order):
    ref, tight, contract = batch_one_bounds(c, x_np, stored_order)
    got = _host(y_dev).astype(np.float64)
    assert np.all(np.isfinite(got)), name
    err = np.abs(got - ref)
    log(f"[step] {name}: err/tight={float(np.max(err / tight)):.3f} contract={contract:.3e}")
    assert float(err.max()) <= contract, f"{name}: contract bound"
    bad = np.flatnonzero(err > tight)
    assert bad.size == 0, f"{name}: rows {bad[:8].tolist()} over the tight bound"


@pytest.fixture(scope="module")
def one_layer():
    from bit_vector_quantized_amd import decode_step as ds
    layer = W.decoder_layer()
    ps = {n: upload_pack(c) for n, c in layer.mats.items()}
    rng = W.rng_for(175)

    def gamma(d):
        return (1.0 + 0.2 * rng.standard_normal(d)).astype(np.float16)

    norms = {"ln_attn": gamma(2560), "ln_mlp": gamma(2560), "q_norm": gamma(128),
             "k_norm": gamma(128)}
    lw = ds.layer_from_packed(ps["q"], ps["k"], ps["v"], ps["o"], ps["gate"], ps["up"],
                              ps["down"], *[_dev(norms[k]) for k in ("ln_attn", "ln_mlp",
                                                                     "q_norm", "k_norm")])
    stack = ds.DecodeStack([lw], ctx=16, max_new=4)
    h = W.draw_x(rng, (2560,))
    return layer, lw, norms, stack, h


def test_attention_input_chain(one_layer):
    """h -> RMSNorm in q/k/v's stored order -> q, k, v with pi = NULL (one launch)."""
    layer, lw, norms, stack, h = one_layer
    a, q, k, v = stack.attn_in(lw, _dev(h))
    a_np = _host(a)
    pi = layer.mats["q"].pi
    _check_ulp("rmsnorm -> q/k/v order",
               a_np, decoder.rmsnorm_permute(h.astype(np.float64),
                                             norms["ln_attn"].astype(np.float64), EPS, pi))
    for name, y in (("q", q), ("k", k), ("v", v)):
        _check_product(f"{name} from the producer", layer.mats[name], a_np, y, stored_order=True)


def test_mlp_chain(one_layer):
    """h -> RMSNorm in gate/up's order -> gate, up -> silu*mul in down's order -> down."""
    layer, lw, norms, stack, h = one_layer
    b, g, u, m, d = stack.mlp(lw, _dev(h))
    b_np, g_np, u_np, m_np = _host(b), _host(g), _host(u), _host(m)
    _check_ulp("rmsnorm -> gate/up order",
               b_np, decoder.rmsnorm_permute(h.astype(np.float64),
                                             norms["ln_mlp"].astype(np.float64), EPS,
                                             layer.mats["gate"].pi))
    _check_product("gate", layer.mats["gate"], b_np, g, stored_order=True)
    _check_product("up", layer.mats["up"], b_np, u, stored_order=True)
    _check_ulp("silu*mul -> down order",
               m_np, decoder.silu_mul_permute(g_np.astype(np.float64), u_np.astype(np.float64),
                                              layer.mats["down"].pi))
    _check_product("down", layer.mats["down"], m_np, d, stored_order=True)


def test_output_projection_gathers(one_layer):
    """The attention output arrives in original order; o gathers it through its pi."""
    layer, lw, norms, stack, h = one_layer
    x = W.draw_x(W.rng_for(176), (4096,))
    y = sage.gemv(lw.o, _dev(x))
    _check_product("o (gathering)", layer.mats["o"], x, y, stored_order=False)


def test_steps_are_finite_and_repeat_bit_for_bit():
    """Two stacks built from the same seed take the same three steps to the same bits."""
    import torch
    from bit_vector_quantized_amd import decode_step as ds
    outs = []
    for _ in range(2):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(77)
        lws = [ds.random_layer(gen) for _ in range(2)]
        stack = ds.DecodeStack(lws, ctx=32, max_new=4, gen=gen)
        h = (torch.randn(2560, device="cuda", generator=gen) * 0.5).half()
        for _ in range(3):
            h = stack.step(h)
        outs.append(_host(h))
        assert stack.pos == 35
    assert np.all(np.isfinite(outs[0].astype(np.float64)))
    assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))


def test_full_cache_is_refused():
    import torch
    from bit_vector_quantized_amd import decode_step as ds
    gen = torch.Generator(device="cuda")
    gen.manual_seed(78)
    stack = ds.DecodeStack([ds.random_layer(gen)], ctx=2, max_new=1, gen=gen)
    h = torch.zeros(2560, dtype=torch.float16, device="cuda")
    stack.step(h)
    with pytest.raises(RuntimeError):
        stack.step(h)
