"""A synthetic end-to-end decode step on SAGE-packed weights (SAGE paper §3.5 and App. A.2).

A Qwen3-4B-shaped decoder stack (hidden 2560, 32 query heads and 8 key/value heads of 128, MLP
9728, 36 layers) whose seven projections per layer are SAGE-packed matrices run by libsage, in
the paper's compiled-decoding form (§3.5): each permuting producer writes its output in the
stored order of the matrices that read it, so those run with pi = NULL.

One layer, for one new token at position n:

    a = RMSNorm(h) written in q/k/v's stored order          (sage_rmsnorm_permute)
    q, k, v = W_q a, W_k a, W_v a                          (one sage_gemv_multi launch)
    q, k = per-head RMSNorm (Qwen3's q/k norms), rotary position n (PyTorch)
    K[:, n], V[:, n] = k, v;  o = softmax(q K[:, :n+1]^T / sqrt(128)) V[:, :n+1]
                                                             (PyTorch, grouped-query, fp16 products)
    h = h + W_o o                                            (sage_gemv: o arrives in original
                                                              order, the product gathers it)
    b = RMSNorm(h) written in gate/up's stored order         (sage_rmsnorm_permute)
    g, u = W_gate b, W_up b                                  (one sage_gemv_multi launch)
    m = silu(g) * u written in down's stored order           (sage_silu_mul_permute)
    h = h + W_down m                                         (sage_gemv)

The token embedding, the final norm and the LM head lie outside the stack. Activations and the
key/value caches are fp16, as in the paper's end-to-end runs (§4.4: FP16 activations and KV cache);
the per-head norms and the rotation are computed in fp32 and rounded to fp16 once.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Tuple

import bit_vector_quantized_amd as sage


@dataclass(frozen=True)
class Dims:
    hidden: int = 2560
    heads: int = 32
    kv_heads: int = 8
    head_dim: int = 128
    inter: int = 9728
    layers: int = 36
    eps: float = 1e-6
    rope_theta: float = 1e6


QWEN3_4B = Dims()


@dataclass
class LayerWeights:
    """One layer's packed projections and norm weights. q/k/v/gate/up/down are stored with
    pi = NULL (their inputs come from the permuting producers in stored order); o keeps its pi."""

    q: sage.Packed
    k: sage.Packed
    v: sage.Packed
    o: sage.Packed
    gate: sage.Packed
    up: sage.Packed
    down: sage.Packed
    pi_attn: "object"     # int32 [hidden], stored order of q/k/v
    pi_mlp: "object"      # int32 [hidden], stored order of gate/up
    pi_down: "object"     # int32 [inter], stored order of down
    ln_attn: "object"     # fp16 [hidden]
    ln_mlp: "object"      # fp16 [hidden]
    q_norm: "object"      # fp16 [head_dim]
    k_norm: "object"      # fp16 [head_dim]


def _without_pi(p: sage.Packed) -> sage.Packed:
    return sage.Packed(p.d_out, p.d_in, p.log2K, p.V, p.packed, p.codebook, None)


def layer_from_packed(q, k, v, o, gate, up, down, ln_attn, ln_mlp, q_norm, k_norm) -> LayerWeights:
    """A layer from packed matrices that carry their pi (q/k/v share one, gate/up share one)."""
    return LayerWeights(_without_pi(q), _without_pi(k), _without_pi(v), o, _without_pi(gate),
                        _without_pi(up), _without_pi(down), q.pi, gate.pi, down.pi,
                        ln_attn, ln_mlp, q_norm, k_norm)


def random_layer(gen, dims: Dims = QWEN3_4B, K: int = 64, V: int = 4,
                 mu_max: float = 0.05, delta_range: Tuple[float, float] = (0.001, 0.01)
                 ) -> LayerWeights:
    """Seeded synthetic layer drawn on the device (torch generator `gen`): uniform codeword
    indices, radius codes and sign bytes, grid offsets in [0, mu_max) and steps in delta_range
    (weights of a few hundredths, as in trained models, so the 36-layer residual stream stays in
    fp16 range), one |N(0, I)| unit codebook per matrix, one random permutation per input."""
    import torch
    dev = "cuda"
    L = K.bit_length() - 1

    def pack(d_out, d_in, pi):
        ns, ng = d_in // 8, d_in // 128
        signs = torch.randint(0, 256, (d_out, ns), dtype=torch.uint8, device=dev, generator=gen)
        idx = torch.randint(0, K, (d_out, ns), dtype=torch.uint8, device=dev, generator=gen)
        rcode = torch.randint(0, 1 << V, (d_out, ns), dtype=torch.uint8, device=dev, generator=gen)
        mu = (torch.rand((d_out, ng), device=dev, generator=gen) * mu_max).half()
        lo, hi = delta_range
        delta = (lo + torch.rand((d_out, ng), device=dev, generator=gen) * (hi - lo)).half()
        cb = torch.randn((K, 8), device=dev, generator=gen).abs()
        cb = (cb / cb.norm(dim=1, keepdim=True)).half()
        return sage.pack(signs, idx, rcode, mu, delta, cb, pi, L, V)

    def perm(d):
        return torch.randperm(d, device=dev, generator=gen).to(torch.int32)

    def gamma(d):
        return (1.0 + 0.1 * torch.randn(d, device=dev, generator=gen)).half()

    H, D = dims.hidden, dims.head_dim
    pa, po, pm, pd = perm(H), perm(dims.heads * D), perm(H), perm(dims.inter)
    return layer_from_packed(
        pack(dims.heads * D, H, pa), pack(dims.kv_heads * D, H, pa), pack(dims.kv_heads * D, H, pa),
        pack(H, dims.heads * D, po), pack(dims.inter, H, pm), pack(dims.inter, H, pm),
        pack(H, dims.inter, pd), gamma(H), gamma(H), gamma(D), gamma(D))


class DecodeStack:
    """The stack with its key/value caches. `ctx` positions are filled with seeded random keys and
    values (the prompt); each step appends one token."""

    def __init__(self, layers: List[LayerWeights], dims: Dims = QWEN3_4B, ctx: int = 1024,
                 max_new: int = 64, gen=None):
        import torch
        self.layers = layers
        self.dims = dims
        self.ctx = ctx
        self.pos = ctx
        n = ctx + max_new
        self.max_len = n
        shape = (len(layers), dims.kv_heads, n, dims.head_dim)
        self.kcache = torch.zeros(shape, dtype=torch.float16, device="cuda")
        self.vcache = torch.zeros(shape, dtype=torch.float16, device="cuda")
        if ctx > 0:
            self.kcache[:, :, :ctx].normal_(generator=gen)
            self.vcache[:, :, :ctx].normal_(generator=gen)
        # rotary tables for every position the caches can hold, [n, head_dim / 2] each
        half = dims.head_dim // 2
        inv_freq = 1.0 / (dims.rope_theta ** (
            torch.arange(0, half, dtype=torch.float64, device="cuda") / half))
        ang = torch.arange(n, dtype=torch.float64, device="cuda")[:, None] * inv_freq[None, :]
        # rotation of a head as x * cos2 + roll(x, half) * sin2: cos2 = [cos, cos], sin2 = [-sin, sin]
        cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
        self.cos2 = torch.cat((cos, cos), dim=1).contiguous()
        self.sin2 = torch.cat((-sin, sin), dim=1).contiguous()
        # per-head norm weights of the 32 query and 8 key heads as one [40, head_dim] block, the
        # query rows scaled by head_dim^-1/2 (the attention scale, folded in once)
        scale = dims.head_dim ** -0.5
        self.qk_w = [torch.cat((lw.q_norm.float().expand(dims.heads, dims.head_dim) * scale,
                                lw.k_norm.float().expand(dims.kv_heads, dims.head_dim)))
                     .contiguous() for lw in layers]

    # -- the linear chains (libsage kernels) --------------------------------------------------
    def attn_in(self, lw: LayerWeights, h):
        """a = RMSNorm(h) in q/k/v's stored order; q, k, v (fp16) from one launch, written next to
        each other in one buffer (so the query and key heads form one block)."""
        import torch
        d = self.dims
        a = sage.rmsnorm_permute(h, lw.ln_attn, d.eps, lw.pi_attn)
        nq, nk = d.heads * d.head_dim, d.kv_heads * d.head_dim
        qkv = torch.empty(nq + 2 * nk, dtype=torch.float16, device=h.device)
        q, k, v = qkv[:nq], qkv[nq:nq + nk], qkv[nq + nk:]
        sage.gemv_multi([lw.q, lw.k, lw.v], [a, a, a], ys=[q, k, v])
        return a, q, k, v

    def mlp(self, lw: LayerWeights, h):
        """b = RMSNorm(h) in gate/up's stored order; g, u; m = silu(g) * u in down's stored order;
        d = W_down m."""
        b = sage.rmsnorm_permute(h, lw.ln_mlp, self.dims.eps, lw.pi_mlp)
        g, u = sage.gemv_multi([lw.gate, lw.up], [b, b])
        m = sage.silu_mul_permute(g, u, lw.pi_down)
        d = sage.gemv(lw.down, m)
        return b, g, u, m, d

    # -- attention (PyTorch) --------------------------------------------------------------------
    def attention(self, li: int, lw: LayerWeights, q, k, v):
        """Attention output (fp16 [heads * head_dim], original order) for the token at self.pos."""
        import torch
        import torch.nn.functional as F
        d = self.dims
        D, nh, g = d.head_dim, d.heads + d.kv_heads, d.heads // d.kv_heads
        if k.data_ptr() == q.data_ptr() + q.numel() * q.element_size():
            qk = torch.as_strided(q, (nh, D), (D, 1))      # q and k adjacent (attn_in)
        else:
            qk = torch.cat((q, k)).view(nh, D)
        # per-head RMSNorm (query rows carry the attention scale) and the rotation, all 40 heads
        x = F.rms_norm(qk.float(), (D,), None, d.eps) * self.qk_w[li]
        x = torch.addcmul(x * self.cos2[self.pos], torch.roll(x, D // 2, dims=1), self.sin2[self.pos])
        self.kcache[li, :, self.pos] = x[d.heads:]        # rounded to fp16 by the copy
        self.vcache[li, :, self.pos] = v.view(d.kv_heads, D)
        n = self.pos + 1
        # grouped-query attention for one query as two batched fp16 products: the g query heads of
        # a key/value head form the columns of one operand [kv_heads, head_dim, g]; the cached keys
        # and values are read in place
        qg = torch.empty((d.kv_heads, D, g), dtype=torch.float16, device=q.device)
        qg.copy_(x[:d.heads].view(d.kv_heads, g, D).transpose(1, 2))
        s = torch.matmul(self.kcache[li, :, :n], qg)                 # [kv_heads, n, g]
        pr = torch.softmax(s, dim=1, dtype=torch.float32).half()
        o = torch.matmul(pr.transpose(1, 2), self.vcache[li, :, :n])  # [kv_heads, g, head_dim]
        return o.reshape(d.heads * D)

    def layer(self, li: int, h):
        lw = self.layers[li]
        _, q, k, v = self.attn_in(lw, h)
        o = self.attention(li, lw, q, k, v)
        h = h + sage.gemv(lw.o, o)
        d = self.mlp(lw, h)[-1]
        return h + d

    def step(self, h):
        """One decode step: the token's hidden state through every layer."""
        if self.pos >= self.max_len:
            raise RuntimeError("key/value caches are full")
        for li in range(len(self.layers)):
            h = self.layer(li, h)
        self.pos += 1
        return h


def time_steps(stack: DecodeStack, h0, warmup: int = 5, measure: int = 10):
    """The pages' protocol (SAGE paper App. A.2): `warmup` steps, then `measure` steps each timed
    with GPU events on the current stream; returns the per-step times in ms (the caller takes
    the median)."""
    import torch
    h = h0
    for _ in range(warmup):
        h = stack.step(h)
    times = []
    for _ in range(measure):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        h = stack.step(h)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    return times, h


def median(xs) -> float:
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
