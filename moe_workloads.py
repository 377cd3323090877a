"""Seeded synthetic inputs for the routed-experts MoE layer.

This module is shared by the tests, the benchmark and the smoke check.  It
holds only the input recipes (random draws, the routing that a router outside
the layer would produce, and the block quantisation that turns fp32 draws
into the fp8 operands), none of the layer's own arithmetic.  It imports
neither the oracle nor the HIP library.

Workloads (shapes follow the model card "DeepSeek-OCR-2 MoE experts", its
benchmark paragraph, and the mirage issue "Supporting MegaKernel for DeepSeek
Models", Layer Tensor Details for moe_w13_fp8_layer / moe_w2_fp8_layer):

* ``tiny``            T=16, H=128, F=64, E=8, k=2, bf16
* ``ocr2_decode_t1``  T=1,  H=1280, F=896, E=64, k=6, bf16
* ``ocr2_decode_t4``  T=4,  same shapes and weights as t1
* ``ocr2_prefill``    T=2048, same shapes, bf16
* ``v3_fp8_decode``   T=128, H=7168, F=2048, E=128, k=8, fp8 block-scaled
* ``v3_fp8_prefill``  T=4096, same shapes and weights, Zipf(1.2) routing
* ``ocr2_prefill_shared``, ``ocr2_decode_t1_shared``: the OCR-2 workloads
  plus the model's two shared experts (same F as a routed expert), which
  every token passes through with weight 1
* ``v3_mxfp4_decode`` / ``v3_mxfp4_prefill``: the V3 expert-share shapes with
  MXFP4 routed weights (E2M1 + E8M0 per 32) and MXFP8 activations (E4M3 +
  E8M0 per 32), decode-batch (T=128) and Zipf prefill (T=4096) routing
"""

from __future__ import annotations

import torch

FP8_MAX = 448.0

CONFIGS = {
    "tiny": dict(T=16, H=128, F=64, E=8, k=2, kind="bf16", seed=1001,
                 routing="uniform_softmax", routed_scale=1.0),
    "ocr2_decode_t1": dict(T=1, H=1280, F=896, E=64, k=6, kind="bf16", seed=1002,
                           routing="uniform_softmax", routed_scale=1.0),
    "ocr2_decode_t4": dict(T=4, H=1280, F=896, E=64, k=6, kind="bf16", seed=1002,
                           routing="uniform_softmax", routed_scale=1.0),
    "ocr2_prefill": dict(T=2048, H=1280, F=896, E=64, k=6, kind="bf16", seed=1003,
                         routing="uniform_softmax", routed_scale=1.0),
    "v3_fp8_decode": dict(T=128, H=7168, F=2048, E=128, k=8, kind="fp8", seed=1004,
                          routing="sigmoid_topk", routed_scale=2.5),
    "v3_fp8_prefill": dict(T=4096, H=7168, F=2048, E=128, k=8, kind="fp8", seed=1004,
                           act_seed=1005, routing="zipf", zipf_s=1.2, zipf_zero=8,
                           routed_scale=2.5),
    "ocr2_prefill_shared": dict(T=2048, H=1280, F=896, E=64, k=6, kind="bf16", seed=1003,
                                routing="uniform_softmax", routed_scale=1.0, S=2, shared_seed=1006),
    "ocr2_decode_t1_shared": dict(T=1, H=1280, F=896, E=64, k=6, kind="bf16", seed=1002,
                                  routing="uniform_softmax", routed_scale=1.0, S=2,
                                  shared_seed=1006),
    "v3_mxfp4_decode": dict(T=128, H=7168, F=2048, E=128, k=8, kind="mxfp4", seed=1007,
                            routing="sigmoid_topk", routed_scale=2.5),
    "v3_mxfp4_prefill": dict(T=4096, H=7168, F=2048, E=128, k=8, kind="mxfp4", seed=1007,
                             act_seed=1005, routing="zipf", zipf_s=1.2, zipf_zero=8,
                             routed_scale=2.5),
}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


# ----------------------------------------------------------------- routing

def route_uniform_softmax(T, E, k, g, device="cpu", scale=1.0):
    """k distinct experts per token, uniform; weights = softmax of N(0,1) logits."""
    keys = torch.rand(T, E, generator=g, device=device)
    idx = keys.argsort(dim=1)[:, :k].to(torch.int32)
    logits = torch.randn(T, k, generator=g, device=device, dtype=torch.float32)
    w = torch.softmax(logits, dim=1) * scale
    return idx.contiguous(), w.to(torch.float32).contiguous()


def route_sigmoid_topk(T, E, k, g, device="cpu", scale=2.5):
    """top-k of sigmoid(N(0,1)) scores; weights = chosen scores / their sum * scale."""
    scores = torch.sigmoid(torch.randn(T, E, generator=g, device=device, dtype=torch.float32))
    top, idx = torch.topk(scores, k, dim=1)
    w = top / top.sum(dim=1, keepdim=True) * scale
    return idx.to(torch.int32).contiguous(), w.to(torch.float32).contiguous()


def route_zipf(T, E, k, g, device="cpu", s=1.2, n_zero=8, scale=2.5):
    """Skewed expert popularity: p(rank r) ~ r^-s over a seeded permutation of
    the experts, the ``n_zero`` coldest ranks get p = 0 (so those experts stay
    empty); k distinct experts per token by Gumbel top-k (sampling without
    replacement); weights = sigmoid(N(0,1)) of the chosen, renormalised * scale.
    """
    order = torch.randperm(E, generator=g, device=device)
    ranks = torch.arange(1, E + 1, device=device, dtype=torch.float64)
    pop_by_rank = ranks.pow(-s)
    if n_zero:
        pop_by_rank[E - n_zero:] = 0.0
    pop = torch.zeros(E, device=device, dtype=torch.float64)
    pop[order] = pop_by_rank
    logp = torch.log(pop / pop.sum())                       # -inf for empty experts
    u = torch.rand(T, E, generator=g, device=device, dtype=torch.float64)
    gumbel = -torch.log(-torch.log(u.clamp_min(1e-300)))
    _, idx = torch.topk(logp[None, :] + gumbel, k, dim=1)
    sc = torch.sigmoid(torch.randn(T, k, generator=g, device=device, dtype=torch.float32))
    w = sc / sc.sum(dim=1, keepdim=True) * scale
    return idx.to(torch.int32).contiguous(), w.to(torch.float32).contiguous()


# ------------------------------------------------------- input quantisation

def quantize_fp8_rows_torch(t):
    """fp32 [.., K] -> (fp8 e4m3fn codes as uint8 [.., K], fp32 scales [.., K/128]).

    Input recipe: one scale per row and 128-wide block, s = amax / 448, codes
    from t * (448 / amax) clamped to +-448 and cast with torch's e4m3fn cast;
    an all-zero block gets s = 1.
    """
    K = t.shape[-1]
    assert K % 128 == 0
    b = t.float().reshape(*t.shape[:-1], K // 128, 128)
    amax = b.abs().amax(dim=-1)
    zero = amax == 0
    safe = torch.where(zero, torch.ones_like(amax), amax)
    scale = torch.where(zero, torch.ones_like(amax), safe / FP8_MAX)
    v = (b * (FP8_MAX / safe)[..., None]).clamp(-FP8_MAX, FP8_MAX)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(t.shape)
    return codes.contiguous(), scale.float().contiguous()


# ------------------------------------------------------------- problems

def make_bf16_problem(T, H, F, E, k, seed, device="cpu", weight_std=0.02,
                      routing="uniform_softmax", routed_scale=1.0, gen_device=None):
    """bf16 operands drawn in the order gate_up, down, hidden, routing.

    Returns a dict of contiguous tensors on ``device``: hidden [T,H] bf16,
    gate_up [E,2F,H] bf16, down [E,H,F] bf16, top_k_index [T,k] int32,
    top_k_weights [T,k] fp32.
    """
    gd = gen_device or "cpu"
    g = _gen(seed, gd)
    gate_up = (torch.randn(E, 2 * F, H, generator=g, device=gd) * weight_std).to(torch.bfloat16)
    down = (torch.randn(E, H, F, generator=g, device=gd) * weight_std).to(torch.bfloat16)
    hidden = torch.randn(T, H, generator=g, device=gd).to(torch.bfloat16)
    if routing == "uniform_softmax":
        idx, w = route_uniform_softmax(T, E, k, g, gd, routed_scale)
    elif routing == "sigmoid_topk":
        idx, w = route_sigmoid_topk(T, E, k, g, gd, routed_scale)
    else:
        raise ValueError(routing)
    d = dict(hidden=hidden, gate_up=gate_up, down=down, top_k_index=idx, top_k_weights=w)
    return {n: v.to(device).contiguous() for n, v in d.items()}


def make_fp8_weights(H, F, E, seed, device="cpu", weight_std=0.02):
    """fp8 weights: per expert N(0, std) draws quantised per (row, 128 K block).

    gate_up codes [E,2F,H] uint8 + scales [E,2F,H/128]; down codes [E,H,F]
    uint8 + scales [E,H,F/128].  Drawn one expert at a time on ``device`` so
    that the fp32 intermediate stays one expert large.
    """
    g = _gen(seed, device)
    w13 = torch.empty(E, 2 * F, H, dtype=torch.uint8, device=device)
    w13s = torch.empty(E, 2 * F, H // 128, dtype=torch.float32, device=device)
    w2 = torch.empty(E, H, F, dtype=torch.uint8, device=device)
    w2s = torch.empty(E, H, F // 128, dtype=torch.float32, device=device)
    for e in range(E):
        c, s = quantize_fp8_rows_torch(torch.randn(2 * F, H, generator=g, device=device) * weight_std)
        w13[e].copy_(c)
        w13s[e].copy_(s)
    for e in range(E):
        c, s = quantize_fp8_rows_torch(torch.randn(H, F, generator=g, device=device) * weight_std)
        w2[e].copy_(c)
        w2s[e].copy_(s)
    return dict(gate_up=w13, gate_up_scale=w13s, down=w2, down_scale=w2s)


def make_fp8_activations(T, H, E, k, seed, device="cpu", routing="sigmoid_topk",
                         routed_scale=2.5, zipf_s=1.2, zipf_zero=8):
    """fp8 hidden states (N(0,1) quantised per token and 128 block) + routing."""
    g = _gen(seed, device)
    x = torch.randn(T, H, generator=g, device=device)
    xq, xs = quantize_fp8_rows_torch(x)
    if routing == "sigmoid_topk":
        idx, w = route_sigmoid_topk(T, E, k, g, device, routed_scale)
    elif routing == "zipf":
        idx, w = route_zipf(T, E, k, g, device, zipf_s, zipf_zero, routed_scale)
    elif routing == "uniform_softmax":
        idx, w = route_uniform_softmax(T, E, k, g, device, routed_scale)
    else:
        raise ValueError(routing)
    return dict(x=xq, x_scale=xs, top_k_index=idx, top_k_weights=w)


def make_fp8_problem(T, H, F, E, k, seed, device="cpu", act_seed=None, **kw):
    """Weights from ``seed`` then activations/routing from ``act_seed`` (or
    the seed + 1), so configs that share weights can share the first part."""
    p = make_fp8_weights(H, F, E, seed, device)
    p.update(make_fp8_activations(T, H, E, k, act_seed if act_seed is not None else seed + 1,
                                  device, **kw))
    return p


# -------------------------------------------- microscaling (MX) operands

_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _mx_exponents(b, emax):
    """Shared exponent per block of the last dim: floor(log2(amax)) - emax,
    clamped to [-127, 127]; an all-zero block gets -127."""
    amax = b.abs().amax(dim=-1)
    _, ex = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
    e = (ex.to(torch.int32) - 1) - emax
    e = torch.where(amax > 0, e, torch.full_like(e, -127))
    return e.clamp(-127, 127)


def quantize_mxfp8_rows_torch(t):
    """fp32 [.., K] -> (E4M3 codes uint8 [.., K], E8M0 scale bytes uint8 [.., K/32]).

    Input recipe (OCP Microscaling MXFP8): per 32-wide block, e =
    floor(log2(amax)) - 8, codes = torch's e4m3fn cast of t / 2^e clamped to
    +-448, scale byte e + 127.
    """
    K = t.shape[-1]
    assert K % 32 == 0
    b = t.float().reshape(*t.shape[:-1], K // 32, 32)
    e = _mx_exponents(b, 8)
    v = torch.ldexp(b, (-e).to(torch.float32)[..., None]).clamp(-448.0, 448.0)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(t.shape)
    return codes.contiguous(), (e + 127).to(torch.uint8).contiguous()


def quantize_mxfp4_rows_torch(t):
    """fp32 [.., K] -> (E2M1 codes packed two per byte uint8 [.., K/2], element
    2i in the low nibble; E8M0 scale bytes uint8 [.., K/32]).

    Input recipe (OCP Microscaling MXFP4): per 32-wide block, e =
    floor(log2(amax)) - 2, values t / 2^e clamped to +-6 and rounded to the
    nearest E2M1 value, ties to the even code (mantissa bit 0).
    """
    K = t.shape[-1]
    assert K % 32 == 0
    b = t.float().reshape(*t.shape[:-1], K // 32, 32)
    e = _mx_exponents(b, 2)
    v = torch.ldexp(b, (-e).to(torch.float32)[..., None]).clamp(-6.0, 6.0)
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float32, device=t.device)
    d = (v.abs()[..., None] - grid).abs()                       # [.., 8]
    is_min = d == d.amin(dim=-1, keepdim=True)
    even = (torch.arange(8, device=t.device) % 2) == 0
    even_min = is_min & even
    pick = torch.where(even_min.any(dim=-1), even_min.to(torch.uint8).argmax(dim=-1),
                       is_min.to(torch.uint8).argmax(dim=-1))
    codes = (pick | (torch.signbit(v).to(torch.int64) << 3)).to(torch.uint8).reshape(t.shape)
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


def make_mxfp4_weights(H, F, E, seed, device="cpu", weight_std=0.02):
    """MXFP4 weights: per expert N(0, std) draws quantised per (row, 32 K block).

    gate_up [E,2F,H/2] packed + scales [E,2F,H/32]; down [E,H,F/2] + [E,H,F/32].
    """
    g = _gen(seed, device)
    w13 = torch.empty(E, 2 * F, H // 2, dtype=torch.uint8, device=device)
    w13s = torch.empty(E, 2 * F, H // 32, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, F // 2, dtype=torch.uint8, device=device)
    w2s = torch.empty(E, H, F // 32, dtype=torch.uint8, device=device)
    for e in range(E):
        c, s_ = quantize_mxfp4_rows_torch(torch.randn(2 * F, H, generator=g, device=device) * weight_std)
        w13[e].copy_(c)
        w13s[e].copy_(s_)
    for e in range(E):
        c, s_ = quantize_mxfp4_rows_torch(torch.randn(H, F, generator=g, device=device) * weight_std)
        w2[e].copy_(c)
        w2s[e].copy_(s_)
    return dict(gate_up=w13, gate_up_scale=w13s, down=w2, down_scale=w2s)


def make_mxfp8_activations(T, H, E, k, seed, device="cpu", routing="sigmoid_topk",
                           routed_scale=2.5, zipf_s=1.2, zipf_zero=8):
    """MXFP8 hidden states (N(0,1) quantised per token and 32 block) + routing."""
    g = _gen(seed, device)
    x = torch.randn(T, H, generator=g, device=device)
    xq, xs = quantize_mxfp8_rows_torch(x)
    if routing == "sigmoid_topk":
        idx, w = route_sigmoid_topk(T, E, k, g, device, routed_scale)
    elif routing == "zipf":
        idx, w = route_zipf(T, E, k, g, device, zipf_s, zipf_zero, routed_scale)
    elif routing == "uniform_softmax":
        idx, w = route_uniform_softmax(T, E, k, g, device, routed_scale)
    else:
        raise ValueError(routing)
    return dict(x=xq, x_scale=xs, top_k_index=idx, top_k_weights=w)


def make_mxfp4_problem(T, H, F, E, k, seed, device="cpu", act_seed=None, weight_std=0.02, **kw):
    """MXFP4 weights from ``seed``, MXFP8 activations and routing from
    ``act_seed`` (or the seed + 1)."""
    p = make_mxfp4_weights(H, F, E, seed, device, weight_std=weight_std)
    p.update(make_mxfp8_activations(T, H, E, k, act_seed if act_seed is not None else seed + 1,
                                    device, **kw))
    return p


def make_shared_experts(S, H, F, seed, device="cpu", weight_std=0.02):
    """Shared-expert weights, drawn like routed ones: shared_gate_up [S,2F,H]
    and shared_down [S,H,F], bf16 N(0, std), gate_up first."""
    g = _gen(seed, "cpu")
    sg = (torch.randn(S, 2 * F, H, generator=g) * weight_std).to(torch.bfloat16)
    sd = (torch.randn(S, H, F, generator=g) * weight_std).to(torch.bfloat16)
    return dict(shared_gate_up=sg.to(device).contiguous(), shared_down=sd.to(device).contiguous())


def make_config(name, device="cpu"):
    """Problem tensors for one named workload (see CONFIGS)."""
    c = CONFIGS[name]
    if c["kind"] == "bf16":
        p = make_bf16_problem(c["T"], c["H"], c["F"], c["E"], c["k"], c["seed"], device,
                              routing=c["routing"], routed_scale=c["routed_scale"])
        if c.get("S"):
            p.update(make_shared_experts(c["S"], c["H"], c["F"], c["shared_seed"], device))
        return p
    extra = {}
    if c["routing"] == "zipf":
        extra = dict(zipf_s=c["zipf_s"], zipf_zero=c["zipf_zero"])
    if c["kind"] == "mxfp4":
        return make_mxfp4_problem(c["T"], c["H"], c["F"], c["E"], c["k"], c["seed"], device,
                                  act_seed=c.get("act_seed"), routing=c["routing"],
                                  routed_scale=c["routed_scale"], **extra)
    return make_fp8_problem(c["T"], c["H"], c["F"], c["E"], c["k"], c["seed"], device,
                            act_seed=c.get("act_seed"), routing=c["routing"],
                            routed_scale=c["routed_scale"], **extra)
