"""CPU oracle for the fused routed-experts MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers); both sides only receive the
same seeded inputs from ``moe_workloads``.

Everything is plain numpy in float64 unless a step is defined by the method in
a narrower precision (the fp8 re-quantisation of the SwiGLU output, done in
float32 exactly as the method prescribes it).  Sources, cited by page title
and section:

* [OCR2] model card "DeepSeek-OCR-2 MoE experts" (aymous/deepseek-ocr2-moe-experts):
  the description paragraph (routed experts, plain SiLU SwiGLU, router-weight
  scale and scatter-add; routing and shared experts stay outside the op) and
  the "Usage" listing (operand layouts gate_up_proj [E, 2F, H],
  down_proj [E, H, F], int32 top_k_index [T, k], fp32 top_k_weights [T, k]).
* [MPK] mirage-project/mirage issue "[Feature Request] - Supporting MegaKernel
  for DeepSeek Models", "Layer Tensor Details": moe_w13_fp8_layer and
  moe_w2_fp8_layer (fp8 E4M3 operands with one fp32 scale per 128-wide K
  block, per row), moe_silu_mul_layer (SwiGLU on [.., 2M] -> [.., M]),
  moe_local_reduction (output is the routing-weighted sum over the k slots),
  bf16_to_fp8_quantize (block-wise quantisation with block size 128).
* [GC] DeepGEMM issue "GC MoE" (its summary paragraph): routed experts with
  optional fused shared experts; FP8 activations with packed FP4 routed
  weights.

Readings of points the pages leave open (each is listed in the design doc):

1. gate_up rows [0, F) are the gate (SiLU applied), rows [F, 2F) are "up".
2. SiLU is z * sigmoid(z) with no clamp.
3. top_k_weights already carry the routed scaling factor; the op only
   multiplies by them.
4. The residual of moe_local_reduction is optional (None: no residual); when
   given it is added once, after the routing-weighted sum.
5. A token that names the same expert in two slots gets both contributions.
6. Expert ids outside [0, E) drop their slot: it contributes nothing and is
   absent from the routing plan.
7. The routing plan orders the flat slot ids s = t*k + j by expert, ties in
   ascending s; perm/inv use -1 for dropped positions.
9. The fp8 path re-quantises h per (row, 128 block) with an fp32 scale
   s = amax / 448, codes = RNE_e4m3fn(clamp(h * (448 / amax), +-448)), and an
   all-zero block gets s = 1 and zero codes.
10. FP8 is OCP E4M3FN: bias 7, max 448, codes 0x7F/0xFF are NaN, no infinity.
11. Shared experts ([GC] "optional fused shared experts"; [OCR2] keeps two
    shared experts beside the routed ones): each of the S shared experts is a
    SwiGLU expert laid out like a routed one (gate_up [S, 2Fs, H],
    down [S, H, Fs]) that every token passes through with weight 1; their
    outputs join the routing-weighted sum, before the residual.
12. MXFP4 routed weights ([GC] "packed FP4 routed weights" with FP8
    activations; DeepGEMM's FP8 x FP4 and "MXF4" kind; [MPK] ue8m0 scales per
    32 elements for FP8 GEMM inputs), read as the OCP Microscaling formats:
    E2M1 elements (sign, 2 exponent bits with bias 1, 1 mantissa bit; values
    0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte with element 2i in the low
    nibble, and one E8M0 scale 2^(s-127) (s = 255 NaN) per 32 consecutive K
    elements of a row.
13. FP8 activations of that layer, and its re-quantised SwiGLU output, are
    MXFP8: E4M3 elements with one E8M0 scale per 32 elements, the shared
    exponent floor(log2(amax)) - 8 (8 = the largest E4M3 exponent), elements
    x / 2^e clamped to +-448 and rounded to nearest even; an all-zero block
    gets s = 0 (2^-127) and zero codes.  The same rule with emax 2 and the
    E2M1 maximum 6 quantises weights to MXFP4.
14. The softmax router ([OCR2]: fp32 softmax over the E router logits, greedy
    top-k, weights scaled by routed_scaling_factor) keeps the k largest
    probabilities without renormalising them.  Softmax is increasing in the
    logit, so the choice is the k largest logits; equal logits go to the lower
    expert id.  Slots are written in the order chosen (largest first).
15. The group-aware sigmoid router ([MPK] moe_topk_sigmoid_routing_layer:
    logits + bias, num_groups, topk_group, routed_scaling_factor) is read as:
    s = sigmoid(logit); the choice score c = s + bias; the E experts form
    num_groups consecutive groups; a group's score is the sum of its
    `group_top` largest c (group_top = 2 is the DeepSeek-V3 rule the page's
    layer serves, group_top = 1 ranks a group by its best member); the
    topk_group best groups are kept (ties: lower group id); the k largest c
    among their experts are chosen (ties: lower expert id), largest first;
    their weights are the unbiased s renormalised to sum 1, times
    routed_scaling_factor.  The choice is made on float64 scores.
16. The ue8m0 variant of the block-128 quantiser ([MPK] bf16_to_fp8_quantize
    names a ue8m0 output scale without its rule) uses the smallest power of
    two 2^e with max|h| <= 448 * 2^e (e clamped to [-127, 127]), codes
    RNE_e4m3(h / 2^e), scale byte e + 127; an all-zero block gets byte 127.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py (brute force, closed forms, invariants, library
routines); none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "silu",
    "routing_plan",
    "moe_experts_reference",
    "moe_experts_reference_batched",
    "e4m3fn_decode",
    "e4m3fn_encode",
    "quantize_block128_fp32",
    "dequantize_block128",
    "moe_experts_fp8_reference",
    "moe_experts_fp8_reference_batched",
    "dequantize_block128_table",
    "quantize_block128_ue8m0",
    "e2m1_decode",
    "e2m1_encode",
    "unpack_e2m1",
    "e8m0_decode",
    "quantize_mxfp8_fp32",
    "dequantize_mx",
    "moe_experts_mxfp4_reference",
    "moe_experts_mxfp4_reference_batched",
    "dequantize_mxfp4_table",
    "route_softmax_topk",
    "route_sigmoid_group_topk",
]

# --------------------------------------------------------------------------
# SwiGLU activation ([OCR2] description: "plain SiLU"; [MPK] silu_mul layers)
# --------------------------------------------------------------------------


def silu(z):
    """SiLU(z) = z / (1 + exp(-z)) in float64 (reading 2: no clamp, no alpha)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# Routing plan (grouping implied by the grouped GEMM of [OCR2]; the [E+1]
# int32 "masks" tensor of [MPK] moe_w13/moe_w2 is the prefix over experts)
# --------------------------------------------------------------------------


def routing_plan(top_k_index, num_experts):
    """Counting sort of the flat slots s = t*k + j by expert id.

    Returns ``counts[E]``, ``offsets[E+1]`` (exclusive prefix, offsets[E] is
    the number of valid slots), ``perm[P]`` (slot ids grouped by expert,
    ascending s inside a group, -1 past offsets[E]) and ``inv[P]`` (position of
    slot s in perm, -1 for a dropped slot).  Written as two plain passes over
    the slots so that it is checkable by eye; reading 6 drops ids outside
    [0, E), reading 7 fixes the tie order.
    """
    ids = np.asarray(top_k_index).reshape(-1).astype(np.int64)
    P = ids.shape[0]
    E = int(num_experts)
    counts = np.zeros(E, dtype=np.int64)
    for s in range(P):
        e = ids[s]
        if 0 <= e < E:
            counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E].copy()
    perm = np.full(P, -1, dtype=np.int64)
    inv = np.full(P, -1, dtype=np.int64)
    for s in range(P):
        e = ids[s]
        if 0 <= e < E:
            perm[cursor[e]] = s
            inv[s] = cursor[e]
            cursor[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv.astype(np.int32))


# --------------------------------------------------------------------------
# Routers: logits -> (top_k_index, top_k_weights) ([OCR2] description: fp32
# softmax + greedy top-k scaled by routed_scaling_factor; [MPK]
# moe_topk_sigmoid_routing_layer: group-aware sigmoid routing)
# --------------------------------------------------------------------------


def _greedy_topk(score, k, allowed=None):
    """Indices of the k largest entries of one row, largest first, equal
    values in ascending index; ``allowed`` masks candidates (plain loop)."""
    E = score.shape[0]
    taken = np.zeros(E, dtype=bool)
    if allowed is not None:
        taken |= ~allowed
    out = []
    for _ in range(k):
        best = -1
        for e in range(E):
            if taken[e]:
                continue
            if best < 0 or score[e] > score[best]:
                best = e
        out.append(best)
        taken[best] = True
    return out


def route_softmax_topk(logits, k, routed_scaling_factor=1.0):
    """Softmax router (reading 14).  logits [T, E] -> idx int32 [T, k] and
    weights [T, k] float64 = softmax(logits)[idx] * routed_scaling_factor."""
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        z = lg[t] - np.max(lg[t])
        p = np.exp(z) / np.sum(np.exp(z))
        ch = _greedy_topk(lg[t], k)
        idx[t] = ch
        w[t] = p[ch] * routed_scaling_factor
    return idx, w


def route_sigmoid_group_topk(logits, bias, k, num_groups, topk_group, routed_scaling_factor=1.0,
                             group_top=2):
    """Group-aware sigmoid router (reading 15).  logits [T, E], bias [E] ->
    idx int32 [T, k], weights float64 [T, k]."""
    lg = np.asarray(logits, dtype=np.float64)
    b = np.asarray(bias, dtype=np.float64).reshape(-1)
    T, E = lg.shape
    if E % num_groups or not 1 <= topk_group <= num_groups:
        raise ValueError("E must split into num_groups groups, 1 <= topk_group <= num_groups")
    gsize = E // num_groups
    if not 1 <= group_top <= gsize or not 1 <= k <= topk_group * gsize:
        raise ValueError("group_top or k out of range")
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        s = 1.0 / (1.0 + np.exp(-lg[t]))
        c = s + b
        gscore = np.zeros(num_groups)
        for g in range(num_groups):
            members = c[g * gsize:(g + 1) * gsize]
            gscore[g] = sum(members[j] for j in _greedy_topk(members, group_top))
        kept = _greedy_topk(gscore, topk_group)
        allowed = np.zeros(E, dtype=bool)
        for g in kept:
            allowed[g * gsize:(g + 1) * gsize] = True
        ch = _greedy_topk(c, k, allowed)
        idx[t] = ch
        w[t] = s[ch] / np.sum(s[ch]) * routed_scaling_factor
    return idx, w


# --------------------------------------------------------------------------
# bf16 layer ([OCR2] description and "Usage"; combine as [MPK]
# moe_local_reduction, its residual optional)
# --------------------------------------------------------------------------


def _as_f64(a):
    return np.asarray(a, dtype=np.float64)


def _swiglu_expert(w13_e, w2_e, xt):
    """One expert on one token: down @ (silu(gate @ x) * (up @ x))."""
    g = _as_f64(w13_e) @ xt
    F = g.shape[0] // 2
    h = silu(g[:F]) * g[F:]
    return _as_f64(w2_e) @ h


def moe_experts_reference(hidden, gate_up, down, top_k_index, top_k_weights, residual=None,
                          shared_gate_up=None, shared_down=None):
    """Routed-experts layer, one token and one slot at a time, in float64.

    hidden [T, H], gate_up [E, 2F, H], down [E, H, F] are the operands' values
    (bf16 inputs upcast exactly); top_k_index int [T, k]; top_k_weights [T, k].
    For every token t and slot j with a valid expert e:
        g   = gate_up[e] @ x[t]               (2F values)
        h   = silu(g[:F]) * g[F:]             (F values)
        y   = down[e] @ h                     (H values)
        out[t] += w[t, j] * y
    then, for every shared expert s (reading 11), out[t] += the same SwiGLU
    expert of shared_gate_up[s], shared_down[s] with weight 1, and finally
    out += residual [T, H] when one is given ([MPK] moe_local_reduction).
    """
    x = _as_f64(hidden)
    w13 = np.asarray(gate_up)
    w2 = np.asarray(down)
    idx = np.asarray(top_k_index)
    wts = _as_f64(top_k_weights)
    T, H = x.shape
    E, F2, _ = w13.shape
    F = F2 // 2
    k = idx.shape[1]
    out = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if not 0 <= e < E:
                continue
            g = _as_f64(w13[e]) @ x[t]
            h = silu(g[:F]) * g[F:]
            y = _as_f64(w2[e]) @ h
            out[t] += wts[t, j] * y
    if shared_gate_up is not None:
        sg, sd = np.asarray(shared_gate_up), np.asarray(shared_down)
        for t in range(T):
            for s_ in range(sg.shape[0]):
                out[t] += _swiglu_expert(sg[s_], sd[s_], x[t])
    if residual is not None:
        out += _as_f64(residual)
    return out


def moe_experts_reference_batched(hidden, gate_up, down, top_k_index, top_k_weights,
                                  residual=None, shared_gate_up=None, shared_down=None):
    """Same sums as :func:`moe_experts_reference`, grouped by expert.

    Each expert's rows are gathered once and multiplied as one float64 matrix
    product, so a large layer does not re-read the expert weights per slot.
    Only the summation order inside the dot products differs from the
    per-slot form.
    """
    x = _as_f64(hidden)
    w13 = np.asarray(gate_up)
    w2 = np.asarray(down)
    idx = np.asarray(top_k_index)
    wts = _as_f64(top_k_weights)
    T, H = x.shape
    E, F2, _ = w13.shape
    F = F2 // 2
    out = np.zeros((T, H), dtype=np.float64)
    for e in range(E):
        tt, jj = np.nonzero(idx == e)
        if tt.size == 0:
            continue
        g = x[tt] @ _as_f64(w13[e]).T
        h = silu(g[:, :F]) * g[:, F:]
        y = h @ _as_f64(w2[e]).T
        contrib = wts[tt, jj][:, None] * y
        np.add.at(out, tt, contrib)
    if shared_gate_up is not None:
        sg, sd = np.asarray(shared_gate_up), np.asarray(shared_down)
        for s_ in range(sg.shape[0]):
            g = x @ _as_f64(sg[s_]).T
            Fs = g.shape[1] // 2
            out += (silu(g[:, :Fs]) * g[:, Fs:]) @ _as_f64(sd[s_]).T
    if residual is not None:
        out += _as_f64(residual)
    return out


# --------------------------------------------------------------------------
# FP8 E4M3FN codec (reading 10; [MPK] moe_w13_fp8_layer dtypes "FP8 E4M3")
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3fn_decode(codes):
    """Exact value of each OCP E4M3FN byte as float64.

    sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
    exponent 0: (-1)^s * 2^-6 * m/8; otherwise (-1)^s * 2^(e-7) * (1 + m/8);
    exponent 15 with mantissa 7 is NaN (no infinities).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def e4m3fn_encode(v):
    """Round-to-nearest-even encoding of finite values with |v| <= 448.

    Callers clamp first (reading 9).  Subnormal range |v| < 2^-6 is a multiple
    of 2^-9; normal range keeps 3 mantissa bits.  A mantissa that rounds up to
    8 carries into the exponent, which the integer code arithmetic does by
    itself (code = (exp+7)*8 + m).
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("e4m3fn_encode expects finite values within +-448")
    neg = np.signbit(np.asarray(v, dtype=np.float64))
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormals: magnitude in units of 2^-9, rounded half to even
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), code)
    # normals: a = 2^E * f with f in [1, 2)
    safe = np.where(sub, 1.0, a)
    mant, exp2 = np.frexp(safe)          # safe = mant * 2^exp2, mant in [0.5, 1)
    E = exp2 - 1                          # so safe = (2*mant) * 2^E
    q = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)   # 0..8
    ncode = (E + 7) * 8 + q
    code = np.where(sub, code, ncode)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def quantize_block128_fp32(h):
    """Block-128 fp8 quantisation of the rows of ``h`` done in float32.

    [MPK] bf16_to_fp8_quantize gives block size 128; the scale dtype follows
    moe_w2_fp8_layer's fp32 input_scale (reading 9).  For each row and each
    128-column block, all in float32 arithmetic:
        a = max |h|,  s = a / 448,  v = clamp(h * (448 / a), -448, 448),
        code = RNE_e4m3fn(v);  a == 0 gives s = 1 and zero codes.
    Returns (codes uint8 [.., K], scales float32 [.., K/128]).
    """
    hb = np.asarray(h, dtype=np.float32)
    K = hb.shape[-1]
    if K % 128:
        raise ValueError("last dimension must be a multiple of 128")
    blocks = hb.reshape(hb.shape[:-1] + (K // 128, 128))
    amax = np.max(np.abs(blocks), axis=-1)                      # float32, exact
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), safe / np.float32(E4M3_MAX)).astype(np.float32)
    recip = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    v = (blocks * recip[..., None]).astype(np.float32)          # fp32 multiply
    v = np.clip(v, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    v = np.where(zero[..., None], np.float32(0.0), v)
    codes = e4m3fn_encode(v).reshape(hb.shape)
    return codes, scale.astype(np.float32)


def quantize_block128_ue8m0(h):
    """Block-128 fp8 quantisation with a power-of-two (ue8m0) scale per block
    ([MPK] bf16_to_fp8_quantize: "FP8 E4M3 + scale ue8m0", block size 128,
    output_scale [..., K/128]).  The page gives no rule; reading 16: for each
    row and 128-column block of the float32 values, e is the smallest integer
    with max|h| <= 448 * 2^e (clamped to [-127, 127]), codes =
    RNE_e4m3fn(clamp(h / 2^e, +-448)) and the scale byte is e + 127 (its
    value 2^e).  An all-zero block gets byte 127 (scale 1, as the fp32 rule
    gives a zero block s = 1) and zero codes.  h / 2^e is exact, so the only
    rounding is the e4m3 one.
    Returns (codes uint8 [.., K], scale bytes uint8 [.., K/128])."""
    hb = np.asarray(h, dtype=np.float32)
    K = hb.shape[-1]
    if K % 128:
        raise ValueError("last dimension must be a multiple of 128")
    blocks = hb.reshape(hb.shape[:-1] + (K // 128, 128)).astype(np.float64)
    amax = np.max(np.abs(blocks), axis=-1)
    e = np.zeros(amax.shape, dtype=np.int64)
    flat_a, flat_e = amax.reshape(-1), e.reshape(-1)
    for i in range(flat_a.size):
        a = flat_a[i]
        if a == 0.0:
            flat_e[i] = 0
            continue
        ei = int(np.ceil(np.log2(a / E4M3_MAX)))       # estimate, then made exact:
        while E4M3_MAX * 2.0 ** ei < a:
            ei += 1
        while E4M3_MAX * 2.0 ** (ei - 1) >= a:
            ei -= 1
        flat_e[i] = min(max(ei, -127), 127)
    e = flat_e.reshape(amax.shape)
    v = blocks / np.exp2(e.astype(np.float64))[..., None]
    v = np.clip(v, -E4M3_MAX, E4M3_MAX)
    codes = e4m3fn_encode(v).reshape(hb.shape)
    return codes, (e + 127).astype(np.uint8)


def dequantize_block128(codes, scales):
    """value = decode(code) * scale[..., col // 128] in float64."""
    vals = e4m3fn_decode(codes)
    K = vals.shape[-1]
    s = np.repeat(np.asarray(scales, dtype=np.float64), 128, axis=-1)[..., :K]
    return vals * s


# --------------------------------------------------------------------------
# FP8 block-scaled layer ([MPK] moe_w13_fp8_layer, moe_silu_mul_layer,
# moe_w2_fp8_layer, moe_local_reduction)
# --------------------------------------------------------------------------


def moe_experts_fp8_reference(x_codes, x_scale, w13_codes, w13_scale,
                              w2_codes, w2_scale, top_k_index, top_k_weights,
                              tokens=None, residual=None):
    """FP8 routed-experts layer in float64 with the method's fp32 re-quantise.

    Operands: x_codes [T, H] + x_scale [T, H/128]; w13_codes [E, 2F, H] +
    w13_scale [E, 2F, H/128]; w2_codes [E, H, F] + w2_scale [E, H, F/128].
    Every operand is dequantised exactly (code value times its block scale).
    Per slot (t, j) with valid expert e:
        g  = W13[e] @ x[t];  h = silu(g[:F]) * g[F:]                (float64)
        (q, s) = quantize_block128_fp32(float32(h));  h~ = decode(q) * s
        y  = W2[e] @ h~;  out[t] += w[t, j] * y
    The loop runs expert by expert so each expert is dequantised once; within
    an expert each slot is its own matrix-vector product.  ``tokens``
    restricts the result to a subset of rows (others stay zero), which is how
    a sampled check of a large layer is made.  ``residual`` [T, H], when
    given, is added after the weighted sum (on the selected rows).
    Returns out [T, H] float64 (and nothing is rounded to bf16).
    """
    xq = np.asarray(x_codes)
    T, H = xq.shape
    idx = np.asarray(top_k_index)
    wts = np.asarray(top_k_weights, dtype=np.float64)
    E = w13_codes.shape[0]
    F = w13_codes.shape[1] // 2
    want = np.zeros(T, dtype=bool)
    if tokens is None:
        want[:] = True
    else:
        want[np.asarray(tokens)] = True
    x = dequantize_block128(xq, x_scale)
    out = np.zeros((T, H), dtype=np.float64)
    for e in range(E):
        tt, jj = np.nonzero((idx == e) & want[:, None])
        if tt.size == 0:
            continue
        W13 = dequantize_block128(np.asarray(w13_codes[e]), np.asarray(w13_scale[e]))
        W2 = dequantize_block128(np.asarray(w2_codes[e]), np.asarray(w2_scale[e]))
        for t, j in zip(tt.tolist(), jj.tolist()):
            g = W13 @ x[t]
            h = silu(g[:F]) * g[F:]
            q, s = quantize_block128_fp32(h.astype(np.float32))
            ht = dequantize_block128(q, s)
            y = W2 @ ht
            out[t] += wts[t, j] * y
    if residual is not None:
        out[want] += np.asarray(residual, dtype=np.float64)[want]
    return out


def dequantize_block128_table(codes, scales):
    """Same values as :func:`dequantize_block128`, computed faster for whole
    expert matrices: each of the 256 codes is decoded once by
    :func:`e4m3fn_decode` and looked up, and every 128-wide block is scaled
    through a reshape instead of a repeated scale array."""
    table = e4m3fn_decode(np.arange(256, dtype=np.uint8))
    c = np.asarray(codes, dtype=np.uint8)
    K = c.shape[-1]
    vals = table[c].reshape(c.shape[:-1] + (K // 128, 128))
    return (vals * np.asarray(scales, dtype=np.float64)[..., None]).reshape(c.shape)


def _fp8_expert_rows(xrows, W13, W2, F):
    """The fp8 layer's expert on a batch of rows: one float64 product per
    matrix, h re-quantised row by row in float32 (reading 9).  Returns
    (y, h in float32, codes, scales)."""
    g = xrows @ W13.T
    h = silu(g[:, :F]) * g[:, F:]
    h32 = h.astype(np.float32)
    q, s = quantize_block128_fp32(h32)
    return dequantize_block128(q, s) @ W2.T, h32, q, s


def moe_experts_fp8_reference_batched(x_codes, x_scale, w13_codes, w13_scale,
                                      w2_codes, w2_scale, top_k_index, top_k_weights,
                                      tokens=None, residual=None, h_report=None):
    """Same sums as :func:`moe_experts_fp8_reference`, grouped by expert.

    Per expert the weights are dequantised once and the rows of every slot
    that chose it are multiplied as one float64 matrix product; h is
    re-quantised per (row, 128 block) in float32 exactly as in the per-slot
    form.  Only the summation order inside the dot products differs (about
    1e-16 relative), which lets the full DeepSeek-V3-shaped layers be checked
    on every output row.  ``tokens`` and ``residual`` as in the per-slot form.
    ``h_report``, a dict, receives the intermediate of every computed slot
    s = t*k + j (rows of dropped or unselected slots stay zero): "h" the
    float32 SwiGLU output [P, F], "codes" its block-128 codes [P, F] and
    "scales" [P, F/128].
    """
    xq = np.asarray(x_codes)
    T, H = xq.shape
    idx = np.asarray(top_k_index)
    wts = np.asarray(top_k_weights, dtype=np.float64)
    E = w13_codes.shape[0]
    F = w13_codes.shape[1] // 2
    want = np.zeros(T, dtype=bool)
    if tokens is None:
        want[:] = True
    else:
        want[np.asarray(tokens)] = True
    x = dequantize_block128_table(xq, x_scale)
    out = np.zeros((T, H), dtype=np.float64)
    k = idx.shape[1]
    if h_report is not None:
        h_report["h"] = np.zeros((T * k, F), np.float32)
        h_report["codes"] = np.zeros((T * k, F), np.uint8)
        h_report["scales"] = np.zeros((T * k, F // 128), np.float32)
    for e in range(E):
        tt, jj = np.nonzero((idx == e) & want[:, None])
        if tt.size == 0:
            continue
        W13 = dequantize_block128_table(np.asarray(w13_codes[e]), np.asarray(w13_scale[e]))
        W2 = dequantize_block128_table(np.asarray(w2_codes[e]), np.asarray(w2_scale[e]))
        y, h32, q, sc = _fp8_expert_rows(x[tt], W13, W2, F)
        np.add.at(out, tt, wts[tt, jj][:, None] * y)
        if h_report is not None:
            rows = tt * k + jj
            h_report["h"][rows], h_report["codes"][rows], h_report["scales"][rows] = h32, q, sc
    if residual is not None:
        out[want] += np.asarray(residual, dtype=np.float64)[want]
    return out


def moe_experts_fp8_bf16_reference(hidden, w13_codes, w13_scale, w2_codes, w2_scale,
                                   top_k_index, top_k_weights, tokens=None, residual=None):
    """FP8 layer fed with bf16 hidden states ([MPK] bf16_to_fp8_quantize before
    moe_w13_fp8_layer): the rows of ``hidden`` (values of bf16 numbers) are
    quantised per 128-wide block by :func:`quantize_block128_fp32` (the same
    fp32 rule as the re-quantisation of h), then the fp8 layer runs on those
    codes and scales."""
    xq, xs = quantize_block128_fp32(np.asarray(hidden, dtype=np.float32))
    return moe_experts_fp8_reference(xq, xs, w13_codes, w13_scale, w2_codes, w2_scale,
                                     top_k_index, top_k_weights, tokens=tokens, residual=residual)


# --------------------------------------------------------------------------
# Microscaling formats (readings 12-13): E2M1 and E4M3 elements, E8M0 scales
# per 32 elements
# --------------------------------------------------------------------------

MX_BLOCK = 32
E2M1_MAX = 6.0


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code (0..15) as float64: sign bit 3, exponent
    bits 2..1 (bias 1), mantissa bit 0; exponent 0 is 0.5 * m (subnormal),
    otherwise 2^(e-1) * (1 + m/2).  No NaN or infinity."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 1).astype(np.float64)
    v = np.where(e == 0, 0.5 * m, np.exp2(e.astype(np.float64) - 1.0) * (1.0 + 0.5 * m))
    return sign * v


def e2m1_encode(v):
    """Round-to-nearest-even E2M1 codes of finite values with |v| <= 6.

    The representable magnitudes are the multiples of 0.5 up to 2 (exponents
    0 and 1), of 1 up to 4 (exponent 2) and of 2 up to 6 (exponent 3); a tie
    goes to the neighbour whose mantissa bit is 0.
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    if np.any(~np.isfinite(a)) or np.any(a > E2M1_MAX):
        raise ValueError("e2m1_encode expects finite values within +-6")
    neg = np.signbit(np.asarray(v, dtype=np.float64))
    # step of the binade the value falls in: 0.5 below 2, 1 below 4, 2 above
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.rint(a / step) * step                     # half-to-even on the step grid
    # rint's "even" is even in units of the step, i.e. mantissa bit 0, except
    # at the binade tops 2 and 4 (reached from below), which are exact codes
    mag = np.minimum(q, E2M1_MAX)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    code = np.searchsorted(grid, mag)
    if not np.all(grid[code] == mag):
        raise AssertionError("E2M1 rounding left the grid")
    return (code | np.where(neg, 8, 0)).astype(np.uint8)


def unpack_e2m1(packed):
    """Bytes [..., K/2] -> 4-bit codes [..., K]; element 2i is the low nibble."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def e8m0_decode(s):
    """2^(s - 127) as float64; s = 255 is NaN."""
    s = np.asarray(s).astype(np.int64)
    return np.where(s == 255, np.nan, np.exp2(s.astype(np.float64) - 127.0))


def _mx_shared_exponent(amax, emax_elem):
    """floor(log2(amax)) - emax_elem, clamped to [-127, 127]; amax 0 gives -127.
    amax is a float32 array; frexp gives amax = m * 2^E with m in [0.5, 1), so
    floor(log2(amax)) = E - 1 exactly."""
    a = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = (E - 1) - emax_elem
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_mxfp8_fp32(h):
    """MXFP8 quantisation of the rows of ``h`` (reading 13), in float32:
    per 32-column block, e = floor(log2(max|h|)) - 8, codes =
    RNE_e4m3(clamp(h / 2^e, +-448)), scale byte e + 127; a zero block gets
    byte 0 and zero codes.  Returns (codes uint8 [.., K], scales uint8 [.., K/32])."""
    hb = np.asarray(h, dtype=np.float32)
    K = hb.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("last dimension must be a multiple of 32")
    blocks = hb.reshape(hb.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    e = _mx_shared_exponent(amax, 8)
    # division by a power of two: exact in float64, then held in float32
    v = (blocks.astype(np.float64) / np.exp2(e.astype(np.float64))[..., None]).astype(np.float32)
    v = np.clip(v, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = e4m3fn_encode(v).reshape(hb.shape)
    return codes, (e + 127).astype(np.uint8)


def dequantize_mx(values, scales):
    """Element values times 2^(s-127) of their 32-element block, float64."""
    vals = np.asarray(values, dtype=np.float64)
    K = vals.shape[-1]
    s = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=-1)[..., :K]
    return vals * s


def moe_experts_mxfp4_reference(x_codes, x_scale, w13_packed, w13_scale, w2_packed, w2_scale,
                                top_k_index, top_k_weights, tokens=None, residual=None):
    """Routed-experts layer with MXFP4 weights and MXFP8 activations, float64,
    with the method's fp32 MXFP8 re-quantisation of h (readings 12-13).

    Operands: x_codes [T, H] E4M3 + x_scale [T, H/32] E8M0; w13_packed
    [E, 2F, H/2] E2M1 pairs + w13_scale [E, 2F, H/32]; w2_packed [E, H, F/2] +
    w2_scale [E, H, F/32].  Per slot (t, j) with valid expert e:
        g = W13[e] @ x[t];  h = silu(g[:F]) * g[F:]
        (q, s) = quantize_mxfp8_fp32(float32(h));  h~ = e4m3(q) * 2^(s-127)
        y = W2[e] @ h~;  out[t] += w[t, j] * y
    then + residual.  ``tokens`` restricts the rows computed (others zero).
    """
    xq = np.asarray(x_codes)
    T, H = xq.shape
    idx = np.asarray(top_k_index)
    wts = np.asarray(top_k_weights, dtype=np.float64)
    E = w13_packed.shape[0]
    F = w13_packed.shape[1] // 2
    want = np.zeros(T, dtype=bool)
    if tokens is None:
        want[:] = True
    else:
        want[np.asarray(tokens)] = True
    x = dequantize_mx(e4m3fn_decode(xq), x_scale)
    out = np.zeros((T, H), dtype=np.float64)
    for e in range(E):
        tt, jj = np.nonzero((idx == e) & want[:, None])
        if tt.size == 0:
            continue
        W13 = dequantize_mx(e2m1_decode(unpack_e2m1(w13_packed[e])), np.asarray(w13_scale[e]))
        W2 = dequantize_mx(e2m1_decode(unpack_e2m1(w2_packed[e])), np.asarray(w2_scale[e]))
        for t, j in zip(tt.tolist(), jj.tolist()):
            g = W13 @ x[t]
            h = silu(g[:F]) * g[F:]
            q, sc = quantize_mxfp8_fp32(h.astype(np.float32))
            ht = dequantize_mx(e4m3fn_decode(q), sc)
            y = W2 @ ht
            out[t] += wts[t, j] * y
    if residual is not None:
        out[want] += np.asarray(residual, dtype=np.float64)[want]
    return out


def dequantize_mxfp4_table(packed, scales):
    """MXFP4 weights as float64: the value of both nibbles of each of the 256
    byte values is taken once from :func:`e2m1_decode` (element 2i in the low
    nibble, as :func:`unpack_e2m1`), and each 32-element block is scaled by
    :func:`e8m0_decode` of its scale byte.  Same values as
    ``dequantize_mx(e2m1_decode(unpack_e2m1(packed)), scales)``."""
    b = np.arange(256, dtype=np.uint8)
    pair = np.stack([e2m1_decode(b & 0xF), e2m1_decode(b >> 4)], axis=-1)   # [256, 2]
    p = np.asarray(packed, dtype=np.uint8)
    K = 2 * p.shape[-1]
    vals = pair[p].reshape(p.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    return (vals * e8m0_decode(scales)[..., None]).reshape(p.shape[:-1] + (K,))


def moe_experts_mxfp4_reference_batched(x_codes, x_scale, w13_packed, w13_scale, w2_packed,
                                        w2_scale, top_k_index, top_k_weights, tokens=None,
                                        residual=None, h_report=None):
    """Same sums as :func:`moe_experts_mxfp4_reference`, grouped by expert:
    per expert the weights are dequantised once, the rows of its slots go
    through one float64 product per matrix, and h is re-quantised to MXFP8
    row by row in float32 (reading 13).  Only the summation order inside the
    dot products differs from the per-slot form.  ``h_report`` as in
    :func:`moe_experts_fp8_reference_batched` ("scales" are the E8M0 bytes
    [P, F/32])."""
    xq = np.asarray(x_codes)
    T, H = xq.shape
    idx = np.asarray(top_k_index)
    wts = np.asarray(top_k_weights, dtype=np.float64)
    E = w13_packed.shape[0]
    F = w13_packed.shape[1] // 2
    want = np.zeros(T, dtype=bool)
    if tokens is None:
        want[:] = True
    else:
        want[np.asarray(tokens)] = True
    x = dequantize_mx(e4m3fn_decode(xq), x_scale)
    out = np.zeros((T, H), dtype=np.float64)
    k = idx.shape[1]
    if h_report is not None:
        h_report["h"] = np.zeros((T * k, F), np.float32)
        h_report["codes"] = np.zeros((T * k, F), np.uint8)
        h_report["scales"] = np.zeros((T * k, F // MX_BLOCK), np.uint8)
    for e in range(E):
        tt, jj = np.nonzero((idx == e) & want[:, None])
        if tt.size == 0:
            continue
        W13 = dequantize_mxfp4_table(np.asarray(w13_packed[e]), np.asarray(w13_scale[e]))
        W2 = dequantize_mxfp4_table(np.asarray(w2_packed[e]), np.asarray(w2_scale[e]))
        g = x[tt] @ W13.T
        h = silu(g[:, :F]) * g[:, F:]
        h32 = h.astype(np.float32)
        q, sc = quantize_mxfp8_fp32(h32)
        y = dequantize_mx(e4m3fn_decode(q), sc) @ W2.T
        np.add.at(out, tt, wts[tt, jj][:, None] * y)
        if h_report is not None:
            rows = tt * k + jj
            h_report["h"][rows], h_report["codes"][rows], h_report["scales"][rows] = h32, q, sc
    if residual is not None:
        out[want] += np.asarray(residual, dtype=np.float64)[want]
    return out
