"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a library routine, a brute
force evaluation written differently, or an invariant of the mathematics, so
that a plausible slip in the oracle (a swapped gate/up, a dropped term, a
wrong scale index, a transposed operand, a wrong tie order) fails one of them.
No GPU is needed.
"""

import itertools

import numpy as np
import pytest
import scipy.special
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import moe_workloads as wl
from oracle import moe_oracle as orc


def _problem(T, H, F, E, k, seed, std=0.3, distinct=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    w13 = rng.standard_normal((E, 2 * F, H)) * std
    w2 = rng.standard_normal((E, H, F)) * std
    if distinct:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    else:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w = rng.random((T, k))
    return x, w13, w2, idx, w


def _dense_bruteforce(x, w13, w2, idx, w):
    """Every expert on every token (einsum over the full tensors, sigmoid from
    scipy), then a mask matrix M[t, e] = sum_j w[t, j] [idx[t, j] == e]."""
    T, H = x.shape
    E, F2, _ = w13.shape
    F = F2 // 2
    G = np.einsum("th,enh->ten", x, w13)                      # [T, E, 2F]
    gate, up = G[..., :F], G[..., F:]
    Hh = gate * scipy.special.expit(gate) * up                # [T, E, F]
    Y = np.einsum("tef,ecf->tec", Hh, w2)                     # [T, E, H]
    M = np.zeros((T, E))
    for t in range(T):
        for j in range(idx.shape[1]):
            if 0 <= idx[t, j] < E:
                M[t, idx[t, j]] += w[t, j]
    return np.einsum("te,tec->tc", M, Y)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ----------------------------------------------------------------- SiLU


def test_silu_matches_library_sigmoid():
    z = np.linspace(-40, 40, 2001)
    ref = z * scipy.special.expit(z)
    np.testing.assert_allclose(orc.silu(z), ref, rtol=1e-14, atol=1e-300)


def test_silu_closed_values(golden):
    assert orc.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert orc.silu(0.0) == 0.0
    assert orc.silu(-800.0) == 0.0   # no overflow trap at large negative arguments


# --------------------------------------------------------- routing plan


def _plan_by_library(ids, E):
    ids = np.asarray(ids).reshape(-1).astype(np.int64)
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    key = np.where(valid, ids, E)                     # dropped slots sort last
    order = np.argsort(key, kind="stable")[: int(valid.sum())]
    perm = np.full(ids.size, -1)
    perm[: order.size] = order
    inv = np.full(ids.size, -1)
    inv[order] = np.arange(order.size)
    return counts, offsets, perm, inv


@pytest.mark.parametrize("name", ["tiny", "ocr2_decode_t4", "ocr2_prefill"])
def test_plan_matches_library_sort(name):
    c = wl.CONFIGS[name]
    g = wl._gen(c["seed"], "cpu")
    idx, _ = wl.route_uniform_softmax(c["T"], c["E"], c["k"], g)
    got = orc.routing_plan(idx.numpy(), c["E"])
    ref = _plan_by_library(idx.numpy(), c["E"])
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)


def test_plan_zipf_with_empty_experts():
    idx, _ = wl.route_zipf(4096, 128, 8, wl._gen(1005, "cpu"))
    counts, offsets, perm, inv = orc.routing_plan(idx.numpy(), 128)
    assert (counts == 0).sum() == 8
    for a, b in zip((counts, offsets, perm, inv), _plan_by_library(idx.numpy(), 128)):
        np.testing.assert_array_equal(a, b)


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 40), st.integers(1, 9), st.integers(1, 12), st.integers(0, 2**31 - 1))
def test_plan_properties(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)     # includes dropped ids
    counts, offsets, perm, inv = orc.routing_plan(ids, E)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    n = int(valid.sum())
    assert counts.sum() == n and offsets[-1] == n and offsets[0] == 0
    assert np.all(perm[n:] == -1)
    assert np.all(inv[~valid] == -1)
    p = perm[:n]
    assert np.all(inv[p] == np.arange(n))                 # inv is perm's inverse
    ex = flat[p]
    assert np.all(np.diff(ex) >= 0)                        # grouped by expert
    for e in range(E):
        seg = p[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)                   # ties by ascending slot id
    for a, b in zip((counts, offsets, perm, inv), _plan_by_library(ids, E)):
        np.testing.assert_array_equal(a, b)


def test_plan_empty_and_all_dropped():
    counts, offsets, perm, inv = orc.routing_plan(np.zeros((0, 3), np.int32), 4)
    assert counts.tolist() == [0] * 4 and offsets.tolist() == [0] * 5 and perm.size == 0
    counts, offsets, perm, inv = orc.routing_plan(np.full((3, 2), -1, np.int32), 4)
    assert offsets[-1] == 0 and np.all(perm == -1) and np.all(inv == -1)


# ------------------------------------------------------------ bf16 layer


def test_closed_form_gate_up_order(golden):
    c = golden["swiglu_h1_f1"]
    out = orc.moe_experts_reference(np.array([c["x"]]), np.array(c["gate_up"]), np.array(c["down"]),
                                    np.array(c["top_k_index"]), np.array(c["top_k_weights"]))
    assert out[0, 0] == pytest.approx(c["out"][0][0], rel=1e-15)
    assert abs(out[0, 0] - c["out_if_gate_up_swapped"][0][0]) > 0.2


def test_closed_form_weighted_slots(golden):
    c = golden["two_slots_weighted"]
    for fn in (orc.moe_experts_reference, orc.moe_experts_reference_batched):
        out = fn(np.array([c["x"]]), np.array(c["gate_up"]), np.array(c["down"]),
                 np.array(c["top_k_index"]), np.array(c["top_k_weights"]))
        assert out[0, 0] == pytest.approx(c["out"][0][0], rel=1e-14)


def test_single_expert_is_dense_swiglu_mlp():
    """E=1, k=1, w=1 is the textbook W2 (silu(Wg x) * (Wu x)) for every token."""
    x, w13, w2, _, _ = _problem(7, 24, 10, 1, 1, seed=3)
    idx = np.zeros((7, 1), np.int32)
    w = np.ones((7, 1))
    Wg, Wu = w13[0, :10], w13[0, 10:]
    a = x @ Wg.T
    ref = (a * scipy.special.expit(a) * (x @ Wu.T)) @ w2[0].T
    out = orc.moe_experts_reference(x, w13, w2, idx, w)
    assert _rel(out, ref) < 1e-13


@pytest.mark.parametrize("shape,seed", [((5, 16, 8, 4, 2), 1), ((9, 12, 6, 7, 3), 2),
                                        ((6, 8, 4, 5, 5), 3), ((4, 10, 6, 3, 3), 4)])
def test_oracle_vs_dense_bruteforce(shape, seed):
    x, w13, w2, idx, w = _problem(*shape, seed=seed, distinct=(seed % 2 == 1))
    ref = _dense_bruteforce(x, w13, w2, idx, w)
    assert _rel(orc.moe_experts_reference(x, w13, w2, idx, w), ref) < 1e-12
    assert _rel(orc.moe_experts_reference_batched(x, w13, w2, idx, w), ref) < 1e-12


def test_oracle_vs_bruteforce_on_tiny_config():
    p = wl.make_config("tiny")
    x = p["hidden"].float().numpy().astype(np.float64)
    w13 = p["gate_up"].float().numpy().astype(np.float64)
    w2 = p["down"].float().numpy().astype(np.float64)
    idx = p["top_k_index"].numpy()
    w = p["top_k_weights"].numpy().astype(np.float64)
    ref = _dense_bruteforce(x, w13, w2, idx, w)
    assert _rel(orc.moe_experts_reference(x, w13, w2, idx, w), ref) < 1e-12
    assert _rel(orc.moe_experts_reference_batched(x, w13, w2, idx, w), ref) < 1e-12


def test_invariants():
    x, w13, w2, idx, w = _problem(6, 16, 8, 6, 3, seed=11)
    f = orc.moe_experts_reference
    base = f(x, w13, w2, idx, w)
    # zero routing weights give exactly zero
    assert np.all(f(x, w13, w2, idx, np.zeros_like(w)) == 0.0)
    # linear in the routing weights
    w_b = np.random.default_rng(5).random(w.shape)
    lin = f(x, w13, w2, idx, 0.7 * w - 1.3 * w_b)
    assert _rel(lin, 0.7 * base - 1.3 * f(x, w13, w2, idx, w_b)) < 1e-12
    # permuting the k slots of each token changes nothing
    for perm in itertools.permutations(range(3)):
        assert _rel(f(x, w13, w2, idx[:, perm], w[:, perm]), base) < 1e-12
    # permuting tokens permutes outputs
    tp = np.random.default_rng(6).permutation(6)
    assert _rel(f(x[tp], w13, w2, idx[tp], w[tp]), base[tp]) < 1e-12
    # a duplicated expert in two slots equals one slot with the summed weight
    idx_d = idx.copy(); idx_d[:, 1] = idx_d[:, 0]
    w_m = w.copy(); w_m[:, 0] += w_m[:, 1]; w_m[:, 1] = 0.0
    assert _rel(f(x, w13, w2, idx_d, w), f(x, w13, w2, idx_d, w_m)) < 1e-12
    # appending an expert nobody routes to changes nothing
    w13x = np.concatenate([w13, np.ones_like(w13[:1])]); w2x = np.concatenate([w2, np.ones_like(w2[:1])])
    assert np.array_equal(f(x, w13x, w2x, idx, w), base)
    # an out-of-range id drops its slot
    idx_bad = idx.copy(); idx_bad[:, 2] = -1
    w_z = w.copy(); w_z[:, 2] = 0.0
    assert _rel(f(x, w13, w2, idx_bad, w), f(x, w13, w2, idx, w_z)) < 1e-12


# ------------------------------------------------------------ fp8 codec


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = orc.e4m3fn_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_golden_codes(golden):
    c = golden["e4m3fn_codes"]
    got = orc.e4m3fn_decode(np.array(c["codes"], np.uint8))
    assert got.tolist() == c["values"]
    assert np.all(np.isnan(orc.e4m3fn_decode(np.array(c["nan_codes"], np.uint8))))
    assert orc.e4m3fn_encode(np.array(c["values"])).tolist() == c["codes"]


def test_e4m3_encode_sweep_vs_torch():
    rng = np.random.default_rng(0)
    finite = orc.e4m3fn_decode(np.arange(256, dtype=np.uint8))
    finite = np.unique(finite[np.isfinite(finite)])
    mids = (finite[:-1] + finite[1:]) / 2                      # exact ties
    vals = np.concatenate([
        finite, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 1e-2,
        rng.standard_normal(20000) * 2.0 ** -8, [2.0 ** -10, -2.0 ** -10, 2.0 ** -11, 0.0, -0.0],
    ]).astype(np.float32)
    vals = np.clip(vals, -448, 448)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3fn_encode(vals)
    assert np.array_equal(got, ref)


def test_e4m3_roundtrip_every_code():
    codes = np.arange(256, dtype=np.uint8)
    v = orc.e4m3fn_decode(codes)
    ok = np.isfinite(v)
    assert np.array_equal(orc.e4m3fn_encode(v[ok]), codes[ok])


def test_e4m3_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        orc.e4m3fn_encode(np.array([449.0]))


def test_block_requant_golden(golden):
    c = golden["block128_requant"]
    h = np.zeros(128, np.float32); h[:4] = c["h_first4"]
    q, s = orc.quantize_block128_fp32(h[None, :])
    assert q[0, :4].tolist() == c["codes_first4"] and np.all(q[0, 4:] == 0)
    assert float(s[0, 0]) == c["scale"]


def test_block_requant_matches_torch_recipe():
    """Same fp32 rule as torch's e4m3fn cast after the same fp32 scaling."""
    rng = np.random.default_rng(1)
    h = (rng.standard_normal((37, 512)) * np.exp(rng.uniform(-8, 4, (37, 1)))).astype(np.float32)
    h[3, 128:256] = 0.0                                       # an all-zero block
    q, s = orc.quantize_block128_fp32(h)
    tq, ts = wl.quantize_fp8_rows_torch(torch.from_numpy(h))
    assert np.array_equal(q, tq.numpy()) and np.array_equal(s, ts.numpy())
    assert s[3, 1] == 1.0 and np.all(q[3, 128:256] == 0)


def test_block_requant_error_bound():
    """|decode(q)*s - h| <= 2^-4 |h| (3 mantissa bits, RNE) or half a
    subnormal step 2^-10 * s; every block's max maps to +-448."""
    rng = np.random.default_rng(2)
    h = (rng.standard_normal((50, 256)) * 3).astype(np.float32)
    q, s = orc.quantize_block128_fp32(h)
    back = orc.dequantize_block128(q, s)
    bound = np.maximum(2.0 ** -4 * np.abs(h), 2.0 ** -10 * np.repeat(s, 128, axis=1)) * (1 + 1e-6)
    assert np.all(np.abs(back - h) <= bound)
    blocks = np.abs(orc.e4m3fn_decode(q)).reshape(50, 2, 128)
    assert np.all(blocks.max(axis=-1) == 448.0)


def test_dequantize_matches_torch():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, size=(9, 384)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0                        # keep away from NaN codes
    sc = rng.random((9, 3)).astype(np.float32) + 0.1
    ref = (torch.from_numpy(codes).view(torch.float8_e4m3fn).double()
           * torch.from_numpy(sc).double().repeat_interleave(128, dim=1)).numpy()
    assert np.array_equal(orc.dequantize_block128(codes, sc), ref)


# ------------------------------------------------------------ fp8 layer


def _fp8_bruteforce(p):
    """Dense evaluation with torch's fp8 decode and torch's quantiser recipe
    for the intermediate; shares no function with the oracle's fp8 code."""
    def deq(c, s):
        return (c.view(torch.float8_e4m3fn).double() * s.double().repeat_interleave(128, dim=-1))
    x = deq(p["x"], p["x_scale"])
    W13 = deq(p["gate_up"], p["gate_up_scale"])
    W2 = deq(p["down"], p["down_scale"])
    idx, w = p["top_k_index"].long(), p["top_k_weights"].double()
    T, H = x.shape
    E, F2, _ = W13.shape
    F = F2 // 2
    out = torch.zeros(T, H, dtype=torch.float64)
    for t in range(T):
        for e in range(E):
            g = W13[e] @ x[t]
            h = torch.nn.functional.silu(g[:F]) * g[F:]
            q, s = wl.quantize_fp8_rows_torch(h.float()[None])
            ht = deq(q, s)[0]
            y = W2[e] @ ht
            m = sum(float(w[t, j]) for j in range(idx.shape[1]) if int(idx[t, j]) == e)
            out[t] += m * y
    return out.numpy()


def test_fp8_oracle_vs_bruteforce():
    p = wl.make_fp8_problem(6, 256, 128, 5, 3, seed=21, routing="uniform_softmax", routed_scale=1.0)
    ref = _fp8_bruteforce(p)
    got = orc.moe_experts_fp8_reference(p["x"].numpy(), p["x_scale"].numpy(), p["gate_up"].numpy(),
                                        p["gate_up_scale"].numpy(), p["down"].numpy(),
                                        p["down_scale"].numpy(), p["top_k_index"].numpy(),
                                        p["top_k_weights"].numpy())
    assert _rel(got, ref) < 1e-12


def test_fp8_oracle_invariants_and_token_subset():
    p = wl.make_fp8_problem(8, 256, 128, 6, 3, seed=22, routing="uniform_softmax", routed_scale=1.0)
    args = [p[n].numpy() for n in ("x", "x_scale", "gate_up", "gate_up_scale", "down", "down_scale")]
    idx, w = p["top_k_index"].numpy(), p["top_k_weights"].numpy().astype(np.float64)
    f = orc.moe_experts_fp8_reference
    base = f(*args, idx, w)
    assert np.all(f(*args, idx, np.zeros_like(w)) == 0.0)
    assert _rel(f(*args, idx, 2.0 * w), 2.0 * base) < 1e-14
    assert _rel(f(*args, idx[:, ::-1], w[:, ::-1]), base) < 1e-12
    sub = f(*args, idx, w, tokens=[1, 5])
    assert np.array_equal(sub[[1, 5]], base[[1, 5]]) and np.all(sub[[0, 2, 3, 4, 6, 7]] == 0)


# ------------------------------------------------------------ residual, bf16-input fp8


def test_residual_closed_form_and_zero_weights(golden):
    """[MPK] moe_local_reduction: out = sum_j w_j y_j + residual.  On the closed
    form above (out = silu(2) * 1 = 1.7615941559557646) a residual of 0.25 gives
    2.0115941559557646; with all routing weights zero the output is the
    residual itself, exactly."""
    c = golden["swiglu_h1_f1"]
    args = [np.array([c["x"]]), np.array(c["gate_up"]), np.array(c["down"]),
            np.array(c["top_k_index"])]
    for fn in (orc.moe_experts_reference, orc.moe_experts_reference_batched):
        out = fn(*args, np.array(c["top_k_weights"]), residual=np.array([[0.25]]))
        assert out[0, 0] == pytest.approx(2.0115941559557646, rel=1e-15)
    p = wl.make_bf16_problem(5, 128, 64, 6, 2, seed=31)
    r = np.random.default_rng(3).standard_normal((5, 128))
    zero = np.zeros(p["top_k_weights"].shape)
    for fn in (orc.moe_experts_reference, orc.moe_experts_reference_batched):
        out = fn(p["hidden"].float().numpy(), p["gate_up"].float().numpy(), p["down"].float().numpy(),
                 p["top_k_index"].numpy(), zero, residual=r)
        assert np.array_equal(out, r)
    q = wl.make_fp8_problem(4, 256, 128, 5, 2, seed=23, routing="uniform_softmax", routed_scale=1.0)
    fargs = [q[n].numpy() for n in ("x", "x_scale", "gate_up", "gate_up_scale", "down", "down_scale")]
    r8 = np.random.default_rng(4).standard_normal((4, 256))
    out = orc.moe_experts_fp8_reference(*fargs, q["top_k_index"].numpy(),
                                        np.zeros(q["top_k_weights"].shape), residual=r8)
    assert np.array_equal(out, r8)


def test_fp8_bf16_input_reduces_to_the_fp8_layer():
    """Hidden states that are e4m3 codes times a power-of-two block scale with
    each block's largest code at 448 quantise without loss (scale = amax/448 is
    the power of two, code = value * 448/amax exactly), so the bf16-input layer
    must equal the fp8 layer on those very codes and scales."""
    rng = np.random.default_rng(5)
    T, H, F, E, k = 4, 256, 128, 5, 2
    codes = rng.integers(0, 256, size=(T, H)).astype(np.uint8)
    codes[(codes & 0x7F) > 0x7E] = 0                 # no NaN, no 448 except where placed
    codes[(codes & 0x7F) == 0x7E] = 0x7D
    codes[:, ::128] = 0x7E                           # +448 leads every block
    scale = np.exp2(-rng.integers(3, 9, size=(T, H // 128))).astype(np.float32)
    hidden = orc.dequantize_block128(codes, scale)   # exact in float32 (and in bf16)
    assert np.array_equal(hidden.astype(np.float32).astype(np.float64), hidden)
    q = wl.make_fp8_problem(T, H, F, E, k, seed=24, routing="uniform_softmax", routed_scale=1.0)
    w = [q[n].numpy() for n in ("gate_up", "gate_up_scale", "down", "down_scale")]
    idx, wts = q["top_k_index"].numpy(), q["top_k_weights"].numpy()
    got = orc.moe_experts_fp8_bf16_reference(hidden, *w, idx, wts)
    ref = orc.moe_experts_fp8_reference(codes, scale, *w, idx, wts)
    assert np.array_equal(got, ref)


# ------------------------------------------------------- shared experts

def test_shared_expert_closed_form(golden):
    """Reading 11 on H = F = 1: routed silu(2) at weight 0.5 plus a shared
    expert -6 silu(1) at weight 1 (values derived by hand in the fixture)."""
    c = golden["shared_expert_h1_f1"]
    args = [np.array([c["x"]]), np.array(c["gate_up"]), np.array(c["down"]), np.array(c["top_k_index"])]
    sh = dict(shared_gate_up=np.array(c["shared_gate_up"]), shared_down=np.array(c["shared_down"]))
    for fn in (orc.moe_experts_reference, orc.moe_experts_reference_batched):
        out = fn(*args, np.array(c["top_k_weights"]), **sh)
        assert out[0, 0] == pytest.approx(c["out"][0][0], rel=1e-15)
        out0 = fn(*args, np.zeros((1, 1)), **sh)
        assert out0[0, 0] == pytest.approx(c["out_routing_weight_zero"][0][0], rel=1e-15)


def test_shared_experts_are_weight_one_slots():
    """A shared expert is a routed expert that every token selects with weight
    1: the same layer with the shared experts appended to the routed ones and
    one extra slot per shared expert gives the same output."""
    T, H, F, E, k, S = 7, 12, 6, 5, 2, 3
    x, w13, w2, idx, w = _problem(T, H, F, E, k, seed=21)
    rng = np.random.default_rng(22)
    sg = rng.standard_normal((S, 2 * F, H)) * 0.3
    sd = rng.standard_normal((S, H, F)) * 0.3
    idx_aug = np.concatenate([idx, np.tile(np.arange(E, E + S, dtype=np.int32), (T, 1))], axis=1)
    w_aug = np.concatenate([w, np.ones((T, S))], axis=1)
    ref = _dense_bruteforce(x, np.concatenate([w13, sg]), np.concatenate([w2, sd]), idx_aug, w_aug)
    for fn in (orc.moe_experts_reference, orc.moe_experts_reference_batched):
        assert _rel(fn(x, w13, w2, idx, w, shared_gate_up=sg, shared_down=sd), ref) < 1e-12


def test_shared_experts_equal_one_wide_expert():
    """S shared experts of width F equal one shared SwiGLU MLP of width S F
    whose gate rows, up rows and down columns are the experts' concatenated
    (SwiGLU is elementwise in F and the down product sums over F)."""
    T, H, F, E, k, S = 5, 10, 4, 3, 2, 2
    x, w13, w2, idx, w = _problem(T, H, F, E, k, seed=23)
    rng = np.random.default_rng(24)
    sg = rng.standard_normal((S, 2 * F, H)) * 0.3
    sd = rng.standard_normal((S, H, F)) * 0.3
    wide_g = np.concatenate([sg[s, :F] for s in range(S)])
    wide_u = np.concatenate([sg[s, F:] for s in range(S)])
    wide_gu = np.concatenate([wide_g, wide_u])[None]          # [1, 2 S F, H]
    wide_d = np.concatenate([sd[s] for s in range(S)], axis=1)[None]  # [1, H, S F]
    a = orc.moe_experts_reference(x, w13, w2, idx, w, shared_gate_up=sg, shared_down=sd)
    b = orc.moe_experts_reference(x, w13, w2, idx, w, shared_gate_up=wide_gu, shared_down=wide_d)
    assert _rel(a, b) < 1e-12
    # and with no routed contribution it is the dense SwiGLU MLP
    g = x @ wide_g.T
    dense = (g * scipy.special.expit(g) * (x @ wide_u.T)) @ wide_d[0].T
    c = orc.moe_experts_reference_batched(x, w13, w2, idx, np.zeros_like(w),
                                          shared_gate_up=sg, shared_down=sd)
    assert _rel(c, dense) < 1e-12


# ------------------------------------------------------- MX formats, MXFP4 layer

def test_e2m1_decode_golden(golden):
    c = golden["e2m1_codes"]
    got = orc.e2m1_decode(np.array(c["codes"]))
    assert np.array_equal(got, np.array(c["values"])) and np.array_equal(np.signbit(got), np.signbit(c["values"]))


def test_e2m1_encode_ties_roundtrip_and_recipe(golden):
    c = golden["e2m1_rne_ties"]
    assert orc.e2m1_encode(np.array(c["inputs"])).tolist() == c["codes"]
    codes = np.arange(16, dtype=np.uint8)
    back = orc.e2m1_encode(orc.e2m1_decode(codes))
    assert np.array_equal(orc.e2m1_decode(back), orc.e2m1_decode(codes))
    # against the input recipe's independent torch encoder on a dense sweep
    v = np.linspace(-6.0, 6.0, 24001).astype(np.float32)[None, :24000 // 32 * 32]
    v = v.reshape(-1, 32)
    v[:, 0] = 6.0                                        # unit block scale (amax 6 -> e = 0)
    packed, sc = wl.quantize_mxfp4_rows_torch(torch.from_numpy(v))
    assert np.all(sc.numpy() == 127)
    assert np.array_equal(orc.e2m1_decode(orc.unpack_e2m1(packed.numpy())),
                          orc.e2m1_decode(orc.e2m1_encode(v)))


def test_e8m0_decode_golden(golden):
    c = golden["e8m0_scales"]
    assert np.array_equal(orc.e8m0_decode(np.array(c["bytes"])), np.array(c["values"]))
    assert np.isnan(orc.e8m0_decode(255))


def test_mxfp8_block_golden_recipe_and_bound(golden):
    c = golden["mxfp8_block"]
    h = np.zeros((1, 32), np.float32)
    h[0, :4] = c["h_first4"]
    q, s = orc.quantize_mxfp8_fp32(h)
    assert q[0, :4].tolist() == c["codes_first4"] and np.all(q[0, 4:] == 0) and s[0, 0] == c["scale_byte"]
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((40, 256)) * np.exp(rng.uniform(-12, 12, (40, 1)))).astype(np.float32)
    x[3, 32:64] = 0.0                                    # an all-zero block
    q, s = orc.quantize_mxfp8_fp32(x)
    qt, st = wl.quantize_mxfp8_rows_torch(torch.from_numpy(x))
    assert np.array_equal(q, qt.numpy()) and np.array_equal(s, st.numpy())
    assert s[3, 1] == 0 and np.all(q[3, 32:64] == 0)
    deq = orc.dequantize_mx(orc.e4m3fn_decode(q), s)
    scale = np.repeat(orc.e8m0_decode(s), 32, axis=-1)
    # E4M3 keeps 3 mantissa bits: half an ulp is 2^-4 of the value in the normal
    # range, 2^-10 of the scale in the subnormal range; values above 448 units saturate
    unit = np.abs(x) / scale
    bound = np.where(unit >= 2.0 ** -6, np.abs(x) * 2.0 ** -4, scale * 2.0 ** -10)
    ok = unit <= 448
    assert np.all(np.abs(deq - x)[ok] <= bound[ok] * (1 + 1e-12))
    assert np.all(np.abs(deq[~ok]) == 448 * scale[~ok])


def _mxfp4_bruteforce(p):
    """Dense evaluation from the operands' definitions, written apart from the
    oracle: an E2M1 value table, torch's e4m3 decode, power-of-two scales, and
    the input recipe's MXFP8 quantiser for the intermediate."""
    table = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)

    def fp4(packed, sc):
        lo, hi = (packed & 0xF).long(), (packed >> 4).long()
        codes = torch.stack([lo, hi], dim=-1).reshape(*packed.shape[:-1], -1)
        v = table[codes & 7] * torch.where((codes & 8) > 0, -1.0, 1.0).double()
        return v * torch.pow(2.0, sc.double() - 127).repeat_interleave(32, dim=-1)

    def fp8(c, sc):
        return c.view(torch.float8_e4m3fn).double() * torch.pow(2.0, sc.double() - 127).repeat_interleave(32, dim=-1)

    x = fp8(p["x"], p["x_scale"])
    W13 = fp4(p["gate_up"], p["gate_up_scale"])
    W2 = fp4(p["down"], p["down_scale"])
    idx, w = p["top_k_index"].long(), p["top_k_weights"].double()
    T, H = x.shape
    E, F2, _ = W13.shape
    F = F2 // 2
    out = torch.zeros(T, H, dtype=torch.float64)
    for t in range(T):
        for e in range(E):
            g = W13[e] @ x[t]
            h = torch.nn.functional.silu(g[:F]) * g[F:]
            q, s = wl.quantize_mxfp8_rows_torch(h.float()[None])
            y = W2[e] @ fp8(q, s)[0]
            m = sum(float(w[t, j]) for j in range(idx.shape[1]) if int(idx[t, j]) == e)
            out[t] += m * y
    return out.numpy()


def _mx_args(p):
    return [p[n].numpy() for n in ("x", "x_scale", "gate_up", "gate_up_scale", "down", "down_scale")]


def test_mxfp4_oracle_vs_bruteforce():
    p = wl.make_mxfp4_problem(6, 128, 64, 5, 3, seed=31, routing="uniform_softmax", routed_scale=1.0)
    ref = _mxfp4_bruteforce(p)
    got = orc.moe_experts_mxfp4_reference(*_mx_args(p), p["top_k_index"].numpy(), p["top_k_weights"].numpy())
    assert _rel(got, ref) < 1e-12


def test_mxfp4_oracle_invariants_and_token_subset():
    p = wl.make_mxfp4_problem(8, 128, 64, 6, 3, seed=32, routing="uniform_softmax", routed_scale=1.0)
    args = _mx_args(p)
    idx, w = p["top_k_index"].numpy(), p["top_k_weights"].numpy().astype(np.float64)
    f = orc.moe_experts_mxfp4_reference
    base = f(*args, idx, w)
    assert np.all(f(*args, idx, np.zeros_like(w)) == 0.0)
    assert _rel(f(*args, idx, 2.0 * w), 2.0 * base) < 1e-14
    assert _rel(f(*args, idx[:, ::-1], w[:, ::-1]), base) < 1e-12
    sub = f(*args, idx, w, tokens=[2, 6])
    assert np.array_equal(sub[[2, 6]], base[[2, 6]]) and np.all(sub[[0, 1, 3, 4, 5, 7]] == 0)
    r = np.random.default_rng(9).standard_normal(base.shape)
    assert _rel(f(*args, idx, w, residual=r), base + r) < 1e-14


# ------------------------------------------------------------------ routers


def test_softmax_router_golden(golden):
    c = golden["softmax_router_quarters"]
    idx, w = orc.route_softmax_topk(np.array(c["logits"]), c["k"], c["routed_scaling_factor"])
    assert idx.tolist() == c["idx"]
    np.testing.assert_allclose(w, c["weights"], rtol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_softmax_router_vs_library(seed):
    """Distinct random logits: the choice is numpy's descending argsort, the
    weights scipy's softmax at those ids times the factor."""
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((40, 64)) * 3
    idx, w = orc.route_softmax_topk(lg, 6, 1.5)
    ref = np.argsort(-lg, axis=1, kind="stable")[:, :6]
    assert np.array_equal(idx, ref)
    p = scipy.special.softmax(lg, axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, ref, 1) * 1.5, rtol=1e-12)


def _rank_choice(score, allowed, k):
    """Chosen ids by counting: e is chosen iff it is allowed and fewer than k
    allowed ids beat it (larger score, or equal score and lower id); ordered
    by that count."""
    E = len(score)
    rank = {}
    for e in range(E):
        if not allowed[e]:
            continue
        rank[e] = sum(1 for f in range(E) if allowed[f] and
                      (score[f] > score[e] or (score[f] == score[e] and f < e)))
    return [e for e, r in sorted(rank.items(), key=lambda kv: kv[1]) if r < k]


def test_softmax_router_ties_shift_and_bruteforce():
    rng = np.random.default_rng(3)
    lg = rng.integers(-2, 3, (50, 8)).astype(np.float64)       # many exact ties
    idx, w = orc.route_softmax_topk(lg, 3, 1.0)
    for t in range(50):
        assert idx[t].tolist() == _rank_choice(lg[t], [True] * 8, 3)
    idx2, w2 = orc.route_softmax_topk(lg + 7.25, 3, 1.0)       # softmax is shift-invariant
    assert np.array_equal(idx, idx2)
    np.testing.assert_allclose(w, w2, rtol=1e-12)
    idx, w = orc.route_softmax_topk(np.zeros((2, 8)), 3, 2.0)  # all equal: first k ids, p = 1/E
    assert idx.tolist() == [[0, 1, 2]] * 2
    np.testing.assert_allclose(w, 2.0 / 8)


def test_sigmoid_router_golden(golden):
    c = golden["sigmoid_group_router_by_hand"]
    for gt, key in ((2, "idx_group_top2"), (1, "idx_group_top1")):
        idx, w = orc.route_sigmoid_group_topk(np.array(c["logits"]), np.array(c["bias"]), c["k"],
                                              c["num_groups"], c["topk_group"],
                                              c["routed_scaling_factor"], group_top=gt)
        assert idx.tolist() == c[key]
        np.testing.assert_allclose(w, c["weights"], rtol=1e-12)


def _sigmoid_router_bruteforce(lg, b, k, G, kg, gt, scale):
    T, E = lg.shape
    gs = E // G
    idx = np.zeros((T, k), np.int64)
    w = np.zeros((T, k))
    for t in range(T):
        s = scipy.special.expit(lg[t])
        c = s + b
        gscore = [sum(sorted(c[g * gs:(g + 1) * gs], reverse=True)[:gt]) for g in range(G)]
        kept = [sum(1 for h in range(G) if gscore[h] > gscore[g] or (gscore[h] == gscore[g] and h < g)) < kg
                for g in range(G)]
        ch = _rank_choice(c, [kept[e // gs] for e in range(E)], k)
        idx[t] = ch
        w[t] = s[ch] / s[ch].sum() * scale
    return idx, w


@pytest.mark.parametrize("gt", [1, 2])
@pytest.mark.parametrize("seed", [0, 1])
def test_sigmoid_router_vs_bruteforce(gt, seed):
    """Integer logits and a two-valued bias make exact ties in expert and in
    group scores; the counting formulation must agree id for id."""
    rng = np.random.default_rng(seed)
    E, G, kg, k = 16, 4, 2, 3
    lg = rng.integers(-2, 3, (60, E)).astype(np.float64)
    b = rng.choice([0.0, 0.25], E)
    idx, w = orc.route_sigmoid_group_topk(lg, b, k, G, kg, 2.5, group_top=gt)
    ri, rw = _sigmoid_router_bruteforce(lg, b, k, G, kg, gt, 2.5)
    assert np.array_equal(idx, ri)
    np.testing.assert_allclose(w, rw, rtol=1e-12)
    np.testing.assert_allclose(w.sum(1), 2.5, rtol=1e-12)


def test_sigmoid_router_one_group_is_plain_topk():
    """One group, no bias: the k largest logits (sigmoid is increasing), weights
    the renormalised sigmoids (torch.topk and scipy's expit as references)."""
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((30, 128))
    idx, w = orc.route_sigmoid_group_topk(lg, np.zeros(128), 8, 1, 1, 2.5)
    tv, ti = torch.topk(torch.from_numpy(lg), 8, dim=1)
    assert np.array_equal(idx, ti.numpy())
    s = scipy.special.expit(tv.numpy())
    np.testing.assert_allclose(w, s / s.sum(1, keepdims=True) * 2.5, rtol=1e-12)


# ------------------------------------------------ expert-batched fp8 and MXFP4 forms


def test_table_dequantisers_equal_the_element_decoders():
    """The table-driven dequantisers used by the batched forms give exactly the
    values of the per-element decoders."""
    rng = np.random.default_rng(41)
    codes = rng.integers(0, 256, size=(7, 384), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 1                         # NaN codes compare unequal
    sc = (rng.random((7, 3)) + 0.01).astype(np.float32)
    assert np.array_equal(orc.dequantize_block128_table(codes, sc), orc.dequantize_block128(codes, sc))
    packed = rng.integers(0, 256, size=(5, 3, 64), dtype=np.uint8)
    e8 = rng.integers(100, 150, size=(5, 3, 4), dtype=np.uint8)
    ref = orc.dequantize_mx(orc.e2m1_decode(orc.unpack_e2m1(packed)), e8)
    assert np.array_equal(orc.dequantize_mxfp4_table(packed, e8), ref)


@pytest.mark.parametrize("shape,seed", [((9, 256, 128, 5, 3), 51), ((24, 384, 256, 8, 2), 52),
                                        ((40, 128, 128, 3, 3), 53)])
def test_fp8_batched_equals_per_slot(shape, seed):
    """Expert-batched fp8 form against the per-slot form (same sums, another
    summation order): dropped ids, a token subset and a residual included."""
    T, H, F, E, k = shape
    p = wl.make_fp8_problem(T, H, F, E, k, seed=seed, routing="uniform_softmax", routed_scale=1.0)
    args = [p[n].numpy() for n in ("x", "x_scale", "gate_up", "gate_up_scale", "down", "down_scale")]
    idx, w = p["top_k_index"].numpy().copy(), p["top_k_weights"].numpy().astype(np.float64)
    idx[::4, 0] = -1
    idx[1::5, -1] = E
    r = np.random.default_rng(seed).standard_normal((T, H))
    a = orc.moe_experts_fp8_reference(*args, idx, w, residual=r)
    b = orc.moe_experts_fp8_reference_batched(*args, idx, w, residual=r)
    assert _rel(b, a) < 1e-12
    sub = [1, T - 1]
    assert _rel(orc.moe_experts_fp8_reference_batched(*args, idx, w, tokens=sub)[sub],
                orc.moe_experts_fp8_reference(*args, idx, w, tokens=sub)[sub]) < 1e-12


@pytest.mark.parametrize("shape,seed", [((9, 128, 64, 5, 3), 61), ((24, 256, 128, 8, 2), 62)])
def test_mxfp4_batched_equals_per_slot(shape, seed):
    T, H, F, E, k = shape
    p = wl.make_mxfp4_problem(T, H, F, E, k, seed=seed, routing="uniform_softmax", routed_scale=1.0)
    args = _mx_args(p)
    idx, w = p["top_k_index"].numpy().copy(), p["top_k_weights"].numpy().astype(np.float64)
    idx[::3, 1] = -1
    r = np.random.default_rng(seed).standard_normal((T, H))
    a = orc.moe_experts_mxfp4_reference(*args, idx, w, residual=r)
    b = orc.moe_experts_mxfp4_reference_batched(*args, idx, w, residual=r)
    assert _rel(b, a) < 1e-12
    sub = [0, 5]
    assert _rel(orc.moe_experts_mxfp4_reference_batched(*args, idx, w, tokens=sub)[sub],
                orc.moe_experts_mxfp4_reference(*args, idx, w, tokens=sub)[sub]) < 1e-12


def test_fp8_batched_vs_bruteforce():
    """The batched form against the torch-based dense brute force directly."""
    p = wl.make_fp8_problem(6, 256, 128, 5, 3, seed=23, routing="uniform_softmax", routed_scale=1.0)
    got = orc.moe_experts_fp8_reference_batched(*(p[n].numpy() for n in (
        "x", "x_scale", "gate_up", "gate_up_scale", "down", "down_scale", "top_k_index",
        "top_k_weights")))
    assert _rel(got, _fp8_bruteforce(p)) < 1e-12


# ------------------------------------------------------------ ue8m0 block-128 quantiser


def test_ue8m0_block_golden(golden):
    c = golden["block128_ue8m0"]
    h = np.zeros((4, 256), np.float32)
    for i, (row, rest) in enumerate(zip(c["rows_first2"], c["rest_of_row"])):
        h[i, :2] = row
        h[i, 2:128] = rest
    q, b = orc.quantize_block128_ue8m0(h)
    assert b[:, 0].tolist() == c["scale_bytes"]
    assert q[:, :2].tolist() == c["codes_first2"]
    assert np.all(b[:, 1] == 127) and np.all(q[:, 128:] == 0)    # all-zero second blocks


def test_ue8m0_matches_torch_recipe_and_bound():
    """torch recipe: e = ceil(log2(amax / 448)) in float64, then the e4m3fn cast of
    h / 2^e; plus the defining property amax / 2^e in (224, 448]."""
    rng = np.random.default_rng(71)
    h = (rng.standard_normal((29, 512)) * np.exp(rng.uniform(-20, 12, (29, 1)))).astype(np.float32)
    h[4, :128] = 0.0
    h[5, 128:256] = 448.0                                      # amax exactly 448 * 2^0
    h[6, :128] = np.float32(2.0 ** -30) * 448                  # exactly 448 * 2^-30
    q, b = orc.quantize_block128_ue8m0(h)
    t = torch.from_numpy(h).double().reshape(29, 4, 128)
    amax = t.abs().amax(-1)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax / 448.0)), torch.zeros_like(amax))
    v = (t / torch.exp2(e)[..., None]).clamp(-448, 448).float()
    tq = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(29, 512)
    assert np.array_equal(q, tq.numpy())
    assert np.array_equal(b.astype(np.int64), (e + 127).long().numpy())
    a = amax.numpy()
    s = np.exp2(b.astype(np.float64) - 127)
    nz = a > 0
    assert np.all(a[nz] / s[nz] <= 448.0) and np.all(a[nz] / s[nz] > 224.0)
    back = orc.e4m3fn_decode(q) * np.repeat(s, 128, axis=1)
    assert np.all(np.abs(back - h) <= np.maximum(2.0 ** -4 * np.abs(h), 2.0 ** -10 * np.repeat(s, 128, axis=1)))
