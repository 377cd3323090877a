"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: the routing plan is bit-exact; bf16 outputs satisfy
|gpu - ref| <= 1e-2 + 1e-2 |ref| per element, fp8 outputs
|gpu - ref| <= 3e-2 + 3e-2 |ref|, against the float64 oracle fed the same
seeded inputs (the fp8 oracle dequantises the same codes and re-quantises h
in fp32 as the method does).
"""

import os
import sys

import numpy as np
import pytest
import torch

import moe_workloads as wl
from oracle import moe_oracle as orc
from oracle_runner import check_quantized_layer

pytestmark = pytest.mark.gpu

BF16_TOL = (1e-2, 1e-2)
FP8_TOL = (3e-2, 3e-2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_routed_amd as moe  # noqa: F401  (fails loudly if the library is missing)
    moe._load()
    yield


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _moe():
    import mixture_experts_routed_amd as moe
    return moe


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_tol(gpu, ref, tol, what=""):
    atol, rtol = tol
    g = f64(gpu)
    err = np.abs(g - ref)
    bound = atol + rtol * np.abs(ref)
    worst = float(np.max(err / bound)) if err.size else 0.0
    rel_l2 = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30))
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    assert worst <= 1.0, f"{what}: worst err/tol {worst:.3f}, rel L2 {rel_l2:.2e}"
    return worst, rel_l2


def bf16_problem(T, H, F, E, k, seed, idx=None, std=0.02):
    p = wl.make_bf16_problem(T, H, F, E, k, seed, "cpu", weight_std=std)
    if idx is not None:
        p["top_k_index"] = torch.as_tensor(idx, dtype=torch.int32).contiguous()
    return p


def bf16_ref(p, batched=True):
    fn = orc.moe_experts_reference_batched if batched else orc.moe_experts_reference
    return fn(f64(p["hidden"]), f64(p["gate_up"]), f64(p["down"]), p["top_k_index"].numpy(),
              f64(p["top_k_weights"]))


def to_gpu(p):
    return {n: v.cuda() for n, v in p.items()}


def run_bf16(entry, g, out=None):
    moe = _moe()
    fn = getattr(moe, entry)
    return fn(g["hidden"], g["gate_up"], g["down"], g["top_k_index"], g["top_k_weights"],
              g["top_k_index"].shape[1], out=out)


# ------------------------------------------------------------------ plan


def _plan_case(idx, E):
    moe = _moe()
    idx = torch.as_tensor(idx, dtype=torch.int32)
    got = [t.cpu().numpy() for t in moe.moe_routing_plan(idx.cuda(), E)]
    ref = orc.routing_plan(idx.numpy(), E)
    for name, a, b in zip(("counts", "offsets", "perm", "inv"), got, ref):
        assert np.array_equal(a, b), f"plan {name} differs"


@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_plan_bit_exact_on_workloads(name):
    c = wl.CONFIGS[name]
    _say(f"plan {name}")
    g = wl._gen(c.get("act_seed", c["seed"]), "cpu")
    if c["routing"] == "zipf":
        idx, _ = wl.route_zipf(c["T"], c["E"], c["k"], g, "cpu", c["zipf_s"], c["zipf_zero"])
    elif c["routing"] == "sigmoid_topk":
        idx, _ = wl.route_sigmoid_topk(c["T"], c["E"], c["k"], g)
    else:
        idx, _ = wl.route_uniform_softmax(c["T"], c["E"], c["k"], g)
    _plan_case(idx, c["E"])


def test_plan_edge_cases():
    rng = np.random.default_rng(7)
    _say("plan edge cases")
    _plan_case(np.zeros((1, 1), np.int32), 1)                         # T=1, E=1
    _plan_case(np.full((700, 1), 3, np.int32), 8)                    # all to one expert
    _plan_case(rng.integers(-3, 11, (333, 4)).astype(np.int32), 8)   # dropped ids both sides
    _plan_case(rng.integers(0, 4, (50, 4)).astype(np.int32), 4)      # duplicates inside tokens
    _plan_case(np.full((5, 3), -1, np.int32), 16)                    # everything dropped
    _plan_case(np.stack([rng.permutation(512)[:8] for _ in range(600)]).astype(np.int32), 512)
    _plan_case(np.tile(np.arange(6, dtype=np.int32), (9, 1)), 6)    # k == E
    _plan_case(rng.integers(0, 128, (40000, 1)).astype(np.int32), 128)  # long run per wave


# ------------------------------------------------------------- bf16 layer


@pytest.mark.parametrize("entry", ["moe_experts_prefill", "moe_experts_decode"])
def test_tiny_config(entry):
    _say(f"tiny {entry}")
    p = wl.make_config("tiny")
    ref = bf16_ref(p, batched=False)
    out = run_bf16(entry, to_gpu(p))
    check_tol(out, ref, BF16_TOL, f"tiny/{entry}")
    # outputs of the tiny config are below atol; also require a small relative L2 error
    rel = np.linalg.norm(f64(out) - ref) / np.linalg.norm(ref)
    assert rel < 1e-2, rel


def test_tiny_scaled_twin():
    """Tiny shapes with weights ~N(0, 1/sqrt(H)) so that outputs are O(1)."""
    _say("tiny scaled twin")
    p = bf16_problem(16, 128, 64, 8, 2, 1001, std=1 / np.sqrt(128))
    ref = bf16_ref(p, batched=False)
    for entry in ("moe_experts_prefill", "moe_experts_decode"):
        check_tol(run_bf16(entry, to_gpu(p)), ref, BF16_TOL, entry)


@pytest.mark.parametrize("shape", [
    (700, 384, 320, 6, 2),     # several M tiles per expert and ragged tails
    (257, 128, 64, 5, 3),      # one row past a tile
    (96, 256, 192, 16, 4),     # many small experts, some empty
    (300, 192, 128, 4, 4),     # k == E; H not a multiple of 128 (64-wide down tiles)
    (64, 1024, 128, 128, 2),   # many experts: the down product keeps 256-wide panel tiles
])
def test_prefill_medium(shape):
    T, H, F, E, k = shape
    _say(f"prefill medium {shape}")
    p = bf16_problem(T, H, F, E, k, seed=11 + T, std=1 / np.sqrt(H))
    ref = bf16_ref(p)
    check_tol(run_bf16("moe_experts_prefill", to_gpu(p)), ref, BF16_TOL, str(shape))


def test_prefill_edge_routing():
    """All tokens to one expert, dropped ids (-1 and E), duplicates in a token, empty experts."""
    _say("prefill edge routing")
    T, H, F, E, k = 600, 128, 64, 6, 2
    rng = np.random.default_rng(3)
    cases = {
        "one_expert": np.stack([np.full(T, 2), np.full(T, 2)], 1),
        "dropped": np.where(rng.random((T, k)) < 0.2, rng.choice([-1, E], (T, k)), rng.integers(0, E, (T, k))),
        "dups": np.stack([rng.integers(0, 3, T)] * 2, 1),
    }
    for name, idx in cases.items():
        p = bf16_problem(T, H, F, E, k, seed=5, idx=idx.astype(np.int32), std=1 / np.sqrt(H))
        ref = bf16_ref(p, batched=False)
        for entry in ("moe_experts_prefill", "moe_experts_decode"):
            check_tol(run_bf16(entry, to_gpu(p)), ref, BF16_TOL, f"{name}/{entry}")


def test_prefill_full_config():
    """T=2048, H=1280, F=896, E=64, top-6: every output element against the oracle."""
    _say("prefill full config")
    p = wl.make_config("ocr2_prefill")
    g = to_gpu(p)
    out = run_bf16("moe_experts_prefill", g)
    torch.cuda.synchronize()
    ref = bf16_ref(p)
    worst, rel = check_tol(out, ref, BF16_TOL, "ocr2_prefill")
    _say(f"  worst err/tol {worst:.3f} rel L2 {rel:.2e}")


@pytest.mark.parametrize("name", ["ocr2_decode_t1", "ocr2_decode_t4"])
def test_decode_full_config(name):
    _say(f"decode {name}")
    p = wl.make_config(name)
    ref = bf16_ref(p, batched=False)
    g = to_gpu(p)
    for entry in ("moe_experts_decode", "moe_experts_prefill"):
        worst, rel = check_tol(run_bf16(entry, g), ref, BF16_TOL, f"{name}/{entry}")
        _say(f"  {entry}: worst err/tol {worst:.3f} rel L2 {rel:.2e}")


@pytest.mark.parametrize("shape", [(3, 128, 64, 8, 2), (4, 256, 1536, 6, 5), (4, 256, 1536, 8, 8),
                                   (4, 256, 2048, 8, 7), (2, 512, 2048, 3, 3),
                                   (4, 128, 128, 40, 8), (1, 1024, 96 * 2, 8, 4),
                                   (2, 1536, 64, 5, 2), (3, 2048, 128, 8, 3), (4, 1536, 64, 8, 2),
                                   (4, 2048, 64, 8, 2), (7, 128, 64, 8, 2)])
def test_decode_shapes(shape):
    """Fast path for T <= 4 (1 to 4 16-byte chunks per lane of an H row, 1 to 4
    tokens, h up to its LDS limit T*k*F = 49152 and 32 slots), grouped path
    above it (T = 7, T = 4 with H = 2048, and T*k*F = 57344)."""
    T, H, F, E, k = shape
    _say(f"decode shape {shape}")
    p = bf16_problem(T, H, F, E, k, seed=T + F, std=1 / np.sqrt(H))
    ref = bf16_ref(p, batched=False)
    check_tol(run_bf16("moe_experts_decode", to_gpu(p)), ref, BF16_TOL, str(shape))


@pytest.mark.parametrize("shape", [(1, 1792, 896, 64, 8), (1, 1920, 896, 64, 8), (1, 1280, 512, 64, 8),
                                   (1, 1280, 896, 64, 3), (2, 1280, 896, 64, 8), (3, 1536, 896, 64, 6),
                                   (4, 1536, 896, 64, 6)])
def test_decode_work_split_boundaries(shape):
    """Work splits of the one-launch decode on a grid of one workgroup per
    CU (256 on MI355X): with H = 1792 and 8 distinct experts each workgroup
    has exactly seven full down steps of 8 rows; with H = 1920 its output
    rows alternate between 7 and 8, so one grid mixes the one-step split
    and the split into two-step prefetches plus the rest; F = 512 gives
    16-row steps; k = 3 leaves a partial last gate/up batch in most
    workgroups; T = 2-4 take the multi-token kernel, whose down products
    skip the tokens not routed to the task's expert (tokens past T too)."""
    T, H, F, E, k = shape
    _say(f"decode split {shape}")
    p = bf16_problem(T, H, F, E, k, seed=7 * T + H, std=1 / np.sqrt(H))
    ref = bf16_ref(p, batched=False)
    check_tol(run_bf16("moe_experts_decode", to_gpu(p)), ref, BF16_TOL, str(shape))


@pytest.mark.parametrize("T", [1, 3])
def test_decode_dropped_slots_with_stale_workspace(T):
    """Dropped slots (-1 and E) on the gather-GEMV path with a workspace whose
    stale contents are NaN: a dropped slot's partial sums are never written and
    must not reach the output (no 0 * NaN)."""
    moe = _moe()
    H, F, E, k = 256, 128, 8, 3
    _say(f"decode dropped slots, stale NaN workspace, T={T}")
    p = bf16_problem(T, H, F, E, k, seed=71, std=1 / np.sqrt(H))
    idx = p["top_k_index"].clone()
    idx[:, 0] = -1
    idx[::2, 1] = E
    p["top_k_index"] = idx.contiguous()
    ref = bf16_ref(p, batched=False)
    g = to_gpu(p)
    n = moe.moe_workspace_size(1, T, H, F, E, k)
    ws = torch.full((n // 4,), float("nan"), device="cuda").view(torch.uint8)
    out = moe.moe_experts_decode(g["hidden"], g["gate_up"], g["down"], g["top_k_index"],
                                 g["top_k_weights"], k, workspace=ws)
    check_tol(out, ref, BF16_TOL, f"dropped slots T={T}")


def test_decode_after_grouped_call_on_one_workspace():
    """A decode call on a workspace a grouped call has just used, whose
    routing gives experts 0, 1, 2 the counts 0, 1, 0 (64 experts): the plan
    then leaves, at the decode's generation word, counts 0 and 1, and at the
    decode's second flag word the offsets 1 and 1, i.e. the generation word
    plus one.  The decode's flag words must not take that for a flag of this
    call; its output equals, bit for bit, the same decode on a fresh
    workspace, and matches the oracle."""
    moe = _moe()
    H, F, E, k, Tg = 1280, 896, 64, 6, 16
    _say("decode after a grouped call on one workspace (counts 0, 1, 0)")
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(np.arange(3, E), size=k, replace=False) for _ in range(Tg)])
    idx[0, 0] = 1
    pg = bf16_problem(Tg, H, F, E, k, seed=73, idx=idx)
    gg = to_gpu(pg)
    lay = moe.moe_workspace_layout(0, Tg, H, F, E, k)
    assert lay["counts"] == 0 and lay["offsets"] == 256, lay   # counts at 0, offsets at 256
    n = max(moe.moe_workspace_size(0, Tg, H, F, E, k), moe.moe_workspace_size(1, 1, H, F, E, k))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    moe.moe_experts_prefill(gg["hidden"], gg["gate_up"], gg["down"], gg["top_k_index"],
                            gg["top_k_weights"], k, workspace=ws)
    torch.cuda.synchronize()
    head = ws[:512].cpu().view(torch.int32).numpy()
    assert list(head[:3]) == [0, 1, 0] and list(head[66:68]) == [1, 1], (head[:3], head[64:68])
    # the decode: one token of the same layer, routed to experts 1 .. 6
    pd = {"hidden": pg["hidden"][:1].clone(), "gate_up": pg["gate_up"], "down": pg["down"],
          "top_k_index": torch.arange(1, k + 1, dtype=torch.int32).view(1, k),
          "top_k_weights": torch.softmax(torch.linspace(-1, 1, k), 0).view(1, k).float()}
    gd = to_gpu(pd)
    args = (gd["hidden"], gd["gate_up"], gd["down"], gd["top_k_index"], gd["top_k_weights"], k)
    out = moe.moe_experts_decode(*args, workspace=ws)
    fresh = moe.moe_experts_decode(*args, workspace=torch.zeros_like(ws))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), fresh.view(torch.int16))
    check_tol(out, bf16_ref(pd, batched=False), BF16_TOL, "decode after grouped call")


@pytest.mark.parametrize("T", [1, 2, 4])
def test_decode_repeated_expert_in_token(T):
    """Gather-GEMV path with a token that lists one expert in several slots
    (each slot adds its own weighted copy of that expert's output), mixed with
    a dropped slot, against the per-slot oracle."""
    moe = _moe()
    H, F, E, k = 256, 128, 8, 4
    _say(f"decode repeated expert in a token, T={T}")
    p = bf16_problem(T, H, F, E, k, seed=90 + T, std=1 / np.sqrt(H))
    idx = p["top_k_index"].clone()
    idx[0] = torch.tensor([3, 3, 5, 3], dtype=torch.int32)
    if T > 1:
        idx[T - 1] = torch.tensor([6, -1, 6, 2], dtype=torch.int32)
    p["top_k_index"] = idx.contiguous()
    ref = bf16_ref(p, batched=False)
    g = to_gpu(p)
    n = moe.moe_workspace_size(1, T, H, F, E, k)
    ws = torch.full((n // 4,), float("nan"), device="cuda").view(torch.uint8)
    out = moe.moe_experts_decode(g["hidden"], g["gate_up"], g["down"], g["top_k_index"],
                                 g["top_k_weights"], k, workspace=ws)
    check_tol(out, ref, BF16_TOL, f"repeated expert T={T}")


def test_stages_prefill():
    """Layered check: h and y (bf16, both in expert order) in the workspace."""
    moe = _moe()
    _say("prefill stages")
    T, H, F, E, k = 300, 256, 128, 5, 2
    p = bf16_problem(T, H, F, E, k, seed=9, std=1 / np.sqrt(H))
    g = to_gpu(p)
    lay = moe.moe_workspace_layout(0, T, H, F, E, k)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    moe.moe_experts_prefill(g["hidden"], g["gate_up"], g["down"], g["top_k_index"],
                            g["top_k_weights"], k, workspace=ws)
    torch.cuda.synchronize()
    P = T * k
    perm = ws[lay["perm"]:lay["perm"] + 4 * P].view(torch.int32).cpu().numpy()
    h = ws[lay["h"]:lay["h"] + 2 * P * F].view(torch.bfloat16).view(P, F)
    y = ws[lay["y"]:lay["y"] + 2 * P * H].view(torch.bfloat16).view(P, H)
    x, w13, w2, idx = f64(p["hidden"]), f64(p["gate_up"]), f64(p["down"]), p["top_k_index"].numpy()
    h_ref = np.zeros((P, F))
    y_ref = np.zeros((P, H))
    for m in range(P):
        s = perm[m]
        e = idx.reshape(-1)[s]
        gv = w13[e] @ x[s // k]
        h_ref[m] = orc.silu(gv[:F]) * gv[F:]
        y_ref[m] = w2[e] @ h_ref[m]
    check_tol(h, h_ref, (1e-2, 1e-2), "h stage")
    check_tol(y, y_ref, (1e-2, 1e-2), "y stage")


def test_out_fully_overwritten_and_deterministic():
    _say("overwrite + determinism")
    p = wl.make_config("ocr2_decode_t4")
    g = to_gpu(p)
    for entry in ("moe_experts_prefill", "moe_experts_decode"):
        poison = torch.full((4, 1280), float("nan"), dtype=torch.bfloat16, device="cuda")
        a = run_bf16(entry, g, out=poison).clone()
        assert torch.isfinite(a.float()).all()
        b = run_bf16(entry, g)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), entry
    p = wl.make_config("ocr2_prefill")
    g = to_gpu(p)
    a = run_bf16("moe_experts_prefill", g).clone()
    b = run_bf16("moe_experts_prefill", g)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_zero_tokens_and_zero_weights():
    _say("T=0 and zero weights")
    moe = _moe()
    p = bf16_problem(0, 128, 64, 4, 2, seed=1)
    g = to_gpu(p)
    assert run_bf16("moe_experts_prefill", g).shape == (0, 128)
    p = bf16_problem(64, 128, 64, 4, 2, seed=1)
    p["top_k_weights"] = torch.zeros_like(p["top_k_weights"])
    g = to_gpu(p)
    for entry in ("moe_experts_prefill", "moe_experts_decode"):
        assert torch.count_nonzero(run_bf16(entry, g).float()) == 0
    assert moe.moe_experts_decode(g["hidden"][:2], g["gate_up"], g["down"], g["top_k_index"][:2],
                                  g["top_k_weights"][:2], 2).abs().sum() == 0


# -------------------------------------------------------------- fp8 layer


def fp8_ref(p, tokens=None):
    return orc.moe_experts_fp8_reference(
        p["x"].cpu().numpy(), p["x_scale"].cpu().numpy(), p["gate_up"], p["gate_up_scale"],
        p["down"], p["down_scale"], p["top_k_index"].cpu().numpy(),
        p["top_k_weights"].cpu().numpy(), tokens=tokens)


def run_fp8(g, out=None):
    moe = _moe()
    return moe.moe_experts_fp8(g["x"], g["x_scale"], g["gate_up"], g["gate_up_scale"], g["down"],
                               g["down_scale"], g["top_k_index"], g["top_k_weights"],
                               g["top_k_index"].shape[1], out=out)


# (T, H, F, E, k)
@pytest.mark.parametrize("shape", [(300, 512, 384, 6, 3), (64, 256, 128, 8, 4), (520, 128, 256, 2, 2),
                                   (600, 256, 128, 4, 2),    # 3 M tiles per expert, 1 K step in down
                                   (700, 512, 256, 3, 2),    # 467 rows per expert
                                   # K / 128 a multiple of 4 (16-byte scale loads) in both
                                   # products, two scale loads per row; then in the
                                   # 128-wide down panels (H % 256 != 0)
                                   (600, 1024, 512, 4, 2), (300, 384, 1024, 4, 2)])
def test_fp8_medium(shape):
    T, H, F, E, k = shape
    _say(f"fp8 medium {shape}")
    p = wl.make_fp8_problem(T, H, F, E, k, seed=31 + T, routing="uniform_softmax", routed_scale=1.0)
    ref = fp8_ref({n: v.numpy() if n not in ("x", "x_scale", "top_k_index", "top_k_weights") else v
                   for n, v in p.items()})
    worst, rel = check_tol(run_fp8(to_gpu(p)), ref, FP8_TOL, str(shape))
    _say(f"  worst err/tol {worst:.3f} rel L2 {rel:.2e}")


# (T, H, F, E, k, hot): decode batches (at most 32 rows per expert on average,
# F % 256 == 0, H % 512 == 0) take 32-row tiles and 512-row panels; `hot`
# tokens all choose expert 0 first, so that it spans several 32-row tiles
@pytest.mark.parametrize("shape", [(48, 512, 256, 16, 4, 0), (64, 1024, 512, 8, 2, 40),
                                   (16, 512, 768, 32, 8, 0)])
def test_fp8_decode_batch_tiles(shape):
    T, H, F, E, k, hot = shape
    _say(f"fp8 decode batch {shape}")
    p = wl.make_fp8_problem(T, H, F, E, k, seed=57 + T, routing="uniform_softmax", routed_scale=1.0)
    if hot:
        idx = p["top_k_index"].clone()
        for t in range(hot):
            row = idx[t]
            row[row == 0] = row[0].clone()   # keep the k ids distinct
            row[0] = 0
        p["top_k_index"] = idx.contiguous()
        assert int((p["top_k_index"] == 0).sum()) >= hot
    ref = fp8_ref({n: v.numpy() if n not in ("x", "x_scale", "top_k_index", "top_k_weights") else v
                   for n, v in p.items()})
    worst, rel = check_tol(run_fp8(to_gpu(p)), ref, FP8_TOL, str(shape))
    _say(f"  worst err/tol {worst:.3f} rel L2 {rel:.2e}")


@pytest.mark.parametrize("shape", [(200, 256, 256, 4, 2), (512, 256, 256, 4, 2),
                                   (40, 512, 512, 8, 2)])   # decode-batch tiles: 4 waves per h block
def test_fp8_h_stage_codes(shape):
    """The re-quantised h in the workspace against the oracle's fp32 rule applied
    to the oracle's h.  The kernel quantises its own fp32-accumulated h, which
    differs from the oracle's float64 h by fp32 summation error (about 1e-5
    relative), so scales agree to 1e-4 and codes agree except for rare
    one-step flips at rounding boundaries.  Bit-exactness of the quantiser on
    identical inputs is test_quantizer_bit_exact and test_fp8_h_stage_exact."""
    moe = _moe()
    _say(f"fp8 h stage {shape}")
    T, H, F, E, k = shape
    p = wl.make_fp8_problem(T, H, F, E, k, seed=41, routing="uniform_softmax", routed_scale=1.0)
    g = to_gpu(p)
    lay = moe.moe_workspace_layout(2, T, H, F, E, k)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    moe.moe_experts_fp8(g["x"], g["x_scale"], g["gate_up"], g["gate_up_scale"], g["down"],
                        g["down_scale"], g["top_k_index"], g["top_k_weights"], k, workspace=ws)
    torch.cuda.synchronize()
    P = T * k
    perm = ws[lay["perm"]:lay["perm"] + 4 * P].view(torch.int32).cpu().numpy()
    hq = ws[lay["h"]:lay["h"] + P * F].cpu().numpy().reshape(P, F)
    hs = ws[lay["h_scale"]:lay["h_scale"] + 4 * P * (F // 128)].view(torch.float32).cpu().numpy().reshape(P, F // 128)
    x = orc.dequantize_block128(p["x"].numpy(), p["x_scale"].numpy())
    idx = p["top_k_index"].numpy().reshape(-1)
    h_ref = np.zeros((P, F), np.float32)
    for m in range(P):
        s = perm[m]
        e = idx[s]
        W = orc.dequantize_block128(p["gate_up"][e].numpy(), p["gate_up_scale"][e].numpy())
        gv = W @ x[s // k]
        h_ref[m] = (orc.silu(gv[:F]) * gv[F:]).astype(np.float32)
    q_ref, s_ref = orc.quantize_block128_fp32(h_ref)
    np.testing.assert_allclose(hs, s_ref, rtol=1e-4)
    diff = hq != q_ref
    assert diff.mean() < 2e-3, diff.mean()
    a, b = orc.e4m3fn_decode(hq[diff]), orc.e4m3fn_decode(q_ref[diff])
    # in code units (h / scale, max 448): one e4m3 step, plus the absolute
    # fp32 accumulation error of h (<= 1e-4 of the block max) that can push a
    # near-zero value across zero
    assert np.all(np.abs(a - b) <= np.maximum(np.abs(a), np.abs(b)) * 2.0 ** -3 + 448e-4)


def test_quantizer_bit_exact():
    """Stand-alone block-128 quantiser (same device routine as the fp8 epilogue)
    against the oracle's rule on identical fp32 and bf16 inputs."""
    moe = _moe()
    _say("quantizer")
    rng = np.random.default_rng(5)
    h = (rng.standard_normal((333, 1024)) * np.exp(rng.uniform(-10, 6, (333, 1)))).astype(np.float32)
    h[7, 256:384] = 0.0
    h[8, :128] = -0.0
    h[9, :128] = 1e-30
    codes, scales = moe.moe_quantize_fp8_block128(torch.from_numpy(h).cuda())
    q_ref, s_ref = orc.quantize_block128_fp32(h)
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    hb = torch.from_numpy(h).to(torch.bfloat16)
    codes, scales = moe.moe_quantize_fp8_block128(hb.cuda())
    q_ref, s_ref = orc.quantize_block128_fp32(hb.float().numpy())
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    assert np.array_equal(scales.cpu().numpy(), s_ref)


def test_quantizer_ue8m0_bit_exact():
    """Power-of-two (ue8m0) block-128 quantiser against the oracle's rule:
    codes and scale bytes bit for bit, fp32 and bf16 inputs, with zero and
    negative-zero blocks, tiny and huge blocks, and block maxima exactly at
    448 * 2^e and just above it (where e steps)."""
    moe = _moe()
    _say("quantizer ue8m0")
    rng = np.random.default_rng(11)
    h = (rng.standard_normal((257, 1024)) * np.exp(rng.uniform(-30, 30, (257, 1)))).astype(np.float32)
    h[3, 256:384] = 0.0
    h[4, :128] = -0.0
    h[5, :128] = 1e-38                       # amax = 1e-38: e clamps at -127
    h[6, 128:256] = 448.0                    # amax = 448 * 2^0 exactly: e = 0
    h[7, 128:256] = -448.0 * 2.0 ** -20      # exactly 448 * 2^-20
    h[8, :128] = np.nextafter(np.float32(448.0), np.float32(1e9))   # just above: e = 1
    h[9, 512:640] = 3.0e38                   # near the fp32 maximum
    t = torch.from_numpy(h).cuda()
    for inp in (t, t.to(torch.bfloat16)):
        codes, sb = moe.moe_quantize_fp8_block128_ue8m0(inp)
        q_ref, s_ref = orc.quantize_block128_ue8m0(inp.float().cpu().numpy())
        assert np.array_equal(sb.cpu().numpy(), s_ref)
        assert np.array_equal(codes.cpu().numpy(), q_ref)
        if inp.dtype == torch.float32:   # the cases at the step of e
            assert s_ref[6, 1] == 127 and s_ref[8, 0] == 128 and s_ref[5, 0] == 0


# Many rows per expert (prefill-sized, 128-row tiles x 256-row panels):
# (T, H, F, E, k, skew).  skew > 0 routes most tokens to expert 0 (many M
# tiles and a ragged last one), gives the last-but-one expert a handful of
# rows (a tile with idle row blocks) and the last expert none.
@pytest.mark.parametrize("shape", [(700, 512, 512, 4, 2, 0), (1000, 1024, 512, 3, 2, 0),
                                   (900, 512, 1024, 5, 2, 1), (64 * 9, 2048, 512, 2, 1, 0)])
def test_fp8_many_rows_per_expert(shape):
    T, H, F, E, k, skew = shape
    _say(f"fp8 many rows {shape}")
    p = wl.make_fp8_problem(T, H, F, E, k, seed=101 + T, routing="uniform_softmax", routed_scale=1.0)
    if skew:
        rng = np.random.default_rng(T)
        idx = np.zeros((T, k), dtype=np.int32)
        for t in range(T):
            first = 0 if t < T - 20 else E - 2
            rest = rng.choice([e for e in range(E - 1) if e != first], k - 1, replace=False)
            idx[t] = [first, *rest]
        p["top_k_index"] = torch.from_numpy(idx)
    g = to_gpu(p)
    moe = _moe()
    out, ws, lay = _run_fp8_ws(moe, g)
    st = check_quantized_layer("fp8", out, g, ws, lay, str(shape), orc)
    _say(f"  {st}")
    again = run_fp8(g)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))


def _run_fp8_ws(moe, g, variant=None):
    T, H = g["x"].shape
    E, F2, _ = g["gate_up"].shape
    k = g["top_k_index"].shape[1]
    lay = moe.moe_workspace_layout(moe.MOE_VARIANT_FP8 if variant is None else variant, T, H,
                                   F2 // 2, E, k)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    out = moe.moe_experts_fp8(g["x"], g["x_scale"], g["gate_up"], g["gate_up_scale"], g["down"],
                              g["down_scale"], g["top_k_index"], g["top_k_weights"], k, workspace=ws)
    torch.cuda.synchronize()
    return out, ws, lay


@pytest.mark.parametrize("name", ["v3_fp8_decode", "v3_fp8_prefill"])
def test_fp8_full_config_every_row(name):
    """Full DeepSeek-V3-shaped expert share (T=128 decode batch, T=4096 Zipf
    prefill with empty experts): every output element against the
    expert-batched oracle (pinned to the per-slot form on the CPU), after
    checking that each requantised h code the kernel chose is a rounding of
    the oracle's h; a second call is bit-identical."""
    moe = _moe()
    _say(f"fp8 full {name}")
    p = wl.make_config(name, device="cuda")
    out, ws, lay = _run_fp8_ws(moe, p)
    st = check_quantized_layer("fp8", out, p, ws, lay, name, orc)
    idx = p["top_k_index"].cpu().numpy()
    counts = np.bincount(idx.reshape(-1), minlength=p["gate_up"].shape[0])
    _say(f"  all {out.shape[0]} rows: {st}; max/mean load {counts.max() / counts.mean():.1f}, "
         f"empty {(counts == 0).sum()}")
    b = run_fp8(p)
    assert torch.equal(out.view(torch.int16), b.view(torch.int16)), "fp8 path not deterministic"


# (T, H, F, E, k): with the persistent grid capped at 8 workgroups every
# workgroup runs many work items in a row (ring slots, scale rings and the
# per-item set-up reused across items): 128-row tiles with 16-byte scale loads,
# 128-wide down panels, and 32-row decode-batch tiles.  The capped call must
# equal the uncapped one bit for bit, and that one the oracle.
@pytest.mark.parametrize("shape", [(600, 1024, 512, 4, 2), (700, 512, 256, 3, 2),
                                   (300, 384, 1024, 4, 2), (128, 1024, 512, 16, 4),
                                   (1000, 1024, 512, 3, 2)])
def test_fp8_many_items_per_workgroup(shape):
    moe = _moe()
    T, H, F, E, k = shape
    _say(f"fp8 capped grid {shape}")
    p = wl.make_fp8_problem(T, H, F, E, k, seed=83 + T, routing="uniform_softmax", routed_scale=1.0)
    g = to_gpu(p)
    out, ws, lay = _run_fp8_ws(moe, g)
    moe.moe_set_grid_cap(8)
    try:
        capped = run_fp8(g)
        torch.cuda.synchronize()
    finally:
        moe.moe_set_grid_cap(0)
    assert torch.equal(out.view(torch.int16), capped.view(torch.int16)), "grid-dependent result"
    st = check_quantized_layer("fp8", out, g, ws, lay, str(shape), orc)
    _say(f"  {st}")


@pytest.mark.parametrize("shape", [(96, 256, 256, 4, 2), (40, 512, 512, 8, 2)])
def test_fp8_h_stage_exact(shape):
    """Small-integer operands with unit scales make every fp32 sum of the
    gate_up product exact; every gate dot product is at least 20, where
    silu(g) = g in fp32 (1 + e^-20 rounds to 1), so h = g_gate * g_up is an
    exact integer and the epilogue's requantised codes and scales must equal
    the oracle's fp32 block-128 rule bit for bit (128-row tiles, then the
    32-row decode-batch tiles)."""
    moe = _moe()
    T, H, F, E, k = shape
    _say(f"fp8 exact h stage {shape}")
    rng = np.random.default_rng(17)
    x = rng.integers(1, 3, size=(T, H)).astype(np.float64)              # 1 or 2
    gate = (rng.random((E, F, H)) < 0.3).astype(np.float64)
    gate[..., :20] = 1.0                                                # >= 20 ones per row
    up = rng.integers(-2, 3, size=(E, F, H)).astype(np.float64)
    down = rng.integers(-2, 3, size=(E, H, F)).astype(np.float64)
    idx, w = wl.route_uniform_softmax(T, E, k, torch.Generator().manual_seed(5), "cpu", 1.0)
    enc = lambda a: torch.from_numpy(orc.e4m3fn_encode(a))
    ones = lambda *s: torch.ones(*s, dtype=torch.float32)
    g = {"x": enc(x), "x_scale": ones(T, H // 128),
         "gate_up": enc(np.concatenate([gate, up], axis=1)), "gate_up_scale": ones(E, 2 * F, H // 128),
         "down": enc(down), "down_scale": ones(E, H, F // 128),
         "top_k_index": idx, "top_k_weights": w}
    g = to_gpu(g)
    lay = moe.moe_workspace_layout(moe.MOE_VARIANT_FP8, T, H, F, E, k)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    moe.moe_experts_fp8(g["x"], g["x_scale"], g["gate_up"], g["gate_up_scale"], g["down"],
                        g["down_scale"], g["top_k_index"], g["top_k_weights"], k, workspace=ws)
    torch.cuda.synchronize()
    P = T * k
    perm = ws[lay["perm"]:lay["perm"] + 4 * P].view(torch.int32).cpu().numpy()
    hq = ws[lay["h"]:lay["h"] + P * F].cpu().numpy().reshape(P, F)
    hs = ws[lay["h_scale"]:lay["h_scale"] + 4 * P * (F // 128)].view(torch.float32).cpu().numpy()
    ids = idx.numpy().reshape(-1)
    h = np.stack([(gate[ids[s]] @ x[s // k]) * (up[ids[s]] @ x[s // k]) for s in perm])
    assert np.all(np.abs(h) < 2.0 ** 24)
    q_ref, s_ref = orc.quantize_block128_fp32(h.astype(np.float32))
    assert np.array_equal(hs.reshape(P, F // 128), s_ref), "h scales differ"
    assert np.array_equal(hq, q_ref), f"{int((hq != q_ref).sum())} h codes differ"


@pytest.mark.parametrize("shape", [(100, 256, 128, 4, 3), (400, 256, 128, 4, 3)])
def test_fp8_overwrite_and_dropped(shape):
    _say(f"fp8 overwrite + dropped {shape}")
    T, H, F, E, k = shape
    p = wl.make_fp8_problem(T, H, F, E, k, seed=3, routing="uniform_softmax", routed_scale=1.0)
    idx = p["top_k_index"].clone()
    idx[::3, 1] = -1
    idx[1::5, 2] = E
    p["top_k_index"] = idx.contiguous()
    ref = fp8_ref({n: v.numpy() if n not in ("x", "x_scale", "top_k_index", "top_k_weights") else v
                   for n, v in p.items()})
    g = to_gpu(p)
    poison = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    check_tol(run_fp8(g, out=poison), ref, FP8_TOL, "fp8 dropped")


def test_stage_recorder_times_every_kernel():
    """The stage-timing recorder sees each kernel of a call, in launch order."""
    moe = _moe()
    _say("stage recorder")
    p = wl.make_config("tiny")
    k = wl.CONFIGS["tiny"]["k"]
    g = to_gpu(p)
    moe.moe_profile_begin(2)
    moe.moe_experts_prefill(g["hidden"], g["gate_up"], g["down"], g["top_k_index"],
                            g["top_k_weights"], k)
    moe.moe_experts_decode(g["hidden"][:1], g["gate_up"], g["down"], g["top_k_index"][:1],
                           g["top_k_weights"][:1], k)
    moe.moe_experts_prefill(g["hidden"], g["gate_up"], g["down"], g["top_k_index"],
                            g["top_k_weights"], k)   # past max_calls: not recorded
    torch.cuda.synchronize()
    calls = moe.moe_profile_end(2)
    assert [s for s, _ in calls[0]] == ["plan", "gate_up", "down", "combine"]
    assert [s for s, _ in calls[1]] == ["decode"]
    assert all(ms > 0 for row in calls for _, ms in row)


# -------------------------------------------------- residual, bf16-input fp8


def _residual(T, H, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(T, H, generator=g).to(torch.bfloat16)


@pytest.mark.parametrize("entry,shape", [("moe_experts_prefill", (300, 256, 128, 6, 2)),
                                         ("moe_experts_decode", (1, 256, 128, 8, 4)),
                                         ("moe_experts_decode", (4, 512, 192, 8, 3)),
                                         ("moe_experts_decode", (7, 128, 64, 8, 2))])
def test_residual_bf16(entry, shape):
    """out = weighted sum + residual ([MPK] moe_local_reduction), on the grouped
    path, the decode form and the decode fallback to the grouped path."""
    moe = _moe()
    T, H, F, E, k = shape
    _say(f"residual {entry} {shape}")
    p = bf16_problem(T, H, F, E, k, seed=51 + T, std=1 / np.sqrt(H))
    r = _residual(T, H, 52 + T)
    ref = orc.moe_experts_reference_batched(f64(p["hidden"]), f64(p["gate_up"]), f64(p["down"]),
                                            p["top_k_index"].numpy(), f64(p["top_k_weights"]),
                                            residual=f64(r))
    g = to_gpu(p)
    out = getattr(moe, entry)(g["hidden"], g["gate_up"], g["down"], g["top_k_index"],
                              g["top_k_weights"], k, residual=r.cuda())
    check_tol(out, ref, BF16_TOL, f"{entry} {shape}")
    # all routing weights zero: the output is the residual, bit for bit
    z = getattr(moe, entry)(g["hidden"], g["gate_up"], g["down"], g["top_k_index"],
                            torch.zeros_like(g["top_k_weights"]), k, residual=r.cuda())
    assert torch.equal(z.cpu().view(torch.int16), r.view(torch.int16))


def test_residual_fp8():
    moe = _moe()
    T, H, F, E, k = 64, 256, 128, 8, 4
    _say("residual fp8")
    p = wl.make_fp8_problem(T, H, F, E, k, seed=53, routing="uniform_softmax", routed_scale=1.0)
    r = _residual(T, H, 54)
    ref = orc.moe_experts_fp8_reference(
        p["x"].numpy(), p["x_scale"].numpy(), p["gate_up"].numpy(), p["gate_up_scale"].numpy(),
        p["down"].numpy(), p["down_scale"].numpy(), p["top_k_index"].numpy(),
        p["top_k_weights"].numpy(), residual=f64(r))
    g = to_gpu(p)
    out = moe.moe_experts_fp8(g["x"], g["x_scale"], g["gate_up"], g["gate_up_scale"], g["down"],
                              g["down_scale"], g["top_k_index"], g["top_k_weights"], k,
                              residual=r.cuda())
    check_tol(out, ref, FP8_TOL, "fp8 residual")


@pytest.mark.parametrize("shape", [(64, 256, 128, 8, 4), (300, 512, 384, 6, 3), (3, 256, 128, 5, 2)])
def test_fp8_bf16in_medium(shape):
    """FP8 layer fed with bf16 hidden states (quantised per 128 block inside the
    call) against the oracle's bf16_to_fp8_quantize + fp8 layer; and bit-equal
    to quantising with moe_quantize_fp8_block128 and calling moe_experts_fp8."""
    moe = _moe()
    T, H, F, E, k = shape
    _say(f"fp8 bf16-in {shape}")
    p = wl.make_fp8_problem(T, H, F, E, k, seed=55 + T, routing="uniform_softmax", routed_scale=1.0)
    hidden = _residual(T, H, 56 + T)
    r = _residual(T, H, 57 + T) if T % 2 else None
    ref = orc.moe_experts_fp8_bf16_reference(
        f64(hidden), p["gate_up"].numpy(), p["gate_up_scale"].numpy(), p["down"].numpy(),
        p["down_scale"].numpy(), p["top_k_index"].numpy(), p["top_k_weights"].numpy(),
        residual=None if r is None else f64(r))
    g = to_gpu(p)
    rg = None if r is None else r.cuda()
    out = moe.moe_experts_fp8_bf16in(hidden.cuda(), g["gate_up"], g["gate_up_scale"], g["down"],
                                     g["down_scale"], g["top_k_index"], g["top_k_weights"], k,
                                     residual=rg)
    worst, rel = check_tol(out, ref, FP8_TOL, f"bf16-in {shape}")
    _say(f"  worst err/tol {worst:.3f} rel L2 {rel:.2e}")
    xq, xs = moe.moe_quantize_fp8_block128(hidden.cuda())
    two = moe.moe_experts_fp8(xq, xs, g["gate_up"], g["gate_up_scale"], g["down"], g["down_scale"],
                              g["top_k_index"], g["top_k_weights"], k, residual=rg)
    assert torch.equal(out.view(torch.int16), two.view(torch.int16))


def test_fp8_bf16in_full_config_every_row():
    """DeepSeek-V3-shaped decode batch (T=128, H=7168, F=2048, 128 experts,
    top-8) fed with bf16 N(0,1) hidden states: the quantised hidden states
    bit-exact against the oracle's block-128 quantiser, then every row of the
    layer against the expert-batched fp8 oracle on those codes."""
    moe = _moe()
    _say("fp8 bf16-in full v3_fp8_decode")
    p = wl.make_config("v3_fp8_decode", device="cuda")
    T, H = p["x"].shape
    k = p["top_k_index"].shape[1]
    E, F2, _ = p["gate_up"].shape
    hidden = _residual(T, H, 58).cuda()
    lay = moe.moe_workspace_layout(moe.MOE_VARIANT_FP8_BF16IN, T, H, F2 // 2, E, k)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    out = moe.moe_experts_fp8_bf16in(hidden, p["gate_up"], p["gate_up_scale"], p["down"],
                                     p["down_scale"], p["top_k_index"], p["top_k_weights"], k,
                                     workspace=ws)
    torch.cuda.synchronize()
    xq, xs = orc.quantize_block128_fp32(f64(hidden).astype(np.float32))
    q = dict(p)
    q["x"], q["x_scale"] = torch.from_numpy(xq), torch.from_numpy(xs)
    st = check_quantized_layer("fp8", out, q, ws, lay, "bf16-in full", orc)
    _say(f"  all rows: {st}")


# ------------------------------------------------------- shared experts

def _shared_problem(T, H, F, E, k, S, seed, std=0.02):
    p = bf16_problem(T, H, F, E, k, seed, std=std)
    p.update(wl.make_shared_experts(S, H, F, seed + 500, weight_std=std))
    return p


def _shared_ref(p, w=None, residual=None, batched=True):
    fn = orc.moe_experts_reference_batched if batched else orc.moe_experts_reference
    return fn(f64(p["hidden"]), f64(p["gate_up"]), f64(p["down"]), p["top_k_index"].numpy(),
              f64(p["top_k_weights"]) if w is None else w, residual=residual,
              shared_gate_up=f64(p["shared_gate_up"]), shared_down=f64(p["shared_down"]))


def _run_shared(entry, g, w=None, residual=None):
    return getattr(_moe(), entry)(g["hidden"], g["gate_up"], g["down"], g["shared_gate_up"],
                                  g["shared_down"], g["top_k_index"],
                                  g["top_k_weights"] if w is None else w,
                                  g["top_k_index"].shape[1], residual=residual)


@pytest.mark.parametrize("entry,shape", [
    ("moe_experts_prefill_shared", (300, 256, 128, 6, 2, 2)),
    ("moe_experts_prefill_shared", (520, 384, 192, 8, 3, 1)),   # 3 M tiles for each shared expert
    ("moe_experts_decode_shared", (1, 256, 128, 8, 2, 2)),
    ("moe_experts_decode_shared", (4, 384, 256, 16, 4, 3)),
    ("moe_experts_decode_shared", (40, 256, 128, 6, 2, 2)),      # grouped path under decode
])
def test_shared_experts(entry, shape):
    """Routed + always-on shared experts (weight 1) against the oracle."""
    T, H, F, E, k, S = shape
    _say(f"shared {entry} {shape}")
    p = _shared_problem(T, H, F, E, k, S, seed=61 + T, std=1 / np.sqrt(H))
    g = to_gpu(p)
    worst, rel = check_tol(_run_shared(entry, g), _shared_ref(p), BF16_TOL, f"{entry} {shape}")
    _say(f"  worst err/tol {worst:.3f} rel L2 {rel:.2e}")


@pytest.mark.parametrize("entry", ["moe_experts_prefill_shared", "moe_experts_decode_shared"])
def test_shared_experts_dropped_ids_zero_weights_residual(entry):
    """Routed ids E (one past the last routed expert) and -1 are dropped, never
    a shared expert; with zero routing weights only the shared experts and the
    residual remain."""
    T, H, F, E, k, S = (3, 256, 128, 8, 3, 2) if "decode" in entry else (200, 256, 128, 8, 3, 2)
    _say(f"shared dropped/zero/residual {entry}")
    p = _shared_problem(T, H, F, E, k, S, seed=71, std=1 / np.sqrt(H))
    idx = p["top_k_index"].clone()
    idx[:, 0] = E
    idx[::2, 1] = -1
    p["top_k_index"] = idx.contiguous()
    g = to_gpu(p)
    r = torch.randn(T, H, generator=torch.Generator().manual_seed(72)).to(torch.bfloat16)
    check_tol(_run_shared(entry, g, residual=r.cuda()), _shared_ref(p, residual=f64(r)), BF16_TOL,
              "dropped + residual")
    zw = torch.zeros_like(g["top_k_weights"])
    check_tol(_run_shared(entry, g, w=zw), _shared_ref(p, w=np.zeros((T, k))), BF16_TOL,
              "zero routing weights")


@pytest.mark.parametrize("name", ["ocr2_decode_t1_shared", "ocr2_prefill_shared"])
def test_shared_full_config(name):
    """The OCR-2 workloads with their two shared experts, every token."""
    _say(f"shared full {name}")
    p = wl.make_config(name)
    g = to_gpu(p)
    entry = "moe_experts_decode_shared" if "decode" in name else "moe_experts_prefill_shared"
    out = _run_shared(entry, g)
    check_tol(out, _shared_ref(p, batched=True), BF16_TOL, name)


# ---------------------------------------- shared experts, quantised layers

def _augment(p, S, w=None):
    """The problem with the S shared experts (the last S of p's experts)
    written as the definition reads: extra experts E .. E+S-1 that every token
    passes through with weight 1, after its routed slots."""
    idx = p["top_k_index"].numpy()
    T = idx.shape[0]
    E = p["gate_up"].shape[0] - S
    wts = p["top_k_weights"].numpy() if w is None else w
    idx_a = np.concatenate([np.where((idx >= 0) & (idx < E), idx, -1),
                            np.tile(np.arange(E, E + S), (T, 1))], axis=1)
    w_a = np.concatenate([wts, np.ones((T, S))], axis=1)
    return idx_a, w_a


def _split_shared(p, S, names):
    """Routed part (first E experts) and shared part (last S) of p's weights."""
    routed = {n: p[n][:-S].contiguous() for n in names}
    shared = tuple(p[n][-S:].contiguous() for n in names)
    return routed, shared


_FP8_W = ("gate_up", "gate_up_scale", "down", "down_scale")


# (T, H, F, E, k, S): grouped tiles; a decode batch (32-row tiles, 512-row
# panels); several M tiles per shared expert
@pytest.mark.parametrize("shape", [(300, 512, 256, 6, 2, 2), (48, 512, 256, 16, 4, 1),
                                   (520, 256, 384, 4, 2, 1)])
def test_fp8_shared_experts(shape):
    """FP8 layer + shared experts in the routed format, against the oracle of
    the same layer with the shared experts as weight-1 slots; with a residual,
    dropped ids (E, -1: never a shared expert) and all-zero routing weights."""
    T, H, F, E, k, S = shape
    _say(f"fp8 shared {shape}")
    p = wl.make_fp8_problem(T, H, F, E + S, k, seed=91 + T, routing="uniform_softmax",
                            routed_scale=1.0)
    g = torch.Generator().manual_seed(92 + T)
    p["top_k_index"], p["top_k_weights"] = wl.route_uniform_softmax(T, E, k, g, "cpu", 1.0)
    idx = p["top_k_index"].clone()
    idx[::5, 0] = E
    idx[1::7, k - 1] = -1
    p["top_k_index"] = idx.contiguous()
    routed, shared = _split_shared(p, S, _FP8_W)
    r = torch.randn(T, H, generator=g).to(torch.bfloat16)
    moe = _moe()
    for w in (None, np.zeros((T, k))):
        idx_a, w_a = _augment(p, S, w)
        ref = orc.moe_experts_fp8_reference_batched(
            p["x"].numpy(), p["x_scale"].numpy(), p["gate_up"].numpy(), p["gate_up_scale"].numpy(),
            p["down"].numpy(), p["down_scale"].numpy(), idx_a, w_a, residual=f64(r))
        wt = p["top_k_weights"] if w is None else torch.zeros(T, k)
        out = moe.moe_experts_fp8_shared(
            p["x"].cuda(), p["x_scale"].cuda(), *[routed[n].cuda() for n in _FP8_W],
            *[t.cuda() for t in shared], idx.cuda(), wt.float().cuda(), k, residual=r.cuda())
        worst, rel = check_tol(out, ref, FP8_TOL, f"fp8 shared {shape}")
        _say(f"  worst err/tol {worst:.3f} rel L2 {rel:.2e}")
