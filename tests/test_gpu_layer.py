"""GPU parity of the one-launch layers (moe_experts_prefill_fused for bf16,
moe_experts_fp8_fused): the routing plan, gate_up, down and the combine in
one persistent launch.

The one-launch form performs the same arithmetic as the stage-by-stage form
(moe_experts_prefill, itself checked on every element against the oracle in
test_gpu_parity.py), so its output must equal that form's bit for bit; it is
also compared with the float64 oracle directly at the bf16 bar
|gpu - ref| <= 1e-2 + 1e-2 |ref|.  The hand-offs between workgroups are
exercised with small persistent grids (many items per workgroup, down items
waiting for gate_up items), repeated calls on one workspace (the generation
stamps) and a workspace full of stale bytes.
"""

import sys

import numpy as np
import pytest
import torch

import moe_workloads as wl
from oracle import moe_oracle as orc

pytestmark = pytest.mark.gpu

BF16_TOL = (1e-2, 1e-2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_routed_amd as moe
    moe._load()
    yield
    moe.moe_set_grid_cap(0)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _moe():
    import mixture_experts_routed_amd as moe
    return moe


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_tol(gpu, ref, what):
    atol, rtol = BF16_TOL
    g = f64(gpu)
    err = np.abs(g - ref)
    worst = float(np.max(err / (atol + rtol * np.abs(ref)))) if err.size else 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    assert worst <= 1.0, f"{what}: worst err/tol {worst:.3f}"


def problem(T, H, F, E, k, seed, device="cuda"):
    return wl.make_bf16_problem(T, H, F, E, k, seed, device)


def oracle(p):
    return orc.moe_experts_reference_batched(f64(p["hidden"]), f64(p["gate_up"]), f64(p["down"]),
                                             p["top_k_index"].cpu().numpy(),
                                             f64(p["top_k_weights"]))


def run(entry, p, residual=None, workspace=None, out=None):
    fn = getattr(_moe(), entry)
    return fn(p["hidden"], p["gate_up"], p["down"], p["top_k_index"], p["top_k_weights"],
              p["top_k_index"].shape[1], residual=residual, workspace=workspace, out=out)


def same_bits(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{what}: bits differ"


# (T, H, F, E, k): one or a few M tiles per expert; experts with more than
# 256 rows (several M tiles); H % 256 != 0 (128-wide down panels); more
# experts than rows; a ragged tail everywhere
SHAPES = [(16, 128, 128, 8, 2), (300, 256, 384, 12, 3), (200, 384, 256, 8, 2),
          (1500, 256, 256, 4, 3), (90, 512, 128, 64, 6), (777, 640, 384, 16, 4)]


@pytest.mark.parametrize("shape", SHAPES)
def test_layer_matches_oracle_and_stage_form(shape):
    T, H, F, E, k = shape
    _say(f"one-launch layer {shape}")
    p = problem(T, H, F, E, k, seed=100 + T)
    got = run("moe_experts_prefill_fused", p)
    same_bits(got, run("moe_experts_prefill", p), str(shape))
    check_tol(got, oracle(p), str(shape))


@pytest.mark.parametrize("cap", [8, 16, 40])
def test_layer_small_grids(cap):
    """Few workgroups: each runs many gate_up and down items, and down items
    wait for gate_up items held by other workgroups."""
    moe = _moe()
    _say(f"one-launch layer, grid cap {cap}")
    p = problem(1200, 256, 384, 10, 3, seed=7)
    ref = run("moe_experts_prefill", p)
    moe.moe_set_grid_cap(cap)
    try:
        got = run("moe_experts_prefill_fused", p)
        torch.cuda.synchronize()
    finally:
        moe.moe_set_grid_cap(0)
    same_bits(got, ref, f"cap {cap}")


def test_layer_repeated_calls_and_stale_workspace():
    """Consecutive calls on one workspace (each stamps its own flags), the
    first one on a workspace full of stale bytes, inputs changing between
    calls."""
    moe = _moe()
    _say("one-launch layer, repeated calls")
    T, H, F, E, k = 400, 256, 256, 8, 2
    n = moe.moe_workspace_size(moe.MOE_VARIANT_PREFILL, T, H, F, E, k)
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    for i in range(5):
        p = problem(T, H, F, E, k, seed=300 + i)
        got = run("moe_experts_prefill_fused", p, workspace=ws)
        same_bits(got, run("moe_experts_prefill", p), f"call {i}")


def test_layer_residual_dropped_slots_and_poisoned_out():
    _say("one-launch layer, residual and dropped slots")
    T, H, F, E, k = 257, 256, 128, 8, 3
    p = problem(T, H, F, E, k, seed=11)
    idx = p["top_k_index"].clone()
    idx[::5, 0] = -1        # dropped
    idx[::7, 1] = E + 3     # out of range: dropped
    p["top_k_index"] = idx
    res = torch.randn(T, H, device="cuda").to(torch.bfloat16)
    poison = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = run("moe_experts_prefill_fused", p, residual=res, out=poison)
    same_bits(got, run("moe_experts_prefill", p, residual=res), "residual")
    check_tol(got, oracle(p) + f64(res), "residual")


def test_layer_full_ocr2_prefill():
    """T=2048, H=1280, F=896, 64 experts, top-6: equal to the stage-by-stage
    form (checked on every element against the oracle elsewhere), and a few
    rows against the oracle directly."""
    _say("one-launch layer, full ocr2_prefill")
    p = wl.make_config("ocr2_prefill", device="cuda")
    got = run("moe_experts_prefill_fused", p)
    same_bits(got, run("moe_experts_prefill", p), "ocr2_prefill")
    rows = [0, 1, 777, 2047]
    sub = {n: (v[rows] if n in ("hidden", "top_k_index", "top_k_weights") else v)
           for n, v in p.items()}
    check_tol(got[rows], oracle(sub), "ocr2_prefill rows")


def test_layer_other_shapes_take_the_stage_form():
    """H not a multiple of 128: the entry point runs the stage-by-stage form."""
    moe = _moe()
    _say("one-launch layer, fallback shape")
    p = problem(64, 192, 128, 4, 2, seed=5)
    moe.moe_profile_begin(1)
    got = run("moe_experts_prefill_fused", p)
    torch.cuda.synchronize()
    calls = moe.moe_profile_end(1)
    assert [s for s, _ in calls[0]] == ["plan", "gate_up", "down", "combine"]
    same_bits(got, run("moe_experts_prefill", p), "fallback")


def test_layer_stage_recorder_and_empty_call():
    moe = _moe()
    p = problem(64, 256, 128, 4, 2, seed=6)
    moe.moe_profile_begin(1)
    run("moe_experts_prefill_fused", p)
    torch.cuda.synchronize()
    calls = moe.moe_profile_end(1)
    assert [s for s, _ in calls[0]] == ["layer"]
    empty = {n: v[:0] if n in ("hidden", "top_k_index", "top_k_weights") else v
             for n, v in p.items()}
    assert run("moe_experts_prefill_fused", empty).shape == (0, 256)


# ------------------------------------------------------------ fp8 layer

FP8_TOL = (3e-2, 3e-2)


def run_fp8(entry, g, workspace=None):
    fn = getattr(_moe(), entry)
    return fn(g["x"], g["x_scale"], g["gate_up"], g["gate_up_scale"], g["down"], g["down_scale"],
              g["top_k_index"], g["top_k_weights"], g["top_k_index"].shape[1], workspace=workspace)


def fp8_oracle(p):
    c = {n: v.cpu() for n, v in p.items()}
    return orc.moe_experts_fp8_reference(
        c["x"].numpy(), c["x_scale"].numpy(), c["gate_up"].numpy(), c["gate_up_scale"].numpy(),
        c["down"].numpy(), c["down_scale"].numpy(), c["top_k_index"].numpy(),
        c["top_k_weights"].numpy())


def check_fp8_tol(gpu, ref, what):
    atol, rtol = FP8_TOL
    g = f64(gpu)
    worst = float(np.max(np.abs(g - ref) / (atol + rtol * np.abs(ref)))) if g.size else 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    assert worst <= 1.0, f"{what}: worst err/tol {worst:.3f}"


# (T, H, F, E, k): H and F multiples of 512, more than 32 slots per expert
FP8_SHAPES = [(600, 512, 512, 6, 3), (1000, 1024, 512, 12, 2), (400, 512, 1024, 3, 2),
              (333, 512, 512, 16, 4)]


@pytest.mark.parametrize("shape", FP8_SHAPES)
def test_fp8_layer_matches_oracle_and_stage_form(shape):
    T, H, F, E, k = shape
    _say(f"one-launch fp8 layer {shape}")
    p = wl.make_fp8_problem(T, H, F, E, k, seed=200 + T, routing="uniform_softmax",
                            routed_scale=1.0)
    g = {n: v.cuda() for n, v in p.items()}
    got = run_fp8("moe_experts_fp8_fused", g)
    same_bits(got, run_fp8("moe_experts_fp8", g), str(shape))
    check_fp8_tol(got, fp8_oracle(p), str(shape))


@pytest.mark.parametrize("cap", [8, 24])
def test_fp8_layer_small_grids(cap):
    moe = _moe()
    _say(f"one-launch fp8 layer, grid cap {cap}")
    p = wl.make_fp8_problem(900, 512, 512, 5, 2, seed=9, routing="uniform_softmax",
                            routed_scale=1.0)
    g = {n: v.cuda() for n, v in p.items()}
    ref = run_fp8("moe_experts_fp8", g)
    moe.moe_set_grid_cap(cap)
    try:
        got = run_fp8("moe_experts_fp8_fused", g)
        torch.cuda.synchronize()
    finally:
        moe.moe_set_grid_cap(0)
    same_bits(got, ref, f"cap {cap}")


def test_fp8_layer_repeated_calls_stale_workspace_and_stages():
    moe = _moe()
    _say("one-launch fp8 layer, repeated calls")
    T, H, F, E, k = 500, 512, 512, 4, 2
    n = moe.moe_workspace_size(moe.MOE_VARIANT_FP8, T, H, F, E, k)
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    for i in range(4):
        p = wl.make_fp8_problem(T, H, F, E, k, seed=400 + i, routing="uniform_softmax",
                                routed_scale=1.0)
        g = {n_: v.cuda() for n_, v in p.items()}
        if i == 3:
            moe.moe_profile_begin(1)
        got = run_fp8("moe_experts_fp8_fused", g, workspace=ws)
        torch.cuda.synchronize()
        if i == 3:
            assert [s for s, _ in moe.moe_profile_end(1)[0]] == ["layer"]
        same_bits(got, run_fp8("moe_experts_fp8", g), f"call {i}")


def test_fp8_layer_decode_batch_takes_the_stage_form():
    """At most 32 slots per expert (32-row tiles): the stage-by-stage form."""
    moe = _moe()
    p = wl.make_fp8_problem(64, 512, 512, 16, 4, seed=3, routing="uniform_softmax",
                            routed_scale=1.0)
    g = {n: v.cuda() for n, v in p.items()}
    moe.moe_profile_begin(1)
    got = run_fp8("moe_experts_fp8_fused", g)
    torch.cuda.synchronize()
    assert [s for s, _ in moe.moe_profile_end(1)[0]] == ["plan", "gate_up", "down", "combine"]
    same_bits(got, run_fp8("moe_experts_fp8", g), "decode batch")


def test_fp8_layer_full_v3_prefill():
    """T=4096 Zipf-routed DeepSeek-V3 expert share: equal to the
    stage-by-stage form (checked on every element against the oracle
    elsewhere)."""
    _say("one-launch fp8 layer, full v3_fp8_prefill")
    p = wl.make_config("v3_fp8_prefill", device="cuda")
    same_bits(run_fp8("moe_experts_fp8_fused", p), run_fp8("moe_experts_fp8", p), "v3_fp8_prefill")


# ------------------------------------------------- the plan inside the launch


def _ws_i32(ws, off, n):
    return ws[off:off + 4 * n].view(torch.int32).cpu().numpy()


# (T, k, E, ids): the plan phase's chunks hold a few slots (T*k < 64 chunks
# too), many slots, every expert id up to 512 experts, and dropped ids
@pytest.mark.parametrize("case", [(5, 2, 8, "uniform"), (300, 3, 12, "uniform"),
                                  (2048, 6, 64, "uniform"), (4096, 8, 512, "skewed"),
                                  (777, 4, 16, "dropped")])
def test_layer_plan_arrays_match_oracle(case):
    """The plan arrays the one-launch layer writes into its workspace are the
    oracle's, bit for bit."""
    moe = _moe()
    T, k, E, kind = case
    _say(f"one-launch layer plan {case}")
    H, F = 128, 128
    p = problem(T, H, F, E, k, seed=900 + T)
    idx = p["top_k_index"].clone()
    if kind == "skewed":
        g = torch.Generator().manual_seed(5)
        idx = (torch.rand(T, k, generator=g) ** 3 * E).to(torch.int32).cuda()
    elif kind == "dropped":
        idx[::3, 0] = -1
        idx[::5, 1] = E + 7
    p["top_k_index"] = idx.contiguous()
    lay = moe.moe_workspace_layout(moe.MOE_VARIANT_PREFILL, T, H, F, E, k)
    ws = torch.full((lay["total"],), 0xEE, dtype=torch.uint8, device="cuda")
    run("moe_experts_prefill_fused", p, workspace=ws)
    torch.cuda.synchronize()
    ref = orc.routing_plan(p["top_k_index"].cpu().numpy(), E)
    P = T * k
    got = (_ws_i32(ws, lay["counts"], E), _ws_i32(ws, lay["offsets"], E + 1),
           _ws_i32(ws, lay["perm"], P), _ws_i32(ws, lay["inv"], P))
    for name, a, r in zip(("counts", "offsets", "perm", "inv"), got, ref):
        assert np.array_equal(a, r), f"plan {name} differs"


# ----------------------------------------------------------- MXFP4 layer

def _mx_helpers():
    import test_gpu_mxfp4 as tm
    return tm


def run_mx(entry, g, workspace=None):
    fn = getattr(_moe(), entry)
    return fn(g["x"], g["x_scale"], g["gate_up"], g["gate_up_scale"], g["down"], g["down_scale"],
              g["top_k_index"], g["top_k_weights"], g["top_k_index"].shape[1], workspace=workspace)


# (T, H, F, E, k): more than 64 slots per expert (the wide tiles), F % 256,
# H % 512
MX_SHAPES = [(600, 512, 256, 4, 2), (1000, 1024, 512, 6, 3), (700, 512, 768, 3, 2)]


@pytest.mark.parametrize("shape", MX_SHAPES)
def test_mx_layer_matches_oracle_and_stage_form(shape):
    tm = _mx_helpers()
    T, H, F, E, k = shape
    _say(f"one-launch MXFP4 layer {shape}")
    p = tm.mx_problem(T, H, F, E, k, seed=60 + T, block_spread=2)
    g = {n: v.cuda() for n, v in p.items()}
    got = run_mx("moe_experts_mxfp4_fused", g)
    same_bits(got, run_mx("moe_experts_mxfp4", g), str(shape))
    check_fp8_tol(got, tm.mx_ref(g), str(shape))


def test_mx_layer_small_grid_repeated_calls_and_stages():
    moe = _moe()
    tm = _mx_helpers()
    _say("one-launch MXFP4 layer, small grid, repeated calls")
    T, H, F, E, k = 800, 512, 512, 4, 2
    n = moe.moe_workspace_size(moe.MOE_VARIANT_MXFP4, T, H, F, E, k)
    ws = torch.full((n,), 0x3C, dtype=torch.uint8, device="cuda")
    for i, cap in enumerate((16, 0, 0)):
        p = tm.mx_problem(T, H, F, E, k, seed=70 + i)
        g = {n_: v.cuda() for n_, v in p.items()}
        ref = run_mx("moe_experts_mxfp4", g)
        moe.moe_set_grid_cap(cap)
        try:
            if i == 2:
                moe.moe_profile_begin(1)
            got = run_mx("moe_experts_mxfp4_fused", g, workspace=ws)
            torch.cuda.synchronize()
            if i == 2:
                assert [s for s, _ in moe.moe_profile_end(1)[0]] == ["layer"]
        finally:
            moe.moe_set_grid_cap(0)
        same_bits(got, ref, f"call {i}")


def test_mx_layer_full_v3_prefill():
    """T=4096 Zipf-routed expert share with MXFP4 weights: equal to the
    stage-by-stage form."""
    _say("one-launch MXFP4 layer, full v3_mxfp4_prefill")
    p = wl.make_config("v3_mxfp4_prefill", device="cuda")
    same_bits(run_mx("moe_experts_mxfp4_fused", p), run_mx("moe_experts_mxfp4", p), "v3_mxfp4_prefill")
