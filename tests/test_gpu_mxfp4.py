"""GPU parity of the MXFP4-weight / MXFP8-activation layer (moe_experts_mxfp4)
against the float64 oracle that decodes the same E2M1 / E4M3 codes and E8M0
scales and re-quantises h to MXFP8 in fp32 as the method does.

Bar: |gpu - ref| <= 3e-2 + 3e-2 |ref| per element, the fp8 bar (the
arithmetic is fp32 accumulation of exactly decoded operands, as on the fp8
path; the only extra error source is the same one: fp32 h next to the
oracle's float64 h before the MXFP8 re-quantisation).  Medium cases draw
weights with std 1/sqrt(K), so outputs are O(1) and the relative term binds.
"""

import sys

import numpy as np
import pytest
import torch

import moe_workloads as wl
from oracle import moe_oracle as orc
from oracle_runner import check_quantized_layer

pytestmark = pytest.mark.gpu

MX_TOL = (3e-2, 3e-2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_routed_amd as moe
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
    worst = float(np.max(err / (atol + rtol * np.abs(ref)))) if err.size else 0.0
    rel_l2 = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30))
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    assert worst <= 1.0, f"{what}: worst err/tol {worst:.3f}, rel L2 {rel_l2:.2e}"
    return worst, rel_l2


class _HostExperts:
    """Lazy host copies of the experts of a device weight tensor."""

    def __init__(self, t):
        self.t, self.cache, self.shape = t, {}, tuple(t.shape)

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.t[e].cpu().numpy()
        return self.cache[e]


def mx_ref(p, tokens=None, residual=None):
    def host(n):
        v = p[n]
        return v.cpu().numpy() if n in ("x", "x_scale", "top_k_index", "top_k_weights") else _HostExperts(v)
    return orc.moe_experts_mxfp4_reference(
        host("x"), host("x_scale"), host("gate_up"), host("gate_up_scale"), host("down"),
        host("down_scale"), host("top_k_index"), host("top_k_weights"), tokens=tokens,
        residual=residual)


def run_mx(g, out=None, residual=None, workspace=None):
    return _moe().moe_experts_mxfp4(g["x"], g["x_scale"], g["gate_up"], g["gate_up_scale"],
                                    g["down"], g["down_scale"], g["top_k_index"],
                                    g["top_k_weights"], g["top_k_index"].shape[1], out=out,
                                    residual=residual, workspace=workspace)


def mx_problem(T, H, F, E, k, seed, block_spread=0):
    """Medium problem with O(1) outputs.  block_spread > 0 multiplies every
    32-wide block of the weight and activation sources by 2^u, u uniform in
    [-block_spread, block_spread], so neighbouring blocks carry very different
    E8M0 scales (a scale applied to the wrong block then shows at once), and
    divides by the RMS of 2^u so that outputs stay O(1): the layer stores each
    slot's y in bf16, so an output that cancels between slots of size M is
    only known to about M * 2^-9, which must stay under the 3e-2 floor."""
    g = torch.Generator().manual_seed(seed)
    us = np.arange(-block_spread, block_spread + 1)
    norm = float(np.sqrt(np.mean(4.0 ** us)))

    def spread(t):
        if not block_spread:
            return t
        K = t.shape[-1]
        u = torch.randint(-block_spread, block_spread + 1, t.shape[:-1] + (K // 32, 1), generator=g)
        return (t.reshape(*t.shape[:-1], K // 32, 32) * (torch.exp2(u.float()) / norm)).reshape(t.shape)

    p = {}
    w13 = spread(torch.randn(E, 2 * F, H, generator=g) / np.sqrt(H))
    w2 = spread(torch.randn(E, H, F, generator=g) / np.sqrt(F))
    p["gate_up"], p["gate_up_scale"] = wl.quantize_mxfp4_rows_torch(w13)
    p["down"], p["down_scale"] = wl.quantize_mxfp4_rows_torch(w2)
    x = spread(torch.randn(T, H, generator=g))
    p["x"], p["x_scale"] = wl.quantize_mxfp8_rows_torch(x)
    p["top_k_index"], p["top_k_weights"] = wl.route_uniform_softmax(T, E, k, g, "cpu", 1.0)
    return p


def to_gpu(p):
    return {n: v.cuda() for n, v in p.items()}


# (T, H, F, E, k): several M tiles and a ragged last one, gate_up h tiles of
# 128, down panels of 256 (H % 256 == 0) and 128 (H = 128, 384), one or many
# 128-K steps, and an odd number of them (H = 384: 3 steps)
SHAPES = [(300, 512, 384, 6, 3), (64, 256, 128, 8, 4), (520, 128, 256, 2, 2),
          (600, 256, 128, 4, 2), (700, 512, 256, 3, 2), (257, 384, 640, 5, 2),
          # decode-batch shapes (at most 32 slots per expert on average, F % 256
          # == 0, H % 512 == 0): 32-row tiles and 512-row panels; the second has
          # experts with more than 32 rows (several tiles) and some with none
          (40, 512, 256, 8, 2), (100, 1024, 512, 16, 4), (9, 1536, 768, 32, 3),
          # more than 64 rows per expert with F % 256 == 0 and H % 512 == 0:
          # the 128 x 512 tiles (ragged last M tile, three h tiles)
          (900, 1024, 768, 5, 2)]


@pytest.mark.parametrize("shape", SHAPES)
def test_mxfp4_medium(shape):
    T, H, F, E, k = shape
    _say(f"mxfp4 medium {shape}")
    p = mx_problem(T, H, F, E, k, seed=61 + T)
    ref = mx_ref(p)
    worst, rel = check_tol(run_mx(to_gpu(p)), ref, MX_TOL, str(shape))
    _say(f"  worst err/tol {worst:.3f} rel L2 {rel:.2e}")


@pytest.mark.parametrize("shape", [(300, 512, 384, 6, 3), (257, 384, 640, 5, 2), (600, 1024, 512, 4, 2)])
def test_mxfp4_block_scales_spread(shape):
    """Every 32-block of weights and activations scaled by 2^u, u in [-4, 4]
    (neighbouring E8M0 bytes up to 2^8 apart): each scale byte must meet its
    own 32 K elements."""
    T, H, F, E, k = shape
    _say(f"mxfp4 spread scales {shape}")
    p = mx_problem(T, H, F, E, k, seed=71 + T, block_spread=4)
    ref = mx_ref(p)
    worst, rel = check_tol(run_mx(to_gpu(p)), ref, MX_TOL, str(shape))
    _say(f"  worst err/tol {worst:.3f} rel L2 {rel:.2e}")


@pytest.mark.parametrize("shape", [(200, 256, 256, 4, 2), (512, 384, 384, 4, 2), (60, 512, 256, 8, 2),
                                   (520, 512, 256, 2, 2)])
def test_mxfp4_h_stage_codes(shape):
    """The MXFP8 h in the workspace against the oracle's fp32 rule applied to
    the oracle's h.  The kernel quantises its fp32-accumulated h; the scale
    byte can differ by one only where a block maximum sits at a power of two
    within fp32 rounding, and codes may flip by one e4m3 step at rounding
    boundaries, both rarely."""
    moe = _moe()
    T, H, F, E, k = shape
    _say(f"mxfp4 h stage {shape}")
    p = mx_problem(T, H, F, E, k, seed=43)
    g = to_gpu(p)
    lay = moe.moe_workspace_layout(moe.MOE_VARIANT_MXFP4, T, H, F, E, k)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    run_mx(g, workspace=ws)
    torch.cuda.synchronize()
    P = T * k
    perm = ws[lay["perm"]:lay["perm"] + 4 * P].view(torch.int32).cpu().numpy()
    hq = ws[lay["h"]:lay["h"] + P * F].cpu().numpy().reshape(P, F)
    hs = ws[lay["h_scale"]:lay["h_scale"] + P * (F // 32)].cpu().numpy().reshape(P, F // 32)
    x = orc.dequantize_mx(orc.e4m3fn_decode(p["x"].numpy()), p["x_scale"].numpy())
    idx = p["top_k_index"].numpy().reshape(-1)
    h_ref = np.zeros((P, F), np.float32)
    W = {}
    for m in range(P):
        s = perm[m]
        e = int(idx[s])
        if e not in W:
            W[e] = orc.dequantize_mx(orc.e2m1_decode(orc.unpack_e2m1(p["gate_up"][e].numpy())),
                                     p["gate_up_scale"][e].numpy())
        gv = W[e] @ x[s // k]
        h_ref[m] = (orc.silu(gv[:F]) * gv[F:]).astype(np.float32)
    q_ref, s_ref = orc.quantize_mxfp8_fp32(h_ref)
    sdiff = hs.astype(np.int64) - s_ref.astype(np.int64)
    assert np.all(np.abs(sdiff) <= 1) and np.mean(sdiff != 0) < 1e-3, np.mean(sdiff != 0)
    same = np.repeat(sdiff == 0, 32, axis=1)
    diff = (hq != q_ref) & same
    assert diff.mean() < 2e-3, diff.mean()
    a, b = orc.e4m3fn_decode(hq[diff]), orc.e4m3fn_decode(q_ref[diff])
    assert np.all(np.abs(a - b) <= np.maximum(np.abs(a), np.abs(b)) * 2.0 ** -3 + 448e-4)
    # dequantised values agree everywhere (also where the scale byte moved)
    hv = orc.dequantize_mx(orc.e4m3fn_decode(hq), hs)
    rv = orc.dequantize_mx(orc.e4m3fn_decode(q_ref), s_ref)
    blk_max = np.repeat(np.max(np.abs(rv).reshape(P, F // 32, 32), axis=2), 32, axis=1)
    assert np.all(np.abs(hv - rv) <= np.abs(rv) * 2.0 ** -3 + blk_max * 1e-3)


@pytest.mark.parametrize("shape", [(100, 256, 128, 4, 3), (400, 384, 256, 4, 3), (50, 512, 256, 8, 3),
                                   (300, 512, 256, 3, 3)])
def test_mxfp4_overwrite_and_dropped(shape):
    """Dropped slots (ids -1 and E) contribute nothing and every output
    element is written (a NaN-filled out buffer)."""
    T, H, F, E, k = shape
    _say(f"mxfp4 overwrite + dropped {shape}")
    p = mx_problem(T, H, F, E, k, seed=5)
    idx = p["top_k_index"].clone()
    idx[::3, 1] = -1
    idx[1::5, 2] = E
    p["top_k_index"] = idx.contiguous()
    ref = mx_ref(p)
    poison = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    check_tol(run_mx(to_gpu(p), out=poison), ref, MX_TOL, "mxfp4 dropped")


def test_mxfp4_residual_and_zero_weights():
    T, H, F, E, k = 150, 256, 256, 4, 2
    _say("mxfp4 residual + zero weights")
    p = mx_problem(T, H, F, E, k, seed=9)
    res = (torch.randn(T, H, generator=torch.Generator().manual_seed(3))).to(torch.bfloat16)
    ref = mx_ref(p, residual=f64(res))
    g = to_gpu(p)
    check_tol(run_mx(g, residual=res.cuda()), ref, MX_TOL, "mxfp4 residual")
    g["top_k_weights"] = torch.zeros_like(g["top_k_weights"])
    assert run_mx(g).abs().sum().item() == 0


def test_mxfp4_zero_tokens():
    p = to_gpu(mx_problem(4, 128, 128, 2, 1, seed=1))
    q = {n: v[:0] if n in ("x", "x_scale", "top_k_index", "top_k_weights") else v for n, v in p.items()}
    assert run_mx(q).shape == (0, 128)


def _run_mx_ws(moe, g):
    T, H = g["x"].shape
    E, F2, _ = g["gate_up"].shape
    k = g["top_k_index"].shape[1]
    lay = moe.moe_workspace_layout(moe.MOE_VARIANT_MXFP4, T, H, F2 // 2, E, k)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    out = run_mx(g, workspace=ws)
    torch.cuda.synchronize()
    return out, ws, lay


@pytest.mark.parametrize("name", ["v3_mxfp4_decode", "v3_mxfp4_prefill"])
def test_mxfp4_full_config_every_row(name):
    """The V3 expert-share shapes with MXFP4 weights: every output element
    against the expert-batched oracle (pinned to the per-slot form on the
    CPU), after checking that each MXFP8 code and scale byte of h the kernel
    chose is a rounding of the oracle's h; a second call is bit-identical."""
    moe = _moe()
    _say(f"mxfp4 full {name}")
    p = wl.make_config(name, device="cuda")
    out, ws, lay = _run_mx_ws(moe, p)
    st = check_quantized_layer("mxfp4", out, p, ws, lay, name, orc)
    idx = p["top_k_index"].cpu().numpy()
    counts = np.bincount(idx.reshape(-1), minlength=p["gate_up"].shape[0])
    _say(f"  all {out.shape[0]} rows: {st}; max/mean load {counts.max() / counts.mean():.1f}, "
         f"empty {(counts == 0).sum()}")
    b = run_mx(p)
    assert torch.equal(out.view(torch.int16), b.view(torch.int16)), "mxfp4 path not deterministic"


# the persistent grid capped at 8 workgroups: many items per workgroup on the
# 128 x 256 tiles, the 32-row decode-batch tiles and the 128 x 512 wide tiles;
# the capped call equals the uncapped one bit for bit, and that one the oracle
@pytest.mark.parametrize("shape", [(600, 256, 128, 4, 2), (100, 1024, 512, 16, 4),
                                   (900, 1024, 768, 5, 2)])
def test_mxfp4_many_items_per_workgroup(shape):
    moe = _moe()
    T, H, F, E, k = shape
    _say(f"mxfp4 capped grid {shape}")
    g = to_gpu(mx_problem(T, H, F, E, k, seed=91 + T))
    out, ws, lay = _run_mx_ws(moe, g)
    moe.moe_set_grid_cap(8)
    try:
        capped = run_mx(g)
        torch.cuda.synchronize()
    finally:
        moe.moe_set_grid_cap(0)
    assert torch.equal(out.view(torch.int16), capped.view(torch.int16)), "grid-dependent result"
    st = check_quantized_layer("mxfp4", out, g, ws, lay, str(shape), orc)
    _say(f"  {st}")


@pytest.mark.parametrize("shape", [(96, 256, 256, 4, 2), (40, 512, 512, 8, 2), (300, 1024, 512, 2, 2)])
def test_mxfp4_h_stage_exact(shape):
    """Small integers (E4M3 activations 1 or 2, E2M1 weights in {0, +-1, +-2},
    unit E8M0 scales): the fp32 sums are exact, every gate dot product is at
    least 20 (silu(g) = g in fp32), so h = g_gate * g_up is an exact integer
    and the epilogue's MXFP8 codes and scale bytes must equal the oracle's
    rule bit for bit (128 x 256 tiles, decode-batch tiles, wide tiles)."""
    moe = _moe()
    T, H, F, E, k = shape
    _say(f"mxfp4 exact h stage {shape}")
    rng = np.random.default_rng(19)
    x = rng.integers(1, 3, size=(T, H)).astype(np.float64)
    gate = (rng.random((E, F, H)) < 0.3).astype(np.float64)
    gate[..., :20] = 1.0
    up = rng.integers(-2, 3, size=(E, F, H)).astype(np.float64)
    down = rng.integers(-2, 3, size=(E, H, F)).astype(np.float64)

    def pack(v):   # E2M1 codes, element 2i in the low nibble
        c = orc.e2m1_encode(v)
        return torch.from_numpy((c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8))

    e8 = lambda *s: torch.full(s, 127, dtype=torch.uint8)
    idx, w = wl.route_uniform_softmax(T, E, k, torch.Generator().manual_seed(6), "cpu", 1.0)
    g = {"x": torch.from_numpy(orc.e4m3fn_encode(x)), "x_scale": e8(T, H // 32),
         "gate_up": pack(np.concatenate([gate, up], axis=1)), "gate_up_scale": e8(E, 2 * F, H // 32),
         "down": pack(down), "down_scale": e8(E, H, F // 32),
         "top_k_index": idx, "top_k_weights": w}
    g = to_gpu(g)
    lay = moe.moe_workspace_layout(moe.MOE_VARIANT_MXFP4, T, H, F, E, k)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    run_mx(g, workspace=ws)
    torch.cuda.synchronize()
    P = T * k
    perm = ws[lay["perm"]:lay["perm"] + 4 * P].view(torch.int32).cpu().numpy()
    hq = ws[lay["h"]:lay["h"] + P * F].cpu().numpy().reshape(P, F)
    hs = ws[lay["h_scale"]:lay["h_scale"] + P * (F // 32)].cpu().numpy().reshape(P, F // 32)
    ids = idx.numpy().reshape(-1)
    h = np.stack([(gate[ids[s]] @ x[s // k]) * (up[ids[s]] @ x[s // k]) for s in perm])
    q_ref, s_ref = orc.quantize_mxfp8_fp32(h.astype(np.float32))
    assert np.array_equal(hs, s_ref), "h scale bytes differ"
    assert np.array_equal(hq, q_ref), f"{int((hq != q_ref).sum())} h codes differ"


# (T, H, F, E, k, S): grouped tiles; a decode batch; the 128 x 512 tiles
@pytest.mark.parametrize("shape", [(300, 512, 256, 6, 2, 2), (40, 512, 256, 8, 2, 1),
                                   (900, 1024, 768, 5, 2, 1)])
def test_mxfp4_shared_experts(shape):
    """MXFP4 layer + shared experts in the routed format, against the oracle
    of the same layer with the shared experts as weight-1 slots (after the
    routed ones); with a residual and dropped ids (E, -1: never shared)."""
    T, H, F, E, k, S = shape
    _say(f"mxfp4 shared {shape}")
    p = mx_problem(T, H, F, E + S, k, seed=95 + T)
    g = torch.Generator().manual_seed(96 + T)
    idx, w = wl.route_uniform_softmax(T, E, k, g, "cpu", 1.0)
    idx = idx.clone()
    idx[::5, 0] = E
    idx[1::7, k - 1] = -1
    idx = idx.contiguous()
    names = ("gate_up", "gate_up_scale", "down", "down_scale")
    routed = {n: p[n][:-S].contiguous() for n in names}
    shared = [p[n][-S:].contiguous() for n in names]
    idx_np = idx.numpy()
    idx_a = np.concatenate([np.where((idx_np >= 0) & (idx_np < E), idx_np, -1),
                            np.tile(np.arange(E, E + S), (T, 1))], axis=1)
    w_a = np.concatenate([w.numpy(), np.ones((T, S))], axis=1)
    r = torch.randn(T, H, generator=g).to(torch.bfloat16)
    ref = orc.moe_experts_mxfp4_reference(
        p["x"].numpy(), p["x_scale"].numpy(), p["gate_up"].numpy(), p["gate_up_scale"].numpy(),
        p["down"].numpy(), p["down_scale"].numpy(), idx_a, w_a, residual=f64(r))
    out = _moe().moe_experts_mxfp4_shared(
        p["x"].cuda(), p["x_scale"].cuda(), *[routed[n].cuda() for n in names],
        *[t.cuda() for t in shared], idx.cuda(), w.cuda(), k, residual=r.cuda())
    worst, rel = check_tol(out, ref, MX_TOL, f"mxfp4 shared {shape}")
    _say(f"  worst err/tol {worst:.3f} rel L2 {rel:.2e}")
