"""The allocation-free decode entry point, called through the C ABI, against
moe_experts_decode (same kernels, so the outputs must be bit-identical), on
consecutive calls of decreasing size; and its size limit."""

import ctypes

import numpy as np
import pytest
import torch

import moe_workloads as wl
from oracle import moe_oracle as orc

pytestmark = pytest.mark.gpu

MOE_ERR_SCRATCH = -7


def _noalloc(lib, g, T, k, residual, out):
    E, F2, H = g["gate_up"].shape
    stream = torch.cuda.current_stream().cuda_stream
    return lib.moe_experts_decode_noalloc(
        g["hidden"][:T].data_ptr(), g["gate_up"].data_ptr(), g["down"].data_ptr(),
        g["top_k_index"][:T].data_ptr(), g["top_k_weights"][:T].data_ptr(),
        None if residual is None else residual.data_ptr(), T, H, F2 // 2, E, k, out.data_ptr(),
        ctypes.c_void_p(stream))


def test_noalloc_decode_matches_decode_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_routed_amd as moe
    lib = moe._load()
    # OCR-2 shapes (H=1280, F=896, 64 experts, top-6): T=16 (the grouped form,
    # its workspace in the static buffer), then T=4 and T=1 (the gather-GEMV
    # form), each call smaller than the one before
    p = wl.make_bf16_problem(16, 1280, 896, 64, 6, seed=1102, device="cpu")
    g = {n: v.cuda().contiguous() for n, v in p.items()}
    res = torch.randn(16, 1280, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).cuda()
    k = 6
    for T, r in ((16, None), (4, res[:4].contiguous()), (1, None), (1, res[:1].contiguous())):
        print(f"noalloc decode T={T} residual={r is not None}", flush=True)
        ref = moe.moe_experts_decode(g["hidden"][:T], g["gate_up"], g["down"],
                                     g["top_k_index"][:T], g["top_k_weights"][:T], k, residual=r)
        out = torch.full((T, 1280), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert _noalloc(lib, g, T, k, r, out) == 0
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"T={T}: differs"
        want = orc.moe_experts_reference_batched(
            p["hidden"][:T].double().numpy(), p["gate_up"].double().numpy(),
            p["down"].double().numpy(), p["top_k_index"][:T].numpy(),
            p["top_k_weights"][:T].double().numpy(),
            residual=None if r is None else r.double().cpu().numpy())
        got = out.double().cpu().numpy()
        assert np.all(np.abs(got - want) <= 1e-2 + 1e-2 * np.abs(want)), f"T={T}: off the oracle"


def test_noalloc_decode_rejects_oversize_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_routed_amd as moe
    lib = moe._load()
    # T=4096 at the OCR-2 shapes needs about 140 MB of workspace: refused on
    # the host, nothing is enqueued
    need = moe.moe_workspace_size(moe.MOE_VARIANT_DECODE, 4096, 1280, 896, 64, 6)
    assert need > (16 << 20)
    dummy = torch.empty(256, dtype=torch.uint8, device="cuda")
    a = dummy.data_ptr()
    rc = lib.moe_experts_decode_noalloc(a, a, a, a, a, None, 4096, 1280, 896, 64, 6, a,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == MOE_ERR_SCRATCH
    assert "static buffer" in moe.moe_strerror(rc)
