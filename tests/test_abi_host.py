"""Host-side checks of the C ABI library (no GPU needed, no kernel launched).

The library must load, export every function declared in
include/moe_experts.h, size and lay out workspaces, and reject bad arguments
with the documented status codes before touching the GPU.
"""

import ctypes
import os
import re

import pytest
import torch

import mixture_experts_routed_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_experts.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH),
                                reason="libmoe_experts.so not built (run __graft_entry__.build())")

OK, ENULL, ESHAPE, EALIGN, EWS, ELAUNCH, EDEV = 0, -1, -2, -3, -4, -5, -6
P16 = 0x10000          # fake, 16-byte-aligned "device" addresses: only used where
P16B = 0x20000         # validation must fail before anything is enqueued


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ["moe_experts_prefill", "moe_experts_decode", "moe_experts_fp8", "moe_routing_plan",
              "moe_workspace_size", "moe_quantize_fp8_block128"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert sorted(moe.exported_symbols()) == declared_functions()


def test_version_and_strerror():
    assert moe.moe_abi_version() == 9
    for rc in (OK, ENULL, ESHAPE, EALIGN, EWS, ELAUNCH, EDEV, -7, -99):
        s = moe.moe_strerror(rc)
        assert isinstance(s, str) and s
    assert moe.moe_strerror(-99) == "unknown status"


@pytest.mark.parametrize("variant", [0, 1, 2, 4, 5])
def test_workspace_sizes_and_layout(variant):
    T, H, F, E, k = 2048, 1280, 896, 64, 6
    if variant in (2, 4, 5):
        T, H, F, E, k = 4096, 7168, 2048, 128, 8
    n = moe.moe_workspace_size(variant, T, H, F, E, k)
    lay = moe.moe_workspace_layout(variant, T, H, F, E, k)
    assert lay["total"] == n
    offs = [v for key, v in lay.items() if key != "total" and v is not None]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and len(set(offs)) == len(offs) and max(offs) < n
    P = T * k
    assert n >= P * H * 2                                   # y [P, H] bf16
    if variant in (2, 4, 5):
        assert lay["h_scale"] - lay["h"] >= P * F           # fp8 codes
        assert n - lay["y"] >= P * H * 2
    if variant == 5:                                        # E8M0 bytes per 32 of F
        assert lay["y"] - lay["h_scale"] >= P * (F // 32)
    if variant == 4:                                        # + the quantised hidden states
        assert n >= moe.moe_workspace_size(2, T, H, F, E, k) + T * H + T * (H // 128) * 4


def test_decode_fast_path_workspace_is_small():
    n1 = moe.moe_workspace_size(1, 1, 1280, 896, 64, 6)
    lay = moe.moe_workspace_layout(1, 4, 1280, 896, 64, 6)

    assert n1 >= 6 * 896 * 2 and n1 < 64 << 10   # flags and h [slots, F] bf16
    assert all(v is None for key, v in lay.items() if key != "total")
    # above the fast path the decode entry uses the grouped layout
    assert moe.moe_workspace_layout(1, 64, 1280, 896, 64, 6)["perm"] is not None


@pytest.mark.parametrize("args", [
    (0, -1, 128, 64, 8, 2),      # T < 0
    (0, 4, 100, 64, 8, 2),       # H not a multiple of 64
    (0, 4, 128, 96, 8, 2),       # F not a multiple of 64
    (0, 4, 128, 64, 8, 9),       # k > E
    (0, 4, 128, 64, 0, 1),       # E < 1
    (0, 4, 128, 64, 513, 2),     # E above MOE_MAX_EXPERTS
    (2, 4, 192, 128, 8, 2),      # fp8 H not a multiple of 128
    (2, 4, 256, 64, 8, 2),       # fp8 F not a multiple of 128
    (5, 4, 192, 128, 8, 2),      # mxfp4 H not a multiple of 128
    (5, 4, 256, 96, 8, 2),       # mxfp4 F not a multiple of 128
    (7, 4, 128, 64, 8, 2),       # unknown variant
    (0, 1 << 30, 128, 64, 8, 4),  # T*k >= 2^31
])
def test_workspace_size_rejects_bad_shapes(args):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(*args)
    assert ei.value.status == ESHAPE


def test_null_out_pointer_status():
    lib = moe._load()
    assert lib.moe_workspace_size(0, 4, 128, 64, 8, 2, None) == ENULL


def _prefill(lib, fn, *, hidden=P16, gu=P16, dn=P16, idx=P16, w=P16, res=None, out=P16, T=4,
             H=128, F=64, E=8, k=2, ws=P16B, ws_bytes=1 << 30):
    return getattr(lib, fn)(hidden, gu, dn, idx, w, res, T, H, F, E, k, out, ws, ws_bytes, None)


@pytest.mark.parametrize("fn", ["moe_experts_prefill", "moe_experts_prefill_fused",
                                "moe_experts_decode"])
def test_bf16_entry_validation(fn):
    lib = moe._load()
    assert _prefill(lib, fn, hidden=None) == ENULL
    assert _prefill(lib, fn, out=None) == ENULL
    assert _prefill(lib, fn, gu=P16 + 2) == EALIGN
    assert _prefill(lib, fn, idx=P16 + 2) == EALIGN
    assert _prefill(lib, fn, res=P16 + 2) == EALIGN          # residual not 16-byte aligned
    assert _prefill(lib, fn, k=9) == ESHAPE
    assert _prefill(lib, fn, H=96) == ESHAPE
    assert _prefill(lib, fn, ws=None) == EWS
    assert _prefill(lib, fn, ws=P16B + 16) == EWS          # not 256-byte aligned
    assert _prefill(lib, fn, ws_bytes=16) == EWS


def test_fp8_and_plan_validation():
    lib = moe._load()
    args = [P16] * 8 + [None, 4, 256, 128, 8, 2, P16, P16B, 1 << 30, None]
    bad = list(args); bad[1] = None
    assert lib.moe_experts_fp8(*bad) == ENULL
    bad = list(args); bad[2] = P16 + 8
    assert lib.moe_experts_fp8(*bad) == EALIGN
    bad = list(args); bad[8] = P16 + 8                         # residual
    assert lib.moe_experts_fp8(*bad) == EALIGN
    for i in (1, 3, 5):                                         # scales: 16-byte aligned
        bad = list(args); bad[i] = P16 + 4
        assert lib.moe_experts_fp8(*bad) == EALIGN, i
    bad = list(args); bad[10] = 192                             # H
    assert lib.moe_experts_fp8(*bad) == ESHAPE
    bad = list(args); bad[16] = 0                               # ws_bytes
    assert lib.moe_experts_fp8(*bad) == EWS
    # bf16-input form: hidden replaces (x, x_scale)
    args = [P16] * 7 + [None, 4, 256, 128, 8, 2, P16, P16B, 1 << 30, None]
    bad = list(args); bad[0] = None
    assert lib.moe_experts_fp8_bf16in(*bad) == ENULL
    bad = list(args); bad[0] = P16 + 2
    assert lib.moe_experts_fp8_bf16in(*bad) == EALIGN
    for i in (2, 4):                                            # weight scales
        bad = list(args); bad[i] = P16 + 4
        assert lib.moe_experts_fp8_bf16in(*bad) == EALIGN, i
    bad = list(args); bad[9] = 192                              # H
    assert lib.moe_experts_fp8_bf16in(*bad) == ESHAPE
    bad = list(args); bad[15] = 16                              # ws_bytes
    assert lib.moe_experts_fp8_bf16in(*bad) == EWS
    assert lib.moe_routing_plan(None, 4, 2, 8, P16, P16, P16, P16, P16B, 1 << 20, None) == ENULL
    assert lib.moe_routing_plan(P16, 4, 9, 8, P16, P16, P16, P16, P16B, 1 << 20, None) == ESHAPE
    assert lib.moe_routing_plan(P16, 4, 2, 8, P16, P16, P16, P16, P16B, 1, None) == EWS
    assert lib.moe_quantize_fp8_block128(P16, 0, 4, 100, P16, P16, None) == ESHAPE
    assert lib.moe_quantize_fp8_block128(None, 0, 4, 128, P16, P16, None) == ENULL


def test_mxfp4_validation():
    lib = moe._load()
    # x, x_scale, gate_up, gate_up_scale, down, down_scale, idx, w, residual, T, H, F, E, k,
    # out, ws, ws_bytes, stream
    args = [P16] * 8 + [None, 4, 256, 128, 8, 2, P16, P16B, 1 << 30, None]
    for i in (0, 1, 2, 3, 4, 5, 6, 7, 14):
        bad = list(args); bad[i] = None
        assert lib.moe_experts_mxfp4(*bad) == ENULL, i
    for i, off in ((0, 8), (2, 8), (4, 8), (14, 8), (8, 8), (1, 2), (3, 2), (5, 2), (6, 2)):
        bad = list(args); bad[i] = (bad[i] or P16) + off
        assert lib.moe_experts_mxfp4(*bad) == EALIGN, i
    bad = list(args); bad[10] = 192                             # H
    assert lib.moe_experts_mxfp4(*bad) == ESHAPE
    bad = list(args); bad[11] = 96                              # F
    assert lib.moe_experts_mxfp4(*bad) == ESHAPE
    bad = list(args); bad[13] = 9                               # k > E
    assert lib.moe_experts_mxfp4(*bad) == ESHAPE
    need = moe.moe_workspace_size(moe.MOE_VARIANT_MXFP4, 4, 256, 128, 8, 2)
    bad = list(args); bad[16] = need - 1                        # ws_bytes
    assert lib.moe_experts_mxfp4(*bad) == EWS
    bad = list(args); bad[15] = P16B + 16                       # ws not 256-byte aligned
    assert lib.moe_experts_mxfp4(*bad) == EWS


def test_router_validation():
    lib = moe._load()
    # logits, bias, bf16, mode, T, E, k, groups, topk_group, group_top, scale, idx, w, stream
    soft = [P16, None, 0, 0, 4, 64, 6, 1, 1, 2, 1.0, P16, P16, None]
    sig = [P16, P16B, 1, 1, 4, 256, 8, 8, 4, 2, 2.5, P16, P16, None]
    for args in (soft, sig):
        for i in (0, 11, 12):
            bad = list(args); bad[i] = None
            assert lib.moe_route_topk(*bad) == ENULL, i
    bad = list(sig); bad[1] = None                                # sigmoid needs the bias
    assert lib.moe_route_topk(*bad) == ENULL
    bad = list(soft); bad[1] = P16B                               # softmax takes no bias
    assert lib.moe_route_topk(*bad) == ESHAPE
    for i, v in ((3, 2), (2, 2), (5, 0), (5, 513), (6, 0), (6, 65), (6, 33), (4, -1)):
        bad = list(soft); bad[i] = v
        assert lib.moe_route_topk(*bad) == ESHAPE, (i, v)
    for i, v in ((7, 3), (7, 0), (7, 128), (8, 0), (8, 9), (9, 3), (9, 0), (6, 33)):
        bad = list(sig); bad[i] = v                               # groups must divide E, etc.
        assert lib.moe_route_topk(*bad) == ESHAPE, (i, v)
    bad = list(sig); bad[6], bad[7], bad[8] = 17, 16, 1           # k > topk_group * group size
    assert lib.moe_route_topk(*bad) == ESHAPE
    bad = list(sig); bad[5], bad[7], bad[9], bad[6] = 8, 8, 2, 1  # groups of one with group_top 2
    assert lib.moe_route_topk(*bad) == ESHAPE
    bad = list(soft); bad[0] = P16 + 2                            # fp32 logits need 4 bytes
    assert lib.moe_route_topk(*bad) == EALIGN
    bad = list(sig); bad[0] = P16 + 2                             # bf16 logits: 2 is enough
    assert lib.moe_route_topk(*bad) in (OK, EDEV)
    plan = soft[:13] + [P16, P16, P16, P16, P16B, 1 << 20, None]
    bad = list(plan); bad[15] = None
    assert lib.moe_route_plan(*bad) == ENULL
    bad = list(plan); bad[18] = 1
    assert lib.moe_route_plan(*bad) == EWS


def test_decode_routed_validation():
    lib = moe._load()
    # hidden, logits, bias, bf16, mode, groups, topk_group, group_top, scale, gate_up, down,
    # residual, T, H, F, E, k, out, idx, w, ws, ws_bytes, stream
    args = [P16, P16, None, 0, 0, 1, 1, 2, 1.0, P16, P16, None, 1, 128, 64, 8, 2, P16, P16, P16,
            P16B, 1 << 30, None]
    for i in (0, 1, 9, 10, 17, 18, 19):
        bad = list(args); bad[i] = None
        assert lib.moe_experts_decode_routed(*bad) == ENULL, i
    bad = list(args); bad[2] = P16B                           # softmax takes no bias
    assert lib.moe_experts_decode_routed(*bad) == ESHAPE
    bad = list(args); bad[13] = 96                            # H not a multiple of 64
    assert lib.moe_experts_decode_routed(*bad) == ESHAPE
    bad = list(args); bad[21] = 1                             # workspace too small
    assert lib.moe_experts_decode_routed(*bad) == EWS
    bad = list(args); bad[9] = P16 + 2
    assert lib.moe_experts_decode_routed(*bad) == EALIGN


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful on a host without a GPU")
def test_valid_arguments_without_gpu_report_device_error():
    lib = moe._load()
    assert _prefill(lib, "moe_experts_prefill") == EDEV
    assert _prefill(lib, "moe_experts_prefill_fused") == EDEV
    assert _prefill(lib, "moe_experts_decode") == EDEV


def test_python_binding_rejects_cpu_tensors():
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    gu = torch.zeros(8, 128, 128, dtype=torch.bfloat16)
    dn = torch.zeros(8, 128, 64, dtype=torch.bfloat16)
    idx = torch.zeros(4, 2, dtype=torch.int32)
    w = torch.zeros(4, 2)
    with pytest.raises(ValueError):
        moe.moe_experts_prefill(x, gu, dn, idx, w, 2)
    with pytest.raises(TypeError):
        moe.moe_experts_prefill(x.float(), gu, dn, idx, w, 2)


def test_profile_recorder_argument_checks():
    lib = moe._load()
    assert lib.moe_profile_begin(0) == ESHAPE
    assert lib.moe_profile_begin(4097) == ESHAPE
    n = ctypes.c_int(-1)
    ms = (ctypes.c_float * 4)()
    ids = (ctypes.c_int * 4)()
    assert lib.moe_profile_end(1, None, ms, ids) == ENULL
    assert lib.moe_profile_end(-1, ctypes.byref(n), ms, ids) == ESHAPE
    # nothing recorded: zero calls, recorder off
    assert lib.moe_profile_end(1, ctypes.byref(n), ms, ids) == OK and n.value == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful on a host without a GPU")
def test_profile_begin_without_gpu_reports_device_error():
    assert moe._load().moe_profile_begin(8) == EDEV


def test_shared_workspace_size_rules():
    T, H, F, E, k, S = 2048, 1280, 896, 64, 6, 2
    for variant in (0, 1, 2, 5):   # prefill, decode, fp8, mxfp4
        n = moe.moe_workspace_size_shared(variant, T, H, F, E, k, S)
        assert n >= moe.moe_workspace_size(variant, T, H, F, E + S, k + S) + 2 * T * (k + S) * 4
    for bad in [(3, T, H, F, E, k, S), (4, T, H, F, E, k, S), (0, T, H, F, E, k, 0),
                (0, T, H, F, 511, k, 2), (0, T, 100, F, E, k, S), (2, T, 1344, F, E, k, S)]:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_workspace_size_shared(*bad)
        assert ei.value.status == ESHAPE


@pytest.mark.parametrize("fn", ["moe_experts_prefill_shared", "moe_experts_decode_shared"])
def test_shared_entry_validation(fn):
    lib = moe._load()

    def call(**kw):
        a = dict(hidden=P16, gu=P16, dn=P16, sgu=P16, sdn=P16, idx=P16, w=P16, res=None, T=4,
                 H=128, F=64, E=8, k=2, S=2, out=P16, ws=P16B, ws_bytes=1 << 30)
        a.update(kw)
        return getattr(lib, fn)(a["hidden"], a["gu"], a["dn"], a["sgu"], a["sdn"], a["idx"], a["w"],
                                a["res"], a["T"], a["H"], a["F"], a["E"], a["k"], a["S"], a["out"],
                                a["ws"], a["ws_bytes"], None)
    assert call(sgu=None) == ENULL
    assert call(sdn=None) == ENULL
    assert call(hidden=None) == ENULL
    assert call(sgu=P16 + 2) == EALIGN
    assert call(sdn=P16 + 8) == EALIGN
    assert call(S=0) == ESHAPE
    assert call(E=511) == ESHAPE          # E + S above MOE_MAX_EXPERTS
    assert call(H=96) == ESHAPE
    assert call(ws_bytes=16) == EWS


def test_grid_cap_argument():
    lib = moe._load()
    assert lib.moe_set_grid_cap(-1) == ESHAPE
    assert lib.moe_set_grid_cap(16) == OK
    assert lib.moe_set_grid_cap(0) == OK


@pytest.mark.parametrize("fn", ["moe_experts_fp8_shared", "moe_experts_mxfp4_shared"])
def test_quantized_shared_entry_validation(fn):
    """Argument errors of the fp8 / mxfp4 shared-expert entry points, found on
    the host before anything is enqueued (no GPU needed)."""
    lib = moe._load()

    def call(**kw):
        a = dict(x=P16, xs=P16, gu=P16, gus=P16, dn=P16, dns=P16, sgu=P16, sgus=P16, sdn=P16,
                 sdns=P16, idx=P16, w=P16, res=None, T=4, H=256, F=128, E=8, k=2, S=2, out=P16,
                 ws=P16B, ws_bytes=1 << 30)
        a.update(kw)
        return getattr(lib, fn)(a["x"], a["xs"], a["gu"], a["gus"], a["dn"], a["dns"], a["sgu"],
                                a["sgus"], a["sdn"], a["sdns"], a["idx"], a["w"], a["res"], a["T"],
                                a["H"], a["F"], a["E"], a["k"], a["S"], a["out"], a["ws"],
                                a["ws_bytes"], None)

    assert call(sgu=None) == ENULL
    assert call(sdns=None) == ENULL
    assert call(sgu=P16 + 1) == EALIGN
    assert call(S=0) == ESHAPE
    assert call(S=600) == ESHAPE
    assert call(E=510, S=3) == ESHAPE        # E + S > 512
    assert call(H=192) == ESHAPE             # not a multiple of 128
