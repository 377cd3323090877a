"""Routed-experts MoE layer for MI355X (gfx950): thin Python binding.

Each function has the name of the C entry point it calls (declared in
``include/moe_experts.h``) and only marshals arguments: it checks dtypes,
shapes and devices, allocates the output and a workspace with torch, and
passes raw device pointers plus torch's current stream.  Every step of the
layer runs in the HIP kernels of ``libmoe_experts.so``; there is no other
implementation here, and a missing library is an error.

The operand contract follows the model card "DeepSeek-OCR-2 MoE experts",
"Usage": ``out = moe_experts_prefill(hidden_states, gate_up_proj, down_proj,
top_k_index.int(), top_k_weights.float(), top_k)`` with gate_up_proj
[E, 2F, H] and down_proj [E, H, F]; the decode op has the same arguments.
"""

from __future__ import annotations

import contextlib
import ctypes
import functools
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_experts.so")

MOE_VARIANT_PREFILL = 0
MOE_VARIANT_DECODE = 1
MOE_VARIANT_FP8 = 2
MOE_VARIANT_PLAN = 3
MOE_VARIANT_FP8_BF16IN = 4
MOE_VARIANT_MXFP4 = 5
MOE_ROUTE_SOFTMAX = 0
MOE_ROUTE_SIGMOID_GROUP = 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m mixture_experts_routed_amd.build` "
            "(the layer has no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sigs = {
        "moe_abi_version": ([], i32),
        "moe_strerror": ([i32], ctypes.c_char_p),
        "moe_workspace_size": ([i32, i64, i32, i32, i32, i32, ctypes.POINTER(sz)], i32),
        "moe_workspace_layout": ([i32, i64, i32, i32, i32, i32, ctypes.POINTER(sz)], i32),
        "moe_routing_plan": ([vp, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_experts_prefill": ([vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp, sz, vp], i32),
        "moe_experts_prefill_fused": ([vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp, sz, vp], i32),
        "moe_experts_decode": ([vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp, sz, vp], i32),
        "moe_experts_prefill_shared": ([vp] * 8 + [i64, i32, i32, i32, i32, i32, vp, vp, sz, vp], i32),
        "moe_experts_decode_shared": ([vp] * 8 + [i64, i32, i32, i32, i32, i32, vp, vp, sz, vp], i32),
        "moe_workspace_size_shared": ([i32, i64, i32, i32, i32, i32, i32, ctypes.POINTER(sz)], i32),
        "moe_experts_fp8": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp, sz, vp],
                            i32),
        "moe_experts_fp8_fused": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp,
                                   sz, vp], i32),
        "moe_experts_fp8_bf16in": ([vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp, sz,
                                    vp], i32),
        "moe_quantize_fp8_block128": ([vp, i32, i64, i32, vp, vp, vp], i32),
        "moe_quantize_fp8_block128_ue8m0": ([vp, i32, i64, i32, vp, vp, vp], i32),
        "moe_experts_mxfp4": ([vp] * 9 + [i64, i32, i32, i32, i32, vp, vp, sz, vp], i32),
        "moe_experts_mxfp4_fused": ([vp] * 9 + [i64, i32, i32, i32, i32, vp, vp, sz, vp], i32),
        "moe_experts_fp8_shared": ([vp] * 13 + [i64, i32, i32, i32, i32, i32, vp, vp, sz, vp], i32),
        "moe_experts_mxfp4_shared": ([vp] * 13 + [i64, i32, i32, i32, i32, i32, vp, vp, sz, vp], i32),
        "moe_route_topk": ([vp, vp, i32, i32, i64, i32, i32, i32, i32, i32, ctypes.c_float, vp, vp,
                            vp], i32),
        "moe_route_plan": ([vp, vp, i32, i32, i64, i32, i32, i32, i32, i32, ctypes.c_float, vp, vp,
                            vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_experts_decode_routed": ([vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_float, vp, vp,
                                       vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp], i32),
        "moe_profile_begin": ([i32], i32),
        "moe_set_grid_cap": ([i32], i32),
        "moe_probe_stream_read": ([vp, sz, i32, vp, vp], i32),
        "moe_experts_decode_noalloc": ([vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp], i32),
        "moe_profile_end": ([i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float),
                             ctypes.POINTER(i32)], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def exported_symbols():
    """Names of the C entry points this binding uses."""
    return ["moe_abi_version", "moe_strerror", "moe_workspace_size", "moe_workspace_layout",
            "moe_routing_plan", "moe_experts_prefill", "moe_experts_decode", "moe_experts_fp8",
            "moe_experts_fp8_bf16in", "moe_quantize_fp8_block128", "moe_profile_begin",
            "moe_profile_end", "moe_experts_prefill_shared", "moe_experts_decode_shared",
            "moe_workspace_size_shared", "moe_experts_mxfp4", "moe_route_topk", "moe_route_plan",
            "moe_experts_decode_routed", "moe_set_grid_cap", "moe_experts_decode_noalloc",
            "moe_probe_stream_read", "moe_quantize_fp8_block128_ue8m0", "moe_experts_fp8_shared",
            "moe_experts_mxfp4_shared", "moe_experts_prefill_fused", "moe_experts_fp8_fused",
            "moe_experts_mxfp4_fused"]


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {moe_strerror(status)} (status {status})")


def _check(rc, where):
    if rc != 0:
        raise MoeError(rc, where)


def moe_abi_version():
    return _load().moe_abi_version()


def moe_strerror(status):
    return _load().moe_strerror(int(status)).decode()


@functools.lru_cache(maxsize=4096)   # a pure function of its arguments; errors are not cached
def moe_workspace_size(variant, T, H, F, E, k):
    n = ctypes.c_size_t(0)
    _check(_load().moe_workspace_size(variant, T, H, F, E, k, ctypes.byref(n)), "moe_workspace_size")
    return n.value


@functools.lru_cache(maxsize=4096)
def moe_workspace_size_shared(variant, T, H, F, E, k, S):
    """Workspace bytes of moe_experts_prefill_shared (variant 0) or
    moe_experts_decode_shared (variant 1)."""
    n = ctypes.c_size_t(0)
    _check(_load().moe_workspace_size_shared(variant, T, H, F, E, k, S, ctypes.byref(n)),
           "moe_workspace_size_shared")
    return n.value


def moe_workspace_layout(variant, T, H, F, E, k):
    """Byte offsets of the workspace stages (counts, offsets, perm, inv, h,
    h scales, y, total); None where a variant has no such stage."""
    arr = (ctypes.c_size_t * 8)()
    _check(_load().moe_workspace_layout(variant, T, H, F, E, k, arr), "moe_workspace_layout")
    none = ctypes.c_size_t(-1).value
    names = ["counts", "offsets", "perm", "inv", "h", "h_scale", "y", "total"]
    return {n: (None if v == none else int(v)) for n, v in zip(names, arr)}


# ------------------------------------------------------------ stage timing
MOE_PROFILE_MAX_STAGES = 5
STAGE_NAMES = {0: "plan", 1: "gate_up", 2: "down", 3: "combine", 4: "decode", 5: "quantize",
               6: "shared_route", 7: "router", 8: "route_plan", 9: "probe", 10: "layer"}


def moe_profile_begin(max_calls):
    """Record HIP events around every kernel of the next `max_calls` layer
    calls (on the stream each kernel runs on)."""
    _check(_load().moe_profile_begin(int(max_calls)), "moe_profile_begin")


def moe_profile_end(max_calls):
    """Wait for the recorded events; returns one list per call of
    (stage name, milliseconds) in launch order."""
    n = ctypes.c_int(0)
    ms = (ctypes.c_float * (max_calls * MOE_PROFILE_MAX_STAGES))()
    ids = (ctypes.c_int * (max_calls * MOE_PROFILE_MAX_STAGES))()
    _check(_load().moe_profile_end(int(max_calls), ctypes.byref(n), ms, ids), "moe_profile_end")
    out = []
    for c in range(n.value):
        row = []
        for i in range(MOE_PROFILE_MAX_STAGES):
            sid = ids[c * MOE_PROFILE_MAX_STAGES + i]
            if sid >= 0:
                row.append((STAGE_NAMES.get(sid, str(sid)), float(ms[c * MOE_PROFILE_MAX_STAGES + i])))
        out.append(row)
    return out


def moe_probe_stream_read(src, grid, sink):
    """Measurement helper: one plain streaming read of the device tensor `src`
    (its whole storage) by `grid` workgroups; `sink` a device tensor of at
    least 4 KB."""
    nbytes = src.numel() * src.element_size()
    with _on(src.device):
        rc = _load().moe_probe_stream_read(_ptr(src), nbytes, int(grid), _ptr(sink),
                                           ctypes.c_void_p(_stream(src.device)))
    _check(rc, "moe_probe_stream_read")


def moe_set_grid_cap(max_workgroups):
    """Test hook: cap the persistent grids at `max_workgroups` (0 = no cap)."""
    _check(_load().moe_set_grid_cap(int(max_workgroups)), "moe_set_grid_cap")


# ------------------------------------------------------------ workspace cache
_ws_cache = {}


def _workspace(nbytes, device, stream):
    """Per (device, stream) workspace that only grows; work on one stream is
    ordered, so consecutive calls on it may share the buffer."""
    key = (device.index, stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


# Per-call host work is kept small (a decode call's GPU time is ~15-20 us):
# pointers go to ctypes as plain integers, the stream handle is read without
# building a stream object, and the device context is entered only when the
# tensors are not on the current device.
def _ptr(t):
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


_SAME_DEVICE = contextlib.nullcontext()


def _on(device):
    """Context making `device` current (a no-op when it already is)."""
    return _SAME_DEVICE if device.index == torch.cuda.current_device() else torch.cuda.device(device)


def _need(t, name, dtype, ndim, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _residual(residual, T, H, dev):
    """Optional residual [T, H] bf16 (None: no residual); returns a pointer."""
    if residual is None:
        return ctypes.c_void_p(None)
    _need(residual, "residual", torch.bfloat16, 2, dev)
    if tuple(residual.shape) != (T, H):
        raise ValueError("residual must be [T, H]")
    return _ptr(residual)


def _out(out, T, H, dev):
    if out is None:
        return torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, 2, dev)
    if tuple(out.shape) != (T, H):
        raise ValueError("out must be [T, H]")
    return out


def _bf16_call(entry, variant, hidden_states, gate_up_proj, down_proj, top_k_index,
               top_k_weights, top_k, residual=None, workspace=None, out=None):
    dev = hidden_states.device
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    _need(gate_up_proj, "gate_up_proj", torch.bfloat16, 3, dev)
    _need(down_proj, "down_proj", torch.bfloat16, 3, dev)
    _need(top_k_index, "top_k_index", torch.int32, 2, dev)
    _need(top_k_weights, "top_k_weights", torch.float32, 2, dev)
    T, H = hidden_states.shape
    E, F2, H2 = gate_up_proj.shape
    F = F2 // 2
    k = int(top_k)
    if H2 != H or F2 != 2 * F or tuple(down_proj.shape) != (E, H, F):
        raise ValueError("expected gate_up_proj [E,2F,H] and down_proj [E,H,F] matching hidden_states [T,H]")
    if tuple(top_k_index.shape) != (T, k) or tuple(top_k_weights.shape) != (T, k):
        raise ValueError("top_k_index and top_k_weights must be [T, top_k]")
    res = _residual(residual, T, H, dev)
    out = _out(out, T, H, dev)
    if T == 0:
        return out
    with _on(dev):
        stream = _stream(dev)
        need = moe_workspace_size(variant, T, H, F, E, k)
        ws = workspace if workspace is not None else _workspace(need, dev, stream)
        rc = getattr(_load(), entry)(_ptr(hidden_states), _ptr(gate_up_proj), _ptr(down_proj),
                                     _ptr(top_k_index), _ptr(top_k_weights), res, T, H, F, E, k,
                                     _ptr(out), _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    _check(rc, entry)
    return out


def moe_experts_prefill(hidden_states, gate_up_proj, down_proj, top_k_index, top_k_weights,
                        top_k, residual=None, workspace=None, out=None):
    """Routed experts, grouped-GEMM form; returns out [T, H] bf16 (plus the
    optional residual [T, H] bf16)."""
    return _bf16_call("moe_experts_prefill", MOE_VARIANT_PREFILL, hidden_states, gate_up_proj,
                      down_proj, top_k_index, top_k_weights, top_k, residual, workspace, out)


def moe_experts_prefill_fused(hidden_states, gate_up_proj, down_proj, top_k_index,
                              top_k_weights, top_k, residual=None, workspace=None, out=None):
    """moe_experts_prefill with gate_up, down and the combine in one
    persistent launch after the plan (same operands, workspace and result)."""
    return _bf16_call("moe_experts_prefill_fused", MOE_VARIANT_PREFILL, hidden_states,
                      gate_up_proj, down_proj, top_k_index, top_k_weights, top_k, residual,
                      workspace, out)


def moe_experts_decode(hidden_states, gate_up_proj, down_proj, top_k_index, top_k_weights,
                       top_k, residual=None, workspace=None, out=None):
    """Routed experts, gather-GEMV form for T <= 4 (grouped form above);
    returns out [T, H] bf16 (plus the optional residual)."""
    return _bf16_call("moe_experts_decode", MOE_VARIANT_DECODE, hidden_states, gate_up_proj,
                      down_proj, top_k_index, top_k_weights, top_k, residual, workspace, out)


def moe_experts_decode_noalloc(hidden_states, gate_up_proj, down_proj, top_k_index,
                               top_k_weights, top_k, residual=None, out=None):
    """moe_experts_decode with the library's static scratch buffer instead of
    a workspace (the C call allocates nothing; pass `out` to allocate nothing
    here either)."""
    dev = hidden_states.device
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    _need(gate_up_proj, "gate_up_proj", torch.bfloat16, 3, dev)
    _need(down_proj, "down_proj", torch.bfloat16, 3, dev)
    _need(top_k_index, "top_k_index", torch.int32, 2, dev)
    _need(top_k_weights, "top_k_weights", torch.float32, 2, dev)
    T, H = hidden_states.shape
    E, F2, H2 = gate_up_proj.shape
    F = F2 // 2
    k = int(top_k)
    if H2 != H or F2 != 2 * F or tuple(down_proj.shape) != (E, H, F):
        raise ValueError("expected gate_up_proj [E,2F,H] and down_proj [E,H,F] matching hidden_states [T,H]")
    if tuple(top_k_index.shape) != (T, k) or tuple(top_k_weights.shape) != (T, k):
        raise ValueError("top_k_index and top_k_weights must be [T, top_k]")
    res = _residual(residual, T, H, dev)
    out = _out(out, T, H, dev)
    with _on(dev):
        rc = _load().moe_experts_decode_noalloc(
            _ptr(hidden_states), _ptr(gate_up_proj), _ptr(down_proj), _ptr(top_k_index),
            _ptr(top_k_weights), res, T, H, F, E, k, _ptr(out), ctypes.c_void_p(_stream(dev)))
    _check(rc, "moe_experts_decode_noalloc")
    return out


def _shared_call(entry, variant, hidden_states, gate_up_proj, down_proj, shared_gate_up,
                 shared_down, top_k_index, top_k_weights, top_k, residual=None, workspace=None,
                 out=None):
    dev = hidden_states.device
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    _need(gate_up_proj, "gate_up_proj", torch.bfloat16, 3, dev)
    _need(down_proj, "down_proj", torch.bfloat16, 3, dev)
    _need(shared_gate_up, "shared_gate_up", torch.bfloat16, 3, dev)
    _need(shared_down, "shared_down", torch.bfloat16, 3, dev)
    _need(top_k_index, "top_k_index", torch.int32, 2, dev)
    _need(top_k_weights, "top_k_weights", torch.float32, 2, dev)
    T, H = hidden_states.shape
    E, F2, H2 = gate_up_proj.shape
    F = F2 // 2
    S = shared_gate_up.shape[0]
    k = int(top_k)
    if H2 != H or F2 != 2 * F or tuple(down_proj.shape) != (E, H, F):
        raise ValueError("expected gate_up_proj [E,2F,H] and down_proj [E,H,F] matching hidden_states [T,H]")
    if tuple(shared_gate_up.shape) != (S, 2 * F, H) or tuple(shared_down.shape) != (S, H, F):
        raise ValueError("expected shared_gate_up [S,2F,H] and shared_down [S,H,F] (the routed F)")
    if tuple(top_k_index.shape) != (T, k) or tuple(top_k_weights.shape) != (T, k):
        raise ValueError("top_k_index and top_k_weights must be [T, top_k]")
    res = _residual(residual, T, H, dev)
    out = _out(out, T, H, dev)
    if T == 0:
        return out
    with _on(dev):
        stream = _stream(dev)
        need = moe_workspace_size_shared(variant, T, H, F, E, k, S)
        ws = workspace if workspace is not None else _workspace(need, dev, stream)
        rc = getattr(_load(), entry)(_ptr(hidden_states), _ptr(gate_up_proj), _ptr(down_proj),
                                     _ptr(shared_gate_up), _ptr(shared_down), _ptr(top_k_index),
                                     _ptr(top_k_weights), res, T, H, F, E, k, S, _ptr(out),
                                     _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    _check(rc, entry)
    return out


def moe_experts_prefill_shared(hidden_states, gate_up_proj, down_proj, shared_gate_up,
                               shared_down, top_k_index, top_k_weights, top_k, residual=None,
                               workspace=None, out=None):
    """Routed experts plus S always-on shared experts (weight 1), grouped
    form; shared_gate_up [S,2F,H], shared_down [S,H,F] bf16."""
    return _shared_call("moe_experts_prefill_shared", MOE_VARIANT_PREFILL, hidden_states,
                        gate_up_proj, down_proj, shared_gate_up, shared_down, top_k_index,
                        top_k_weights, top_k, residual, workspace, out)


def moe_experts_decode_shared(hidden_states, gate_up_proj, down_proj, shared_gate_up,
                              shared_down, top_k_index, top_k_weights, top_k, residual=None,
                              workspace=None, out=None):
    """Decode form of moe_experts_prefill_shared."""
    return _shared_call("moe_experts_decode_shared", MOE_VARIANT_DECODE, hidden_states,
                        gate_up_proj, down_proj, shared_gate_up, shared_down, top_k_index,
                        top_k_weights, top_k, residual, workspace, out)


def _codes(t):
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def _fp8_call(entry, variant, lead, gate_up, gate_up_scale, down, down_scale, top_k_index,
              top_k_weights, top_k, residual, workspace, out):
    gate_up, down = _codes(gate_up), _codes(down)
    dev = lead[0].device
    _need(gate_up, "gate_up", torch.uint8, 3, dev)
    _need(gate_up_scale, "gate_up_scale", torch.float32, 3, dev)
    _need(down, "down", torch.uint8, 3, dev)
    _need(down_scale, "down_scale", torch.float32, 3, dev)
    _need(top_k_index, "top_k_index", torch.int32, 2, dev)
    _need(top_k_weights, "top_k_weights", torch.float32, 2, dev)
    T, H = lead[0].shape
    E, F2, H2 = gate_up.shape
    F = F2 // 2
    k = int(top_k)
    if (H2 != H or F2 != 2 * F or tuple(down.shape) != (E, H, F)
            or tuple(gate_up_scale.shape) != (E, 2 * F, H // 128)
            or tuple(down_scale.shape) != (E, H, F // 128)):
        raise ValueError("fp8 operand shapes do not match [T,H], [E,2F,H], [E,H,F] with per-128 scales")
    if tuple(top_k_index.shape) != (T, k) or tuple(top_k_weights.shape) != (T, k):
        raise ValueError("top_k_index and top_k_weights must be [T, top_k]")
    res = _residual(residual, T, H, dev)
    out = _out(out, T, H, dev)
    if T == 0:
        return out
    with _on(dev):
        stream = _stream(dev)
        need = moe_workspace_size(variant, T, H, F, E, k)
        ws = workspace if workspace is not None else _workspace(need, dev, stream)
        rc = getattr(_load(), entry)(*[_ptr(t) for t in lead], _ptr(gate_up), _ptr(gate_up_scale),
                                     _ptr(down), _ptr(down_scale), _ptr(top_k_index),
                                     _ptr(top_k_weights), res, T, H, F, E, k, _ptr(out), _ptr(ws),
                                     ws.numel(), ctypes.c_void_p(stream))
    _check(rc, entry)
    return out


def moe_experts_fp8(x, x_scale, gate_up, gate_up_scale, down, down_scale, top_k_index,
                    top_k_weights, top_k, residual=None, workspace=None, out=None):
    """FP8 block-scaled routed experts.  fp8 operands are uint8 tensors of
    E4M3FN codes (or torch.float8_e4m3fn tensors); returns out [T, H] bf16
    (plus the optional residual [T, H] bf16)."""
    x = _codes(x)
    _need(x, "x", torch.uint8, 2)
    _need(x_scale, "x_scale", torch.float32, 2, x.device)
    if tuple(x_scale.shape) != (x.shape[0], x.shape[1] // 128):
        raise ValueError("x_scale must be [T, H/128]")
    return _fp8_call("moe_experts_fp8", MOE_VARIANT_FP8, [x, x_scale], gate_up, gate_up_scale,
                     down, down_scale, top_k_index, top_k_weights, top_k, residual, workspace, out)


def moe_experts_fp8_fused(x, x_scale, gate_up, gate_up_scale, down, down_scale, top_k_index,
                          top_k_weights, top_k, residual=None, workspace=None, out=None):
    """moe_experts_fp8 with the products and the combine in one persistent
    launch after the plan (same operands, workspace and result)."""
    x = _codes(x)
    _need(x, "x", torch.uint8, 2)
    _need(x_scale, "x_scale", torch.float32, 2, x.device)
    if tuple(x_scale.shape) != (x.shape[0], x.shape[1] // 128):
        raise ValueError("x_scale must be [T, H/128]")
    return _fp8_call("moe_experts_fp8_fused", MOE_VARIANT_FP8, [x, x_scale], gate_up,
                     gate_up_scale, down, down_scale, top_k_index, top_k_weights, top_k, residual,
                     workspace, out)


def moe_experts_fp8_bf16in(hidden_states, gate_up, gate_up_scale, down, down_scale, top_k_index,
                           top_k_weights, top_k, residual=None, workspace=None, out=None):
    """The FP8 layer fed with bf16 hidden states [T, H], quantised per
    128-wide block inside the call; returns out [T, H] bf16."""
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    return _fp8_call("moe_experts_fp8_bf16in", MOE_VARIANT_FP8_BF16IN, [hidden_states], gate_up,
                     gate_up_scale, down, down_scale, top_k_index, top_k_weights, top_k, residual,
                     workspace, out)


def _quant_shared_call(entry, variant, x, x_scale, gate_up, gate_up_scale, down, down_scale,
                       shared, top_k_index, top_k_weights, top_k, residual, workspace, out):
    """Shared-expert forms of the fp8 / mxfp4 layers: `shared` is (gate_up,
    gate_up_scale, down, down_scale) of S experts in the routed format."""
    x = _codes(x)
    dev = x.device
    sgu, sgus, sdn, sdns = (_codes(shared[0]), shared[1], _codes(shared[2]), shared[3])
    gate_up, down = _codes(gate_up), _codes(down)
    mx = variant == MOE_VARIANT_MXFP4
    sdt = torch.uint8 if mx else torch.float32
    for t, name, nd, dt in ((x, "x", 2, torch.uint8), (x_scale, "x_scale", 2, sdt),
                            (gate_up, "gate_up", 3, torch.uint8), (gate_up_scale, "gate_up_scale", 3, sdt),
                            (down, "down", 3, torch.uint8), (down_scale, "down_scale", 3, sdt),
                            (sgu, "shared_gate_up", 3, torch.uint8), (sgus, "shared_gate_up_scale", 3, sdt),
                            (sdn, "shared_down", 3, torch.uint8), (sdns, "shared_down_scale", 3, sdt)):
        _need(t, name, dt, nd, dev)
    _need(top_k_index, "top_k_index", torch.int32, 2, dev)
    _need(top_k_weights, "top_k_weights", torch.float32, 2, dev)
    T, H = x.shape
    E, F2, _ = gate_up.shape
    F = F2 // 2
    S = sgu.shape[0]
    k = int(top_k)
    pk, sb = (2, 32) if mx else (1, 128)   # codes per byte, values per scale
    want = {"gate_up": (E, 2 * F, H // pk), "gate_up_scale": (E, 2 * F, H // sb),
            "down": (E, H, F // pk), "down_scale": (E, H, F // sb),
            "shared_gate_up": (S, 2 * F, H // pk), "shared_gate_up_scale": (S, 2 * F, H // sb),
            "shared_down": (S, H, F // pk), "shared_down_scale": (S, H, F // sb),
            "x_scale": (T, H // sb)}
    got = {"gate_up": gate_up, "gate_up_scale": gate_up_scale, "down": down, "down_scale": down_scale,
           "shared_gate_up": sgu, "shared_gate_up_scale": sgus, "shared_down": sdn,
           "shared_down_scale": sdns, "x_scale": x_scale}
    for name, shape in want.items():
        if tuple(got[name].shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}, got {list(got[name].shape)}")
    if tuple(top_k_index.shape) != (T, k) or tuple(top_k_weights.shape) != (T, k):
        raise ValueError("top_k_index and top_k_weights must be [T, top_k]")
    res = _residual(residual, T, H, dev)
    out = _out(out, T, H, dev)
    if T == 0:
        return out
    with _on(dev):
        stream = _stream(dev)
        need = moe_workspace_size_shared(variant, T, H, F, E, k, S)
        ws = workspace if workspace is not None else _workspace(need, dev, stream)
        rc = getattr(_load(), entry)(_ptr(x), _ptr(x_scale), _ptr(gate_up), _ptr(gate_up_scale),
                                     _ptr(down), _ptr(down_scale), _ptr(sgu), _ptr(sgus), _ptr(sdn),
                                     _ptr(sdns), _ptr(top_k_index), _ptr(top_k_weights), res, T, H,
                                     F, E, k, S, _ptr(out), _ptr(ws), ws.numel(),
                                     ctypes.c_void_p(stream))
    _check(rc, entry)
    return out


def moe_experts_fp8_shared(x, x_scale, gate_up, gate_up_scale, down, down_scale, shared_gate_up,
                           shared_gate_up_scale, shared_down, shared_down_scale, top_k_index,
                           top_k_weights, top_k, residual=None, workspace=None, out=None):
    """moe_experts_fp8 plus S always-on shared experts (weight 1) in the
    routed experts' FP8 format: shared_gate_up [S,2F,H] + fp32 [S,2F,H/128],
    shared_down [S,H,F] + fp32 [S,H,F/128]."""
    return _quant_shared_call("moe_experts_fp8_shared", MOE_VARIANT_FP8, x, x_scale, gate_up,
                              gate_up_scale, down, down_scale,
                              (shared_gate_up, shared_gate_up_scale, shared_down, shared_down_scale),
                              top_k_index, top_k_weights, top_k, residual, workspace, out)


def moe_experts_mxfp4_shared(x, x_scale, gate_up, gate_up_scale, down, down_scale, shared_gate_up,
                             shared_gate_up_scale, shared_down, shared_down_scale, top_k_index,
                             top_k_weights, top_k, residual=None, workspace=None, out=None):
    """moe_experts_mxfp4 plus S always-on shared experts (weight 1) in the
    routed experts' MXFP4 format."""
    return _quant_shared_call("moe_experts_mxfp4_shared", MOE_VARIANT_MXFP4, x, x_scale, gate_up,
                              gate_up_scale, down, down_scale,
                              (shared_gate_up, shared_gate_up_scale, shared_down, shared_down_scale),
                              top_k_index, top_k_weights, top_k, residual, workspace, out)


def moe_experts_mxfp4(x, x_scale, gate_up, gate_up_scale, down, down_scale, top_k_index,
                      top_k_weights, top_k, residual=None, workspace=None, out=None):
    """Routed experts with MXFP4 weights and MXFP8 activations.  x uint8 [T, H]
    E4M3 codes (or torch.float8_e4m3fn) with x_scale uint8 [T, H/32] E8M0;
    gate_up uint8 [E, 2F, H/2] and down uint8 [E, H, F/2] hold two E2M1 codes
    per byte (element 2i in the low nibble) with uint8 E8M0 scales
    [E, 2F, H/32] and [E, H, F/32].  Returns out [T, H] bf16 (plus the
    optional residual [T, H] bf16)."""
    return _mx_call("moe_experts_mxfp4", x, x_scale, gate_up, gate_up_scale, down, down_scale,
                    top_k_index, top_k_weights, top_k, residual, workspace, out)


def moe_experts_mxfp4_fused(x, x_scale, gate_up, gate_up_scale, down, down_scale, top_k_index,
                            top_k_weights, top_k, residual=None, workspace=None, out=None):
    """moe_experts_mxfp4 in one persistent launch (plan, both products and the
    combine; same operands, workspace and result)."""
    return _mx_call("moe_experts_mxfp4_fused", x, x_scale, gate_up, gate_up_scale, down,
                    down_scale, top_k_index, top_k_weights, top_k, residual, workspace, out)


def _mx_call(entry, x, x_scale, gate_up, gate_up_scale, down, down_scale, top_k_index,
             top_k_weights, top_k, residual, workspace, out):
    x = _codes(x)
    dev = x.device
    _need(x, "x", torch.uint8, 2)
    for t, name, nd in ((x_scale, "x_scale", 2), (gate_up, "gate_up", 3),
                        (gate_up_scale, "gate_up_scale", 3), (down, "down", 3),
                        (down_scale, "down_scale", 3)):
        _need(t, name, torch.uint8, nd, dev)
    _need(top_k_index, "top_k_index", torch.int32, 2, dev)
    _need(top_k_weights, "top_k_weights", torch.float32, 2, dev)
    T, H = x.shape
    E, F2, Hh = gate_up.shape
    F = F2 // 2
    k = int(top_k)
    if (2 * Hh != H or F2 != 2 * F or tuple(x_scale.shape) != (T, H // 32)
            or tuple(gate_up_scale.shape) != (E, 2 * F, H // 32)
            or tuple(down.shape) != (E, H, F // 2) or tuple(down_scale.shape) != (E, H, F // 32)):
        raise ValueError("mxfp4 operand shapes do not match x [T,H], gate_up [E,2F,H/2], "
                         "down [E,H,F/2] with per-32 scales")
    if tuple(top_k_index.shape) != (T, k) or tuple(top_k_weights.shape) != (T, k):
        raise ValueError("top_k_index and top_k_weights must be [T, top_k]")
    res = _residual(residual, T, H, dev)
    out = _out(out, T, H, dev)
    if T == 0:
        return out
    with _on(dev):
        stream = _stream(dev)
        need = moe_workspace_size(MOE_VARIANT_MXFP4, T, H, F, E, k)
        ws = workspace if workspace is not None else _workspace(need, dev, stream)
        rc = getattr(_load(), entry)(_ptr(x), _ptr(x_scale), _ptr(gate_up), _ptr(gate_up_scale),
                                     _ptr(down), _ptr(down_scale), _ptr(top_k_index),
                                     _ptr(top_k_weights), res, T, H, F, E, k, _ptr(out),
                                     _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    _check(rc, entry)
    return out


def _route_args(logits, k, mode, bias, num_groups, topk_group, group_top):
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("logits must be float32 or bfloat16")
    _need(logits, "logits", logits.dtype, 2)
    dev = logits.device
    if mode not in (MOE_ROUTE_SOFTMAX, MOE_ROUTE_SIGMOID_GROUP):
        raise ValueError("mode must be MOE_ROUTE_SOFTMAX or MOE_ROUTE_SIGMOID_GROUP")
    if bias is not None:
        _need(bias, "bias", logits.dtype, 1, dev)
        if bias.shape[0] != logits.shape[1]:
            raise ValueError("bias must be [E]")
    T, E = logits.shape
    idx = torch.empty(T, int(k), dtype=torch.int32, device=dev)
    w = torch.empty(T, int(k), dtype=torch.float32, device=dev)
    args = [_ptr(logits), ctypes.c_void_p(None) if bias is None else _ptr(bias),
            int(logits.dtype == torch.bfloat16), int(mode), T, E, int(k), int(num_groups),
            int(topk_group), int(group_top)]
    return dev, T, E, idx, w, args


def moe_route_topk(logits, k, mode=MOE_ROUTE_SOFTMAX, bias=None, num_groups=1, topk_group=1,
                   group_top=2, routed_scaling_factor=1.0):
    """Router: logits [T, E] (fp32 or bf16) -> (top_k_index int32 [T, k],
    top_k_weights fp32 [T, k]).  MOE_ROUTE_SOFTMAX: softmax top-k times the
    factor; MOE_ROUTE_SIGMOID_GROUP: group-aware sigmoid routing with bias [E]
    (same dtype as the logits)."""
    dev, T, E, idx, w, args = _route_args(logits, k, mode, bias, num_groups, topk_group, group_top)
    if T == 0:
        return idx, w
    with _on(dev):
        rc = _load().moe_route_topk(*args, float(routed_scaling_factor), _ptr(idx), _ptr(w),
                                    ctypes.c_void_p(_stream(dev)))
    _check(rc, "moe_route_topk")
    return idx, w


def moe_route_plan(logits, k, mode=MOE_ROUTE_SOFTMAX, bias=None, num_groups=1, topk_group=1,
                   group_top=2, routed_scaling_factor=1.0):
    """Router then routing plan (one launch for small batches):
    (top_k_index, top_k_weights, counts[E], offsets[E+1], perm[T*k], inv[T*k])."""
    dev, T, E, idx, w, args = _route_args(logits, k, mode, bias, num_groups, topk_group, group_top)
    P = T * int(k)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(P, dtype=torch.int32, device=dev)
    inv = torch.empty(P, dtype=torch.int32, device=dev)
    if T == 0:   # an empty batch: empty plan
        return idx, w, counts.zero_(), offsets.zero_(), perm, inv
    with _on(dev):
        stream = _stream(dev)
        ws = _workspace(moe_workspace_size(MOE_VARIANT_PLAN, T, 0, 0, E, int(k)), dev, stream)
        rc = _load().moe_route_plan(*args, float(routed_scaling_factor), _ptr(idx), _ptr(w),
                                    _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(ws),
                                    ws.numel(), ctypes.c_void_p(stream))
    _check(rc, "moe_route_plan")
    return idx, w, counts, offsets, perm, inv


def moe_experts_decode_routed(hidden_states, router_logits, gate_up_proj, down_proj, top_k,
                              mode=MOE_ROUTE_SOFTMAX, bias=None, num_groups=1, topk_group=1,
                              group_top=2, routed_scaling_factor=1.0, residual=None,
                              workspace=None, out=None):
    """bf16 decode from router logits [T, E] (fp32 or bf16): routing fused
    into the decode kernels (T <= 4 gather-GEMV form).  Returns (out [T, H]
    bf16, top_k_index int32 [T, k], top_k_weights fp32 [T, k])."""
    dev = hidden_states.device
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    _need(gate_up_proj, "gate_up_proj", torch.bfloat16, 3, dev)
    _need(down_proj, "down_proj", torch.bfloat16, 3, dev)
    T, H = hidden_states.shape
    E, F2, H2 = gate_up_proj.shape
    F = F2 // 2
    k = int(top_k)
    if H2 != H or F2 != 2 * F or tuple(down_proj.shape) != (E, H, F):
        raise ValueError("expected gate_up_proj [E,2F,H] and down_proj [E,H,F] matching hidden_states [T,H]")
    _, Tl, El, idx, w, rargs = _route_args(router_logits, k, mode, bias, num_groups, topk_group,
                                           group_top)
    if (Tl, El) != (T, E):
        raise ValueError("router_logits must be [T, E]")
    res = _residual(residual, T, H, dev)
    out = _out(out, T, H, dev)
    if T == 0:
        return out, idx, w
    with _on(dev):
        stream = _stream(dev)
        need = moe_workspace_size(MOE_VARIANT_DECODE, T, H, F, E, k)
        ws = workspace if workspace is not None else _workspace(need, dev, stream)
        lg, bp, bf, md = rargs[0], rargs[1], rargs[2], rargs[3]
        rc = _load().moe_experts_decode_routed(
            _ptr(hidden_states), lg, bp, bf, md, int(num_groups), int(topk_group), int(group_top),
            float(routed_scaling_factor), _ptr(gate_up_proj), _ptr(down_proj), res, T, H, F, E, k,
            _ptr(out), _ptr(idx), _ptr(w), _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    _check(rc, "moe_experts_decode_routed")
    return out, idx, w


def moe_routing_plan(top_k_index, num_experts):
    """(counts[E], offsets[E+1], perm[T*k], inv[T*k]) as int32 device tensors."""
    dev = top_k_index.device
    _need(top_k_index, "top_k_index", torch.int32, 2)
    T, k = top_k_index.shape
    E = int(num_experts)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    with _on(dev):
        stream = _stream(dev)
        need = moe_workspace_size(MOE_VARIANT_PLAN, T, 0, 0, E, k)
        ws = _workspace(need, dev, stream)
        rc = _load().moe_routing_plan(_ptr(top_k_index), T, k, E, _ptr(counts), _ptr(offsets),
                                      _ptr(perm), _ptr(inv), _ptr(ws), ws.numel(),
                                      ctypes.c_void_p(stream))
    _check(rc, "moe_routing_plan")
    return counts, offsets, perm, inv


def moe_quantize_fp8_block128(t):
    """fp32 or bf16 [rows, K] -> (codes uint8 [rows, K], scales fp32 [rows, K/128])."""
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("input must be float32 or bfloat16")
    _need(t, "input", t.dtype, 2)
    rows, K = t.shape
    codes = torch.empty(rows, K, dtype=torch.uint8, device=t.device)
    scales = torch.empty(rows, max(K // 128, 0), dtype=torch.float32, device=t.device)
    with _on(t.device):
        rc = _load().moe_quantize_fp8_block128(_ptr(t), int(t.dtype == torch.bfloat16), rows, K,
                                               _ptr(codes), _ptr(scales),
                                               ctypes.c_void_p(_stream(t.device)))
    _check(rc, "moe_quantize_fp8_block128")
    return codes, scales


def moe_quantize_fp8_block128_ue8m0(t):
    """fp32 or bf16 [rows, K] -> (codes uint8 [rows, K], scale bytes uint8
    [rows, K/128], value 2^(byte - 127))."""
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("input must be float32 or bfloat16")
    _need(t, "input", t.dtype, 2)
    rows, K = t.shape
    codes = torch.empty(rows, K, dtype=torch.uint8, device=t.device)
    scales = torch.empty(rows, max(K // 128, 0), dtype=torch.uint8, device=t.device)
    with _on(t.device):
        rc = _load().moe_quantize_fp8_block128_ue8m0(_ptr(t), int(t.dtype == torch.bfloat16), rows,
                                                     K, _ptr(codes), _ptr(scales),
                                                     ctypes.c_void_p(_stream(t.device)))
    _check(rc, "moe_quantize_fp8_block128_ue8m0")
    return codes, scales


__all__ = [
    "moe_abi_version", "moe_strerror", "moe_workspace_size", "moe_workspace_layout",
    "moe_profile_begin", "moe_profile_end",
    "moe_routing_plan", "moe_experts_prefill", "moe_experts_prefill_fused", "moe_experts_decode",
    "moe_experts_fp8", "moe_experts_fp8_fused", "moe_experts_fp8_bf16in", "moe_quantize_fp8_block128",
    "moe_quantize_fp8_block128_ue8m0",
    "moe_experts_fp8_shared", "moe_experts_mxfp4_shared", "moe_experts_prefill_shared",
    "moe_experts_decode_shared", "moe_workspace_size_shared", "moe_experts_mxfp4",
    "moe_experts_mxfp4_fused", "MoeError",
    "MOE_VARIANT_PREFILL", "MOE_VARIANT_DECODE", "MOE_VARIANT_FP8", "MOE_VARIANT_PLAN",
    "MOE_VARIANT_FP8_BF16IN", "MOE_VARIANT_MXFP4", "moe_route_topk", "moe_route_plan",
    "moe_experts_decode_routed",
    "MOE_ROUTE_SOFTMAX", "MOE_ROUTE_SIGMOID_GROUP",
    "LIB_PATH",
]
