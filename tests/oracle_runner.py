"""Helpers for checking whole DeepSeek-V3-shaped layers against the oracle.

The oracle's expert-batched forms are evaluated over disjoint subsets of the
experts in a few host threads: the layer is a sum over slots, so the outputs
of the subsets (every other slot dropped by giving it id -1, which the oracle
skips) add up to the whole layer.  Weights stay on the GPU and are copied to
the host one expert at a time.
"""

import concurrent.futures as cf
import os

import numpy as np


class DeviceExperts:
    """Indexable view of a device weight tensor [E, ...]: item e is a host
    copy of expert e (nothing is kept)."""

    def __init__(self, t):
        self.t, self.shape = t, tuple(t.shape)

    def __getitem__(self, e):
        return self.t[int(e)].cpu().numpy()


def by_expert_subsets(fn, operands, idx, w, E, threads=None):
    """fn(*operands, idx, w) summed over disjoint expert subsets evaluated in
    parallel host threads; idx [T, k] int, w [T, k]."""
    if threads is None:
        threads = max(1, min(4, len(os.sched_getaffinity(0)) // 4))
    idx = np.asarray(idx)
    groups = [g for g in np.array_split(np.arange(E), threads) if g.size]

    def part(g):
        sel = np.where(np.isin(idx, g), idx, -1).astype(np.int32)
        return fn(*operands, sel, w)

    with cf.ThreadPoolExecutor(len(groups)) as ex:
        outs = list(ex.map(part, groups))
    return np.sum(outs, axis=0)


# ----------------------------------------------------------------------------
# Every-row check of the quantised layers (fp8 block-128, MXFP4/MXFP8).
#
# Both sides re-quantise the SwiGLU output h in fp32, but from h values that
# differ in the last bits (the GPU accumulates in fp32, the oracle in
# float64).  Where the oracle's h lies within those bits of a rounding
# midpoint, either neighbouring code is a correct result of the rule, and a
# code near the top of its block moves one y row by about 1e-2 relative,
# more than an output near zero may differ.  So the check validates the
# GPU's h codes first: each must be the rule's code for some h within
# `margin` (relative to the block maximum) of the oracle's h, with a block
# scale the rule gives for a block maximum within the same margin.  Then
# every output element must meet the tolerance widened by exactly what the
# validated code differences can move it: sum over the token's differing
# codes of w * |down[:, f]| * |h_gpu - h_oracle|.  Tokens without differing
# codes get the plain tolerance.
# ----------------------------------------------------------------------------

def _gpu_h_slot_order(ws, lay, P, F, nscale, scale_dtype):
    import torch
    perm = ws[lay["perm"]:lay["perm"] + 4 * P].view(torch.int32).cpu().numpy()
    nbytes = np.dtype(scale_dtype).itemsize
    hq = ws[lay["h"]:lay["h"] + P * F].cpu().numpy().reshape(P, F)
    hs = ws[lay["h_scale"]:lay["h_scale"] + nbytes * P * nscale].cpu().numpy().view(scale_dtype)
    hs = hs.reshape(P, nscale)
    valid = perm >= 0
    q = np.zeros((P, F), np.uint8)
    s = np.zeros((P, nscale), scale_dtype)
    q[perm[valid]] = hq[valid]
    s[perm[valid]] = hs[valid]
    return q, s


def check_quantized_layer(kind, out, p, ws, lay, what, orc, tol=(3e-2, 3e-2), margin=1e-4,
                          threads=None):
    """kind "fp8" or "mxfp4"; out the GPU output [T, H]; p the device problem;
    ws / lay the workspace of that call and its layout.  Returns a dict of
    statistics; asserts on any failure."""
    T, k = p["top_k_index"].shape
    E = p["gate_up"].shape[0]
    F = p["gate_up"].shape[1] // 2
    P = T * k
    idx = p["top_k_index"].cpu().numpy()
    w = p["top_k_weights"].cpu().numpy().astype(np.float64)
    ops = [p["x"].cpu().numpy(), p["x_scale"].cpu().numpy()] + [
        DeviceExperts(p[n]) for n in ("gate_up", "gate_up_scale", "down", "down_scale")]
    fn = orc.moe_experts_fp8_reference_batched if kind == "fp8" else orc.moe_experts_mxfp4_reference_batched
    if threads is None:
        threads = max(1, min(4, len(os.sched_getaffinity(0)) // 4))
    groups = [g for g in np.array_split(np.arange(E), threads) if g.size]

    def part(g):
        sel = np.where(np.isin(idx, g), idx, -1).astype(np.int32)
        rep = {}
        return fn(*ops, sel, w, h_report=rep), rep

    with cf.ThreadPoolExecutor(len(groups)) as ex:
        parts = list(ex.map(part, groups))
    ref = np.sum([o for o, _ in parts], axis=0)
    h32 = np.sum([r["h"] for _, r in parts], axis=0)
    q_ref = np.sum([r["codes"].astype(np.int64) for _, r in parts], axis=0).astype(np.uint8)
    s_ref = np.sum([r["scales"] for _, r in parts], axis=0)

    if kind == "fp8":
        nb, qmax = 128, 448.0
        q_gpu, s_gpu = _gpu_h_slot_order(ws, lay, P, F, F // nb, np.float32)
    else:
        nb, qmax = 32, 448.0
        q_gpu, s_gpu = _gpu_h_slot_order(ws, lay, P, F, F // nb, np.uint8)
    valid = ((idx >= 0) & (idx < E)).reshape(-1)

    # block scales as values (fp32 rule: s; MX: 2^(byte - 127))
    def scale_val(s):
        return s.astype(np.float64) if kind == "fp8" else np.exp2(s.astype(np.float64) - 127.0)
    sg, sr = scale_val(s_gpu), scale_val(s_ref)
    amax = np.abs(h32.astype(np.float64)).reshape(P, F // nb, nb).max(-1)
    if kind == "fp8":
        # the GPU's scale is amax'/448 for some amax' within the margin
        lo, hi = amax * (1 - margin) / qmax, amax * (1 + margin) / qmax
        zero = amax == 0
        bad_scale = ~np.where(zero, sg == 1.0, (sg >= lo * (1 - 1e-7)) & (sg <= hi * (1 + 1e-7)))
    else:
        def rule(a):
            _, e = np.frexp(np.where(a > 0, a, 1.0))
            return np.where(a > 0, np.clip(e - 1 - 8, -127, 127), -127)
        eg = s_gpu.astype(np.int64) - 127
        bad_scale = ~((eg == rule(amax * (1 - margin))) | (eg == rule(amax * (1 + margin))) |
                      (eg == rule(amax)))
    bad_scale &= valid[:, None]
    assert not bad_scale.any(), f"{what}: {int(bad_scale.sum())} h block scales outside the rule"

    # codes: the rule's code of some h within margin * block max of the oracle's h,
    # under the GPU's own block scale
    dec = orc.e4m3fn_decode(np.arange(256, dtype=np.uint8))
    diff = (q_gpu != q_ref) & valid[:, None]
    if kind == "mxfp4":
        diff |= (np.repeat(s_gpu != s_ref, nb, axis=1) & valid[:, None])
    rows, cols = np.nonzero(diff)
    stats = {"h_codes_checked": int(valid.sum()) * F, "h_codes_differing": int(rows.size)}
    widen = np.zeros_like(ref)
    if rows.size:
        sgf = sg[rows, cols // nb]
        srf = sr[rows, cols // nb]
        m = margin * amax[rows, cols // nb] / sgf
        v = h32[rows, cols].astype(np.float64) / sgf
        lo = orc.e4m3fn_encode(np.clip(v - m, -qmax, qmax))
        hi = orc.e4m3fn_encode(np.clip(v + m, -qmax, qmax))
        vg = dec[q_gpu[rows, cols]]
        ok = (vg >= np.minimum(dec[lo], dec[hi])) & (vg <= np.maximum(dec[lo], dec[hi]))
        if not ok.all():
            i = int(np.nonzero(~ok)[0][0])
            raise AssertionError(
                f"{what}: {int((~ok).sum())} of {rows.size} differing h codes are not a rounding of "
                f"the oracle's h (first: slot {rows[i]}, col {cols[i]}, h/scale {v[i]:.5f}, gpu code "
                f"value {vg[i]}, oracle code value {dec[q_ref[rows[i], cols[i]]]})")
        # distance of the oracle's h from the midpoint between the two codes,
        # relative to the block maximum: how far the GPU's h must have moved
        vr = dec[q_ref[rows, cols]]
        mid = 0.5 * (vr + vg)
        stats["max_midpoint_distance"] = float(np.max(np.abs(v - mid) * sgf / amax[rows, cols // nb]))
        stats["max_code_steps"] = int(np.max(np.abs(q_gpu[rows, cols].astype(np.int64) & 0x7F) -
                                             (q_ref[rows, cols].astype(np.int64) & 0x7F)))
        assert rows.size <= 1e-2 * stats["h_codes_checked"] + 8, f"{what}: too many differing h codes"
        dh = np.abs(vg * sgf - dec[q_ref[rows, cols]] * srf)
        # widen: w[t, j] * |down_e[:, f]| * |dh| for every differing code
        ids = idx.reshape(-1)[rows]
        for e in np.unique(ids):
            sel = ids == e
            fcols = cols[sel]
            uf, inv = np.unique(fcols, return_inverse=True)
            dn = p["down"][int(e)]
            dsc = p["down_scale"][int(e)]
            if kind == "fp8":
                codes = dn[:, uf].cpu().numpy()
                colv = np.abs(dec[codes] * dsc[:, uf // 128].cpu().numpy().astype(np.float64))
            else:
                byte = dn[:, uf // 2].cpu().numpy()
                nib = np.where(uf % 2 == 0, byte & 0xF, byte >> 4)
                colv = np.abs(orc.e2m1_decode(nib) * orc.e8m0_decode(dsc[:, uf // 32].cpu().numpy()))
            for r, ii, d in zip(rows[sel], inv, dh[sel]):
                widen[r // k] += w.reshape(-1)[r] * colv[:, ii] * d
    g = out.float().cpu().numpy().astype(np.float64)
    atol, rtol = tol
    base = atol + rtol * np.abs(ref)
    err = np.abs(g - ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    worst = float(np.max(err / (base + widen)))
    stats.update(worst=worst, worst_plain=float(np.max(err / base)),
                 widened_elements=int((err > base).sum()),
                 rel_l2=float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)))
    assert worst <= 1.0, f"{what}: worst err/tol {worst:.3f} after accounting for {rows.size} h-code roundings"
    return stats
