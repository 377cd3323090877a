"""Benchmark of the routed-experts MoE layer on one MI355X.

Default workload: DeepSeek-OCR-2-shaped decode, T=1 token, H=1280, F=896,
64 experts, top-6, bf16 (the gather-GEMV entry point).  A step is one call of
the whole layer (routing plan or routing lookup, gate_up + SwiGLU, down,
combine) on one batch of resident synthetic inputs.  Each step uses a fresh
routing and one of several copies of the weights, chosen so that the weights
a step reads were not read by any of the recent steps; the MI355X's 256 MB
last-level cache therefore cannot serve them, and they stream from HBM as in
a real decode loop.

Two passes over the same steps:
  A. the timed region: W untimed warm-up steps, then exactly K steps between
     two synchronisations (value, ms_per_step, per-call percentiles);
  B. the same K steps with the library's stage-timing recorder on: a HIP
     event on the kernel's own stream before every kernel and after the
     last, giving every kernel's mean duration.  The dominant kernel's
     algorithmic bytes (or flops) per launch over that duration is
     `roofline.achieved`.
`roofline.traffic` is the HBM bytes per launch of that kernel from the
committed rocprofv3 counter summary of this workload
(profiles/hbm_<workload>.json, FETCH_SIZE and WRITE_SIZE scaled by a plain
copy kernel), or null when the kernel sources changed since it was taken.

Prints one JSON line.  --config picks another workload (ocr2_decode_t4,
ocr2_prefill, v3_fp8_decode, v3_fp8_prefill, tiny, ocr2_prefill_shared /
ocr2_decode_t1_shared with the model's two shared experts, and
v3_mxfp4_decode / v3_mxfp4_prefill with MXFP4 weights).

By default the line also carries `all_configs`: every other workload measured
the same way (passes A and B, fewer steps), so that each configuration has a
number from the same run; --only skips them.

Helper modes:
  --probe                   ceiling probes: a plain streaming read of the
                            decode workloads' weight bytes, dense torch GEMMs
  --copy-calibration        a plain 256 MiB device copy, for counter scaling
  --summarize-stats CSV     markdown table from a rocprofv3 kernel_stats.csv
  --summarize-pmc ...       HBM bytes per kernel from FETCH_SIZE/WRITE_SIZE runs
"""

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-experts µs/call + tokens/s; % HBM peak (decode), % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0
# Dense MFMA peaks.  The MXFP4 layer multiplies E4M3 activations by E2M1
# weights; a scaled MFMA with an fp8 operand issues at the fp8 rate, so its
# peak is fp8's (the fp4 figure holds for fp4 x fp4 only).
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 5000.0}
# default warm-up: at least this much work before the timed steps (a GPU
# under sustained load settles on its steady clocks after tens of ms)
kWarmupSeconds = 0.1
kWarmupMaxSteps = 1000
# The model card's own decode figure for exactly this workload (T=1, H=1280,
# F=896, 64 experts, top-6, bf16): 0.191 ms per call on an NVIDIA GB10.
PAGE_DECODE_T1_TOKENS_PER_S = 1.0 / 0.191e-3

# kernel-name prefix -> stage, for matching rocprofv3 rows to recorder stages
KERNEL_STAGES = [
    ("moe::plan_kernel", "plan"),
    ("moe::decode_kernel", "decode"),
    ("moe::combine_kernel", "combine"),
    ("moe::gemm_bf16_kernel<", "gemm_bf16"),
    ("moe::gemm_fp8_kernel<", "gemm_fp8"),
    ("moe::gemm_mx_kernel<", "gemm_mx"),
    ("moe::gemm_mx_wide_kernel<", "gemm_mx"),
    ("moe::quantize_kernel", "quantize"),
    ("moe::augment_routing_kernel", "shared_route"),
    ("moe::route_kernel", "router"),
    ("moe::route_plan_kernel", "route_plan"),
    ("moe::layer_bf16_kernel", "layer"),
    ("moe::layer_fp8_kernel", "layer"),
    ("moe::layer_mx_kernel", "layer"),
]


def kernel_stage(name):
    name = name.replace("void ", "").split("(")[0]
    for prefix, stage in KERNEL_STAGES:
        if name.startswith(prefix):
            if stage.startswith("gemm"):   # the first bool template argument is SWIGLU
                targs = name[name.find("<") + 1:name.rfind(">")].replace(" ", "").split(",")
                flags = [t for t in targs if t in ("true", "false")]
                return "gate_up" if flags and flags[0] == "true" else "down"
            return stage
    return None


def source_digest():
    """sha256 over the kernel sources and the C header: counter figures taken
    under another digest no longer describe these kernels."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "mixture_experts_routed_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="ocr2_decode_t1")
    ap.add_argument("--sets", type=int, default=None, help="weight copies rotated over steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stage-pass", action="store_true", help="skip pass B (profiling runs)")
    ap.add_argument("--all-configs", dest="all_configs", action="store_true", default=True,
                    help="also measure every other workload compactly (the default)")
    ap.add_argument("--only", dest="all_configs", action="store_false",
                    help="measure the chosen workload only")
    ap.add_argument("--probe", action="store_true",
                    help="only run the ceiling probes (plain streaming reads, dense GEMMs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (calibrates HBM counters)")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("CSV", "TITLE", "COMMAND"))
    ap.add_argument("--summarize-pmc", nargs=6,
                    metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV",
                             "COMMAND"))
    return ap.parse_args()


# ------------------------------------------------------------ helper modes
def copy_calibration():
    """A plain copy of a known size: under rocprofv3 --pmc its FETCH_SIZE and
    WRITE_SIZE per dispatch give the counters' scale (expect 262144 KiB each)."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        flush.fill_(0)            # evict src/dst from the 256 MB last-level cache
        torch.cuda.synchronize()
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n}), flush=True)


def summarize_stats(path, title, command):
    rows = list(csv.DictReader(open(path)))
    print(f"# {title}\n\ncommand: `{command}`\n")
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"].split("(")[0].replace("void ", "")
        if not name.startswith("moe::") and "copyBuffer" not in name:
            continue
        print(f"| {name} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
              f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | {float(r['Percentage']):.1f}% |")


def _per_kernel(path, counter):
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"].split("(")[0].replace("void ", "")].append(float(r["Counter_Value"]))
    return vals


def summarize_pmc(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, command):
    """Per-kernel HBM bytes per dispatch: FETCH_SIZE and WRITE_SIZE (KiB) of
    each moe:: kernel, scaled by what the same counters read for a plain
    256 MiB copy.  Writes JSON (with the kernel-source digest) to stdout."""
    copy_kib = 256 * 1024
    cf = _per_kernel(copy_fetch_csv, "FETCH_SIZE")["__amd_rocclr_copyBuffer"]
    cw = _per_kernel(copy_write_csv, "WRITE_SIZE")["__amd_rocclr_copyBuffer"]
    f_scale = copy_kib / max(cf)   # the largest dispatch is the 256 MiB copy
    w_scale = copy_kib / max(cw)
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    out = {"workload": workload, "command": command, "source_sha256": source_digest(),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "stages": {}}
    for k in sorted(fetch):
        st = kernel_stage(k)
        if st is None:
            continue
        f = sum(fetch[k]) / len(fetch[k])
        w = sum(write.get(k, [0.0])) / max(len(write.get(k, [])), 1)
        out["stages"][st] = {"kernel": k, "fetch_kib": round(f, 1), "write_kib": round(w, 1),
                             "hbm_bytes": int((f * f_scale + w * w_scale) * 1024)}
    print(json.dumps(out, indent=1))


# ------------------------------------------------------------ algorithmic work
def stage_work(stage, kind, T, H, F, k, touched, valid):
    """Algorithmic (bytes, flops) of one launch of `stage`: the weights of the
    touched experts it reads (with their block scales: fp32 per 128 for fp8,
    one E8M0 byte per 32 for mxfp4) plus the layer inputs/outputs it reads or
    writes; intermediates (h, y, partial sums) are implementation overhead and
    are not counted."""
    if kind == "mxfp4":
        bw, sc = 0.5, 1.0 / 32                       # E2M1 pairs + E8M0 per 32
        x_bytes = T * H * (1 + 1.0 / 32)             # E4M3 + E8M0 per 32
    else:
        bw = 2 if kind == "bf16" else 1
        sc = 0 if kind == "bf16" else 4.0 / 128
        x_bytes = T * H * bw + (0 if kind == "bf16" else T * (H // 128) * 4)
    out_bytes = T * H * 2
    route_bytes = T * k * 8
    gu_w = touched * 2 * F * H * (bw + sc)
    dn_w = touched * H * F * (bw + sc)
    if stage == "plan":
        return T * k * 4, 0
    if stage == "gate_up":
        return gu_w + x_bytes, 2 * valid * 2 * F * H
    if stage == "down":
        return dn_w, 2 * valid * H * F
    if stage == "combine":
        return out_bytes + route_bytes, 2 * valid * H
    if stage in ("decode", "layer"):   # the whole layer in one launch
        return gu_w + dn_w + x_bytes + out_bytes + route_bytes, 2 * valid * 3 * F * H
    if stage == "shared_route":
        return route_bytes, 0
    raise ValueError(stage)


def algorithmic_bytes(kind, T, H, F, k, touched):
    """Bytes the whole layer must move once (every stage's share)."""
    stages = ["gate_up", "down", "combine"]   # the plan's id read is in the combine's share
    return sum(stage_work(s, kind, T, H, F, k, touched, 0)[0] for s in stages)


def algorithmic_flops(valid_slots, H, F):
    return 2 * valid_slots * 3 * F * H


def roofline_for(stage, kind, dtype, bytes_, flops, ms):
    ridge = MFMA_PEAK_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    secs = ms * 1e-3
    if flops > 0 and flops / max(bytes_, 1) > ridge:
        ach = flops / secs / 1e12
        peak = MFMA_PEAK_TFLOPS[dtype]
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4)}
    ach = bytes_ / secs / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4)}


def committed_traffic(workload, stage):
    """HBM bytes per launch of `stage` from the committed counter summary, or
    None if there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_sha256") != source_digest():
        return None
    st = d.get("stages", {}).get(stage)
    return None if st is None else int(st["hbm_bytes"])


# ------------------------------------------------------------ main
# the workloads the default run also measures (compactly) beside the headline
ALL_CONFIGS = ["tiny", "ocr2_decode_t1", "ocr2_decode_t4", "ocr2_prefill", "v3_fp8_decode",
               "v3_fp8_prefill", "ocr2_prefill_shared", "ocr2_decode_t1_shared", "v3_mxfp4_decode",
               "v3_mxfp4_prefill"]


def default_steps(name, kind):
    decode = name.startswith("ocr2_decode") or name == "tiny"
    return 200 if decode else (20 if kind == "bf16" else 10)


def measure(moe, torch, np, wl, name, steps, warmup, sets_arg=None, stage_pass=True, extras=True):
    """One workload: pass A (timed steps), pass B (per-kernel stage times),
    and, with `extras`, the router pass and the router-fused decode pass.
    Returns (bench dict, context for the CPU baseline)."""
    cfg = dict(wl.CONFIGS[name])
    T, H, F, E, k, kind = cfg["T"], cfg["H"], cfg["F"], cfg["E"], cfg["k"], cfg["kind"]
    S = cfg.get("S", 0)   # shared experts (every token, weight 1)
    decode = name.startswith("ocr2_decode") or name == "tiny"
    explicit_warmup = warmup is not None
    warmup = warmup if explicit_warmup else 20
    dev = torch.device("cuda:0")

    # ---------------------------------------------------------------- inputs
    n_route = steps + warmup
    routes = []
    hidden = gu_sets = dn_sets = None
    if kind == "bf16":
        base = wl.make_config(name, device="cpu")
        weight_bytes = sum(base[n].numel() * 2 for n in ("gate_up", "down", "shared_gate_up", "shared_down")
                           if n in base)
        sets = sets_arg or (16 if decode else max(1, min(16, int(np.ceil(2.5e9 / weight_bytes)))))
        gu_sets = [base["gate_up"].to(dev) for _ in range(sets)]
        dn_sets = [base["down"].to(dev) for _ in range(sets)]
        hidden = base["hidden"].to(dev)
        for i in range(n_route):
            g = wl._gen(cfg["seed"] * 1000 + i, "cpu")
            idx, w = wl.route_uniform_softmax(T, E, k, g, "cpu", cfg["routed_scale"])
            routes.append((idx.to(dev), w.to(dev)))
        # routing on the host too (the CPU baseline reads it; no copies while timed)
        host_routes = [(i.cpu().numpy(), w.cpu().numpy().astype(np.float64)) for i, w in routes]
        out_buf = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        if S:   # the shared experts' weights rotate with the routed ones
            sgu_sets = [base["shared_gate_up"].to(dev) for _ in range(sets)]
            sdn_sets = [base["shared_down"].to(dev) for _ in range(sets)]
            entry_sh = moe.moe_experts_decode_shared if decode else moe.moe_experts_prefill_shared

            def step(i):
                s = i % sets
                idx, w = routes[i % len(routes)]
                return entry_sh(hidden, gu_sets[s], dn_sets[s], sgu_sets[s], sdn_sets[s], idx, w, k,
                                out=out_buf)
        else:
            entry = moe.moe_experts_decode if decode else moe.moe_experts_prefill

            def step(i):
                s = i % sets
                idx, w = routes[i % len(routes)]
                return entry(hidden, gu_sets[s], dn_sets[s], idx, w, k, out=out_buf)
        dtype = "bf16"
        problem = base
    else:
        p = wl.make_config(name, device=dev)
        sets = 1
        routes = [(p["top_k_index"], p["top_k_weights"])] * n_route
        host_routes = [(p["top_k_index"].cpu().numpy(), p["top_k_weights"].cpu().numpy())] * n_route
        out_buf = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        entry = moe.moe_experts_mxfp4 if kind == "mxfp4" else moe.moe_experts_fp8

        def step(i):
            return entry(p["x"], p["x_scale"], p["gate_up"], p["gate_up_scale"], p["down"],
                         p["down_scale"], p["top_k_index"], p["top_k_weights"], k, out=out_buf)
        dtype = kind
        problem = p
    torch.cuda.synchronize()

    # ------------------------------------------------------- pass A: timing
    # The GPU reaches its steady clocks only after tens of milliseconds of
    # sustained load (a T=2048 bf16 prefill call runs about 20% faster then),
    # so the default warm-up runs at least kWarmupSeconds of steps (at most
    # kWarmupMaxSteps); the steps run are reported as "warmup".
    t0 = time.perf_counter()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    if not explicit_warmup:
        per_step = (time.perf_counter() - t0) / warmup
        extra = min(kWarmupMaxSteps, max(warmup, int(kWarmupSeconds / per_step) + 1)) - warmup
        for i in range(warmup, warmup + extra):
            step(i)
        warmup += extra
        torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(steps):
        step(warmup + i)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / steps

    # ------------------------------------------------------ algorithmic work
    touched_l, valid_l = [], []
    for i in range(steps):
        idx = host_routes[(warmup + i) % len(host_routes)][0].reshape(-1)
        valid = idx[(idx >= 0) & (idx < E)]
        touched_l.append(len(np.unique(valid)) + S)     # shared experts: every token
        valid_l.append(valid.size + T * S)
    touched, valid = float(np.mean(touched_l)), float(np.mean(valid_l))
    mean_bytes = algorithmic_bytes(kind, T, H, F, k, touched)
    mean_flops = algorithmic_flops(valid, H, F)
    mean_us = ms_per_step * 1e3

    # ------------------------------------- pass B: per-kernel stage timing
    stages = {}
    if stage_pass:
        moe.moe_profile_begin(steps)
        for i in range(steps):
            step(warmup + i)
        torch.cuda.synchronize()
        calls = moe.moe_profile_end(steps)
        per = collections.defaultdict(list)
        for row in calls:
            for st, ms in row:
                per[st].append(ms)
        stages = {st: float(np.mean(v)) for st, v in per.items()}
        kernel_us = np.array([sum(ms for _, ms in row) * 1e3 for row in calls])

    out = {
        "metric": METRIC,
        "value": None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded generators; random-init weights of the named shapes)",
        "config": {"workload": name, "T": T, "H": H, "F": F, "E": E, "top_k": k,
                   "shared_experts": S, "weight_copies_rotated": sets},
    }
    value = T / (ms_per_step * 1e-3)
    out["value"] = round(value, 1)
    out["vs_baseline"] = round(value / PAGE_DECODE_T1_TOKENS_PER_S, 3) if name == "ocr2_decode_t1" else None
    out["us_per_call"] = round(mean_us, 2)
    if stages:   # kernel time per call (pass B), without the gaps between launches
        out["kernel_us_per_call"] = {"mean": round(float(kernel_us.mean()), 2),
                                     "p10": round(float(np.percentile(kernel_us, 10)), 2),
                                     "p50": round(float(np.percentile(kernel_us, 50)), 2),
                                     "p90": round(float(np.percentile(kernel_us, 90)), 2)}
    out["layer"] = {"algorithmic_bytes_per_call": int(mean_bytes),
                    "algorithmic_flops_per_call": int(mean_flops),
                    "touched_experts": round(touched, 2),
                    "hbm_GBps": round(mean_bytes / (mean_us * 1e-6) / 1e9, 1),
                    "TFLOPps": round(mean_flops / (mean_us * 1e-6) / 1e12, 3)}
    if stages:
        out["stage_us"] = {st: round(ms * 1e3, 2) for st, ms in stages.items()}
        dom = max(stages, key=stages.get)
        b, f = stage_work(dom, kind, T, H, F, k, touched, valid)
        roof = roofline_for(dom, kind, dtype, b, f, stages[dom])
        roof["traffic"] = committed_traffic(name, dom)
        roof["kernel"] = dom
        roof["kernel_us"] = round(stages[dom] * 1e3, 2)
        roof["algorithmic_bytes_per_launch"] = int(b)
        roof["algorithmic_flops_per_launch"] = int(f)
        out["roofline"] = roof

    # ------------------------------------------- pass C: router (+ plan)
    if extras and stage_pass:
        out["router"] = router_pass(moe, torch, np, name, kind, T, E, k, cfg, steps, warmup)
        if decode and kind == "bf16" and not S:
            # pass D: the same decode steps from router logits, the routing
            # fused into the decode kernel (moe_experts_decode_routed, its own
            # kernel instantiation)
            gl = torch.Generator().manual_seed(cfg["seed"] + 78)
            logit_sets = [(torch.randn(T, E, generator=gl) * 2).to(dev) for _ in range(n_route)]

            def step_routed(i):
                s_ = i % sets
                return moe.moe_experts_decode_routed(hidden, logit_sets[i % len(logit_sets)], gu_sets[s_],
                                                     dn_sets[s_], k,
                                                     mode=moe.MOE_ROUTE_SOFTMAX,
                                                     routed_scaling_factor=cfg["routed_scale"])
            for i in range(warmup):
                step_routed(i)
            torch.cuda.synchronize()
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record()
            for i in range(steps):
                step_routed(warmup + i)
            ev1.record()
            torch.cuda.synchronize()
            moe.moe_profile_begin(steps)
            for i in range(steps):
                step_routed(warmup + i)
            torch.cuda.synchronize()
            calls = moe.moe_profile_end(steps)
            out["router"]["decode_routed"] = {
                "entry": "moe_experts_decode_routed (softmax router fused into the decode kernel)",
                "us_per_call": round(ev0.elapsed_time(ev1) / steps * 1e3, 2),
                "kernel_us_per_call": round(float(np.mean([sum(ms for _, ms in row) for row in calls])) * 1e3, 2),
                "launches": len(calls[0]) if calls else 0}
    # ------------------------------ pass E: the single-kernel form, if any
    if stage_pass:
        fused_entry = None
        if kind == "bf16" and not decode and not S:
            fused_entry = "moe_experts_prefill_fused"

            def step_fused(i):
                s_ = i % sets
                idx, w = routes[i % len(routes)]
                return moe.moe_experts_prefill_fused(hidden, gu_sets[s_], dn_sets[s_], idx, w, k,
                                                     out=out_buf)
        elif kind == "fp8" and T * k > 32 * E:
            fused_entry = "moe_experts_fp8_fused"

            def step_fused(i):
                return moe.moe_experts_fp8_fused(p["x"], p["x_scale"], p["gate_up"], p["gate_up_scale"],
                                                 p["down"], p["down_scale"], p["top_k_index"],
                                                 p["top_k_weights"], k, out=out_buf)
        elif kind == "mxfp4" and T * k > 64 * E:
            fused_entry = "moe_experts_mxfp4_fused"

            def step_fused(i):
                return moe.moe_experts_mxfp4_fused(p["x"], p["x_scale"], p["gate_up"],
                                                   p["gate_up_scale"], p["down"], p["down_scale"],
                                                   p["top_k_index"], p["top_k_weights"], k,
                                                   out=out_buf)
        if fused_entry:
            # pass E: the same steps through the one-launch form (the plan,
            # then gate_up, down and the combine in one persistent launch)
            for i in range(warmup):
                step_fused(i)
            torch.cuda.synchronize()
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record()
            for i in range(steps):
                step_fused(warmup + i)
            ev1.record()
            torch.cuda.synchronize()
            moe.moe_profile_begin(steps)
            for i in range(steps):
                step_fused(warmup + i)
            torch.cuda.synchronize()
            calls = moe.moe_profile_end(steps)
            per = collections.defaultdict(list)
            for row in calls:
                for st, ms in row:
                    per[st].append(ms)
            out["fused_layer"] = {
                "entry": f"{fused_entry} (one persistent launch: plan, both products, combine)",
                "us_per_call": round(ev0.elapsed_time(ev1) / steps * 1e3, 2),
                "kernel_us_per_call": round(float(np.mean([sum(ms for _, ms in row) for row in calls])) * 1e3, 2),
                "stage_us": {st: round(float(np.mean(v)) * 1e3, 2) for st, v in per.items()}}
            if "layer" in per:   # its roofline: the whole layer's work per launch
                lms = float(np.mean(per["layer"]))
                lb, lf = stage_work("layer", kind, T, H, F, k, touched, valid)
                lroof = roofline_for("layer", kind, dtype, lb, lf, lms)
                lroof["traffic"] = committed_traffic(name, "layer")
                lroof["kernel_us"] = round(lms * 1e3, 2)
                out["fused_layer"]["roofline"] = lroof
    ctx = (cfg, host_routes, warmup, problem)
    return out, ctx


def summary_of(out):
    """The compact per-workload entry of the headline line."""
    r = out.get("roofline", {})
    return {"us_per_call": out["us_per_call"], "tokens_per_s": out["value"], "steps": out["steps"],
            "kernel_us_per_call": out.get("kernel_us_per_call", {}).get("mean"),
            "layer_hbm_GBps": out["layer"]["hbm_GBps"], "layer_TFLOPps": out["layer"]["TFLOPps"],
            "dominant_kernel": r.get("kernel"), "dominant_kernel_us": r.get("kernel_us"),
            "roofline": {kk: r.get(kk) for kk in ("bound", "achieved", "peak", "unit", "frac")} if r else None,
            "stage_us": out.get("stage_us"),
            **({"fused_layer": {"us_per_call": out["fused_layer"]["us_per_call"],
                                "kernel_us": out["fused_layer"].get("roofline", {}).get("kernel_us"),
                                "roofline_frac": out["fused_layer"].get("roofline", {}).get("frac"),
                                "traffic": out["fused_layer"].get("roofline", {}).get("traffic")}}
               if "fused_layer" in out else {})}


def probe(moe, torch, np):
    """Ceiling probes, for context (never a denominator): a plain streaming
    read of 41.3 MB (the T=1 decode's weights) and of 143 MB (T=4), rotating
    over windows that together exceed the last-level cache, timed per launch;
    and dense torch GEMMs of the prefill workloads' flops (bf16, fp8)."""
    dev = torch.device("cuda:0")
    res = {}
    sink = torch.zeros(4096, dtype=torch.uint8, device=dev)
    buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    for label, nbytes in (("read_41MB", 41290240), ("read_143MB", 143 << 20)):
        nwin = (1 << 30) // nbytes
        wins = [buf[i * nbytes:(i + 1) * nbytes] for i in range(nwin)]
        for grid in (256, 512, 1024):
            for i in range(10):
                moe.moe_probe_stream_read(wins[i % nwin], grid, sink)
            torch.cuda.synchronize()
            n = 50
            moe.moe_profile_begin(n)
            for i in range(n):
                moe.moe_probe_stream_read(wins[i % nwin], grid, sink)
            torch.cuda.synchronize()
            us = np.array([row[0][1] * 1e3 for row in moe.moe_profile_end(n)])
            res[f"{label}_grid{grid}"] = {"us_mean": round(float(us.mean()), 2),
                                          "us_min": round(float(us.min()), 2),
                                          "GBps_mean": round(nbytes / (us.mean() * 1e-6) / 1e9, 1)}
    del buf, wins
    # dense GEMMs with the flops of the prefill layers' gate_up products
    for label, (M, N, K, dt) in {"bf16_12288x1792x1280": (12288, 1792, 1280, torch.bfloat16),
                                 "bf16_8192x8192x8192": (8192, 8192, 8192, torch.bfloat16),
                                 "fp8_32768x4096x7168": (32768, 4096, 7168, "fp8")}.items():
        if dt == "fp8":
            a = torch.randn(M, K, device=dev).to(torch.float8_e4m3fn)
            b = torch.randn(N, K, device=dev).to(torch.float8_e4m3fn).t()
            one = torch.ones((), device=dev)

            def run():
                return torch._scaled_mm(a, b, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        else:
            a = torch.randn(M, K, device=dev, dtype=dt)
            b = torch.randn(K, N, device=dev, dtype=dt)

            def run():
                return a @ b
        try:
            for _ in range(5):
                run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                run()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 20
            res[f"torch_gemm_{label}"] = {"ms": round(ms, 4), "TFLOPps": round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        except Exception as exc:   # a torch build without the fp8 product
            res[f"torch_gemm_{label}"] = {"error": str(exc)[:120]}
    return res


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_routed_amd as moe
    import moe_workloads as wl

    torch.cuda.set_device(torch.device("cuda:0"))
    moe._load()
    if args.probe:
        print(json.dumps({"probe": probe(moe, torch, np)}), flush=True)
        return

    name = args.config
    kind = wl.CONFIGS[name]["kind"]
    steps = args.steps if args.steps is not None else default_steps(name, kind)
    out, (cfg, host_routes, warmup, problem) = measure(
        moe, torch, np, wl, name, steps, args.warmup, args.sets, stage_pass=not args.no_stage_pass)

    # every other configuration, compactly (its own default steps, capped by --steps)
    if args.all_configs and not args.no_stage_pass:
        allc = {}
        for other in ALL_CONFIGS:
            if other == name:
                allc[other] = summary_of(out)
                continue
            o_kind = wl.CONFIGS[other]["kind"]
            o_steps = min(default_steps(other, o_kind), max(steps, 10))
            o_out, _ = measure(moe, torch, np, wl, other, o_steps, None, None, stage_pass=True,
                               extras=False)
            allc[other] = summary_of(o_out)
            del o_out
            torch.cuda.empty_cache()
        out["all_configs"] = allc

    # ------------------------------------------------------------ CPU oracle
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(name, cfg, args.cpu_seconds, host_routes, warmup, problem)
    print(json.dumps(out), flush=True)


def router_pass(moe, torch, np, name, kind, T, E, k, cfg, steps, warmup):
    """moe_route_plan on seeded logits of this workload's shape: the model
    card's softmax router for the OCR-2 shapes, the MegaKernel layer's
    group-aware sigmoid router (8 groups, 4 kept, bf16 logits and bias) for the
    V3 shapes.  Reported beside the layer (the layer itself takes ids)."""
    g = torch.Generator().manual_seed(cfg["seed"] + 77)
    if kind == "bf16":
        lg = (torch.randn(T, E, generator=g) * 2).cuda()
        kw = dict(mode=moe.MOE_ROUTE_SOFTMAX, routed_scaling_factor=cfg["routed_scale"])
        rule = "softmax"
    else:
        lg = (torch.randn(T, E, generator=g) * 2).to(torch.bfloat16).cuda()
        bias = (torch.randn(E, generator=g) * 0.1).to(torch.bfloat16).cuda()
        kw = dict(mode=moe.MOE_ROUTE_SIGMOID_GROUP, bias=bias, num_groups=8, topk_group=4,
                  group_top=2, routed_scaling_factor=cfg["routed_scale"])
        rule = "sigmoid_group(8 groups, 4 kept, top-2 group score)"
    for _ in range(warmup):
        moe.moe_route_plan(lg, k, **kw)
    torch.cuda.synchronize()
    moe.moe_profile_begin(steps)
    for _ in range(steps):
        moe.moe_route_plan(lg, k, **kw)
    torch.cuda.synchronize()
    calls = moe.moe_profile_end(steps)
    per = collections.defaultdict(list)
    for row in calls:
        for st, ms in row:
            per[st].append(ms)
    return {"entry": "moe_route_plan", "rule": rule, "launches": len(calls[0]) if calls else 0,
            "kernel_us": {st: round(float(np.mean(v)) * 1e3, 2) for st, v in per.items()},
            "kernel_us_total": round(float(np.mean([sum(ms for _, ms in row) for row in calls])) * 1e3, 2)}


def cpu_baseline(name, cfg, seconds, routes, warmup, problem):
    """The oracle as it stands, timed on this host over a bounded sample of the
    same workload, scaled to tokens/s."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as orc

    T, E, k = cfg["T"], cfg["E"], cfg["k"]
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    if cfg["kind"] == "bf16":
        x = problem["hidden"].float().numpy().astype(np.float64)
        w13 = problem["gate_up"].float().numpy().astype(np.float64)
        w2 = problem["down"].float().numpy().astype(np.float64)
        sh = {}
        if "shared_gate_up" in problem:
            sh = dict(shared_gate_up=problem["shared_gate_up"].float().numpy().astype(np.float64),
                      shared_down=problem["shared_down"].float().numpy().astype(np.float64))
        done_tokens, calls = 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            idx, w = routes[(warmup + calls) % len(routes)]   # host copies, made before timing
            if T <= 16:
                orc.moe_experts_reference(x, w13, w2, idx, w, **sh)
                done_tokens += T
            else:   # a bounded sample: the first 64 tokens through the per-token loop
                n = min(64, T)
                orc.moe_experts_reference(x[:n], w13, w2, idx[:n], w[:n], **sh)
                done_tokens += n
            calls += 1
        el = time.perf_counter() - t0
        sample = f"{calls} oracle calls, {done_tokens} tokens, per-token float64 loop"
    else:
        # per-expert dequantisation dominates; sample 2 tokens of the real problem
        import torch
        tokens = [0, 1]
        p = problem
        hp = {n: p[n] for n in ("x", "x_scale", "top_k_index", "top_k_weights")}

        class Lazy:
            def __init__(self, t):
                self.t, self.shape = t, tuple(t.shape)

            def __getitem__(self, e):
                return self.t[int(e)].cpu().numpy()
        ref = (orc.moe_experts_mxfp4_reference if cfg["kind"] == "mxfp4"
               else orc.moe_experts_fp8_reference)
        host = [hp[n].cpu().numpy() for n in ("x", "x_scale", "top_k_index", "top_k_weights")]
        t0 = time.perf_counter()
        ref(host[0], host[1], Lazy(p["gate_up"]), Lazy(p["gate_up_scale"]), Lazy(p["down"]),
            Lazy(p["down_scale"]), host[2], host[3], tokens=tokens)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        done_tokens = len(tokens)
        sample = f"{len(tokens)} tokens of the same problem (each selected expert dequantised once)"
    return {"value": round(done_tokens / el, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "sample": sample, "seconds": round(el, 2),
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
