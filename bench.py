"""Benchmark of the routed-experts MoE layer on one MI355X.

Default workload: DeepSeek-OCR-2-shaped decode, T=1 token, H=1280, F=896,
64 experts, top-6, bf16 (the gather-GEMV entry point).  A step is one call of
the whole layer (plan, gate_up + SwiGLU, down, combine) on one batch of
resident synthetic inputs.  Each step uses a fresh routing and one of several
copies of the weights, chosen so that the weights a step reads were not read
by any of the recent steps; the MI355X's 256 MB last-level cache therefore
cannot serve them, and they stream from HBM as in a real decode loop.

Prints one JSON line.  --config picks another workload (ocr2_decode_t4,
ocr2_prefill, v3_fp8_decode, v3_fp8_prefill, tiny).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-experts µs/call + tokens/s; % HBM peak (decode), % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
# The model card's own decode figure for exactly this workload (T=1, H=1280,
# F=896, 64 experts, top-6, bf16): 0.191 ms per call on an NVIDIA GB10.
PAGE_DECODE_T1_TOKENS_PER_S = 1.0 / 0.191e-3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="ocr2_decode_t1")
    ap.add_argument("--sets", type=int, default=None, help="weight copies rotated over steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (calibrates HBM counters)")
    return ap.parse_args()


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


def algorithmic_bytes(kind, T, H, F, k, touched):
    """Bytes the layer must move once: the touched experts' weights (plus
    their fp32 block scales for fp8), activations in, bf16 out, routing."""
    if kind == "bf16":
        w = touched * 3 * F * H * 2
        act = T * H * 2
    else:
        w = touched * (3 * F * H + 3 * F * H // 128 * 4)
        act = T * H + T * (H // 128) * 4
    return w + act + T * H * 2 + T * k * 8


def algorithmic_flops(valid_slots, H, F):
    return 2 * valid_slots * 3 * F * H


def main():
    args = parse()
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

    cfg = dict(wl.CONFIGS[args.config])
    name = args.config
    T, H, F, E, k, kind = cfg["T"], cfg["H"], cfg["F"], cfg["E"], cfg["k"], cfg["kind"]
    decode = name.startswith("ocr2_decode") or name == "tiny"
    steps = args.steps if args.steps is not None else (200 if decode else (20 if kind == "bf16" else 10))
    warmup = args.warmup if args.warmup is not None else (20 if decode else 3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe._load()

    # ---------------------------------------------------------------- inputs
    n_route = steps + warmup
    routes = []
    if kind == "bf16":
        base = wl.make_config(name, device="cpu")
        weight_bytes = base["gate_up"].numel() * 2 + base["down"].numel() * 2
        sets = args.sets or (16 if decode else max(1, min(16, int(np.ceil(2.5e9 / weight_bytes)))))
        gu_sets = [base["gate_up"].to(dev) for _ in range(sets)]
        dn_sets = [base["down"].to(dev) for _ in range(sets)]
        hidden = base["hidden"].to(dev)
        for i in range(n_route):
            g = wl._gen(cfg["seed"] * 1000 + i, "cpu")
            idx, w = wl.route_uniform_softmax(T, E, k, g, "cpu", cfg["routed_scale"])
            routes.append((idx.to(dev), w.to(dev)))
        entry = moe.moe_experts_decode if decode else moe.moe_experts_prefill

        def step(i):
            s = i % sets
            idx, w = routes[i]
            return entry(hidden, gu_sets[s], dn_sets[s], idx, w, k)
        dtype = "bf16"
    else:
        p = wl.make_config(name, device=dev)
        sets = 1
        routes = [(p["top_k_index"], p["top_k_weights"])] * n_route

        def step(i):
            return moe.moe_experts_fp8(p["x"], p["x_scale"], p["gate_up"], p["gate_up_scale"],
                                       p["down"], p["down_scale"], p["top_k_index"],
                                       p["top_k_weights"], k)
        dtype = "fp8"
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timing
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        ev[i][0].record()
        step(warmup + i)
        ev[i][1].record()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per_call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    ms_per_step = total_ms / steps

    # ------------------------------------------------------ algorithmic work
    bytes_per_call, flops_per_call = [], []
    for i in range(steps):
        idx = routes[warmup + i][0].cpu().numpy().reshape(-1)
        valid = idx[(idx >= 0) & (idx < E)]
        bytes_per_call.append(algorithmic_bytes(kind, T, H, F, k, len(np.unique(valid))))
        flops_per_call.append(algorithmic_flops(valid.size, H, F))
    mean_bytes = float(np.mean(bytes_per_call))
    mean_flops = float(np.mean(flops_per_call))
    mean_us = float(per_call_us.mean())

    hbm_gbs = mean_bytes / (mean_us * 1e-6) / 1e9
    tflops = mean_flops / (mean_us * 1e-6) / 1e12
    bound = "hbm" if (decode or name == "v3_fp8_decode" or name == "ocr2_prefill") else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        peak = MFMA_PEAK_TFLOPS[dtype]
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4), "traffic": None}
    roof["kernel"] = "whole layer per call (HIP events around each call)"

    value = T / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / PAGE_DECODE_T1_TOKENS_PER_S, 3) if name == "ocr2_decode_t1" else None),
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": name, "T": T, "H": H, "F": F, "E": E, "top_k": k,
                   "weight_copies_rotated": sets},
        "us_per_call": {"mean": round(mean_us, 2), "p10": round(float(np.percentile(per_call_us, 10)), 2),
                        "p50": round(float(np.percentile(per_call_us, 50)), 2),
                        "p90": round(float(np.percentile(per_call_us, 90)), 2)},
        "algorithmic": {"bytes_per_call": int(mean_bytes), "flops_per_call": int(mean_flops),
                        "hbm_GBps": round(hbm_gbs, 1), "TFLOPps": round(tflops, 3)},
        "roofline": roof,
    }

    # ------------------------------------------------------------ CPU oracle
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(name, cfg, args.cpu_seconds, routes, warmup,
                                           base if kind == "bf16" else p)
    print(json.dumps(out), flush=True)


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
        done_tokens, calls = 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            idx, w = routes[(warmup + calls) % len(routes)]
            idx = idx.cpu().numpy()
            w = w.cpu().numpy().astype(np.float64)
            if T <= 16:
                orc.moe_experts_reference(x, w13, w2, idx, w)
                done_tokens += T
            else:   # a bounded sample: the first 64 tokens through the per-token loop
                n = min(64, T)
                orc.moe_experts_reference(x[:n], w13, w2, idx[:n], w)
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
        t0 = time.perf_counter()
        orc.moe_experts_fp8_reference(hp["x"].cpu().numpy(), hp["x_scale"].cpu().numpy(),
                                      Lazy(p["gate_up"]), Lazy(p["gate_up_scale"]),
                                      Lazy(p["down"]), Lazy(p["down_scale"]),
                                      hp["top_k_index"].cpu().numpy(),
                                      hp["top_k_weights"].cpu().numpy(), tokens=tokens)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        done_tokens = len(tokens)
        sample = f"{len(tokens)} tokens of the same problem (each selected expert dequantised once)"
    return {"value": round(done_tokens / el, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "sample": sample, "seconds": round(el, 2),
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
