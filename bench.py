#!/usr/bin/env python3
"""Benchmark of one sparse-MoE FFN layer forward on one MI355X.

A step is one whole-layer forward (router logits, gate, Top-K, histogram /
capacity / permutation, dispatch, grouped SwiGLU experts, shared expert,
combine) through ``moe_forward`` of the C-ABI library, on seeded synthetic
inputs already resident in HBM.  Default workload: the largest one, a
DeepSeek-V3-style fine-grained layer (T=4096, d_model=7168, 256 routed
experts of d_ff=2048, sigmoid gate with a selection bias, Top-8
renormalised, one shared expert of d_ff=2048, bf16, fp32 router).

Expert weights are packed once by ``moe_pack_weights`` before anything is
timed, for the GEMMs the workload's default names (``--packed``; the line's
``config.packed_weights`` and ``weight_pack_ms`` report the choice and its
one-time cost).

Prints one JSON line: tokens/s, the dominant kernel's roofline position
(measured with HIP events on the launch stream inside the timed region), the
whole layer's flops and bytes rates, and the CPU oracle timed on a bounded
sample of the same workload.

Byte and flop accounting (per launch):
  algorithmic  what the method must move: a grouped-GEMM launch reads the
               weights of every expert it touches once (W1 and W3 for GEMM1,
               W2 for GEMM2; E4M3 row scales included), 2*R*d*F flops per
               weight matrix for R rows.  The layer: router 2*T*d*E, experts
               6*d*F per kept row, shared expert 6*d*Fs per token; bytes: the
               touched experts' and the shared expert's weights, x, y, W_g.
  implementation  what this implementation moves besides: the dispatched rows
               read by GEMM1, h written by GEMM1 and read by GEMM2, the fp32
               expert rows written by GEMM2 (reported separately, never in
               the roofline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/sec; achieved MFMA TFLOP/s (prefill) and HBM GB/s (decode)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
DEFAULT_WORKLOAD = "deepseek_v3_fine"
EVENT_EVERY = 4               # the dominant kernel is event-timed in the last step of every 4
# Which GEMMs' weights a bf16 workload's weights are packed for (moe_pack_weights), by default: the
# layout its GEMMs stream fastest with the plans the library takes for each (same box, alternating runs,
# against row-major weights): DeepSeek-style GEMM1 3.62 -> 3.46 ms, GEMM2 1.93 -> 1.89 ms; prefill GEMM1
# 1.80 -> 1.76 ms, GEMM2 908 -> 889 us; Switch GEMM1 235 -> 228 us, GEMM2 132 -> 118 us; decode GEMM2
# 178 -> 169 us, GEMM1 294 -> 313 us (so decode keeps W1 / W3 row-major).
DEFAULT_PACKING = {"deepseek_v3_fine": "both", "mixtral_prefill": "both", "switch_top1_capacity": "both",
                   "mixtral_decode": "down"}
# E4M3 expert weights likewise (same box, alternating runs, layer ms row-major -> packed): DeepSeek-style
# 5.11-5.12 -> 5.01 (W1 / W3; all: 5.05), prefill 2.83 -> 2.71-2.73 (all), decode 0.414-0.416 -> 0.396-0.399
# (W1 / W3), Switch 0.366-0.375 -> 0.345 (all).
DEFAULT_PACKING_FP8 = {"deepseek_v3_fine": "up", "mixtral_prefill": "both", "switch_top1_capacity": "both",
                       "mixtral_decode": "up"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--tokens", type=int, default=0, help="override the workload's token count (a size sweep)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="also time every kernel in an untimed extra pass")
    ap.add_argument("--stats", action="store_true", help="also compute the fused router statistics every step")
    ap.add_argument("--drop-policy", default="first_come", choices=["first_come", "affinity", "reroute"],
                    help="which assignments an expert over capacity drops")
    ap.add_argument("--expert-choice", action="store_true", help="expert-choice routing instead of token choice")
    ap.add_argument("--fp8", action="store_true", help="FP8 E4M3 expert weights with per-row scales")
    ap.add_argument("--packed", default="auto", choices=["auto", "none", "up", "down", "both"],
                    help="which GEMMs' expert weights moe_pack_weights packs once before timing (bf16 or E4M3); "
                         "auto: the layout measured fastest for the workload")
    return ap.parse_args()


GEMM_SOURCES = ("gemm_bf16.h", "gemm_bf16_up.hip", "gemm_bf16.hip")


def gemm_source_hash() -> str:
    """sha256[:16] of the grouped-GEMM kernel and launcher sources."""
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_sparse_route_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_accounting(wl, R: int, touched: int):
    """Algorithmic flops and bytes per launch of each GEMM of one step, and
    the implementation bytes beside them (see the module docstring)."""
    esz = 2 if wl.dtype == "bf16" else 4           # activations
    fp8 = wl.wdtype == "fp8"
    wsz = 1 if fp8 else esz                         # expert weights
    d, F = wl.d, wl.F
    sc_up = 2.0 * F * 4 if fp8 else 0.0             # fp32 row scales of W1, W3
    sc_dn = d * 4.0 if fp8 else 0.0                 # of W2
    acc = {
        "gemm_gate_up": dict(flops=4.0 * d * F * R, bytes=touched * (2.0 * F * d * wsz + sc_up),
                             impl_bytes=R * d * esz + R * F * esz),
        "gemm_down": dict(flops=2.0 * d * F * R, bytes=touched * (1.0 * F * d * wsz + sc_dn),
                          impl_bytes=R * F * esz + R * d * 4.0),
    }
    if wl.n_shared:
        Fs, T = wl.Fs, wl.T
        acc["shared_gate_up"] = dict(flops=4.0 * d * Fs * T, bytes=2.0 * Fs * d * wsz + (2.0 * Fs * 4 if fp8 else 0.0),
                                     impl_bytes=T * d * esz + T * Fs * esz)
        acc["shared_down"] = dict(flops=2.0 * d * Fs * T, bytes=1.0 * Fs * d * wsz + sc_dn,
                                  impl_bytes=T * Fs * esz + T * d * 4.0)
    layer_flops = 6.0 * d * F * R + 2.0 * wl.T * d * wl.E + (6.0 * d * wl.Fs * wl.T if wl.n_shared else 0.0)
    layer_bytes = (touched * (3.0 * F * d * wsz + sc_up + sc_dn)
                   + ((3.0 * wl.Fs * d * wsz + (2.0 * wl.Fs * 4 + d * 4.0 if fp8 else 0.0)) if wl.n_shared else 0.0)
                   + 2.0 * wl.T * d * esz + wl.E * d * 4.0)
    return acc, layer_flops, layer_bytes


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, h, budget_s: float, policy: str = "first_come", expert_choice: bool = False):
    """The oracle as it stands on a bounded sample: routing of all T tokens
    (capacity needs every token), then tokens in blocks of 64 through the
    experts and combine until the budget is spent; the whole-layer time is
    extrapolated from the per-token rate."""
    import numpy as np
    import oracle

    oracle.build(force=False)
    L = oracle.layer_of(wl)
    t0 = time.perf_counter()
    if expert_choice:
        L.renorm = 0
        rt = oracle.route_expert_choice(L, h["x"], h["Wg"], h["logit_bias"])
        rt["w"] = np.nan_to_num(rt["w"])
        L = oracle.ec_layer(L)
    else:
        rt = oracle.route(L, h["x"], h["Wg"], h["logit_bias"], h["sel_bias"], policy=policy)
    t_route = time.perf_counter() - t0
    scales = {k: h.get(k) for k in ("S1", "S3", "S2", "Ss1", "Ss3", "Ss2")}
    done = 0
    t_rows = 0.0
    while done < wl.T and t_rows < budget_s:
        toks = np.arange(done, min(wl.T, done + 64), dtype=np.int64)
        t1 = time.perf_counter()
        oracle.forward_rows(L, h["x"], rt["idx"], rt["w"], rt["dest"], h["W1"], h["W3"], h["W2"], h["Ws1"],
                            h["Ws3"], h["Ws2"], tokens=toks, **scales)
        t_rows += time.perf_counter() - t1
        done += len(toks)
    t_layer = t_route + t_rows * wl.T / done
    return {"value": wl.T / t_layer, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"routing of all {wl.T} tokens ({t_route:.2f} s) + experts and combine for the first "
                      f"{done} tokens ({t_rows:.2f} s), extrapolated to {wl.T} tokens",
            "seconds_measured": round(t_route + t_rows, 2)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the layer runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "expert parallelism across GPUs is not part of it.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_sparse_route_amd as moe
    from moe_synth import workload

    wl = workload(args.workload, **({"wdtype": "fp8"} if args.fp8 else {}), **({"T": args.tokens} if args.tokens else {}))
    packing = args.packed
    if packing == "auto":
        table = DEFAULT_PACKING_FP8 if wl.wdtype == "fp8" else DEFAULT_PACKING
        packing = table.get(wl.name, "none") if wl.dtype == "bf16" else "none"
    lib = moe.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    t_gen = time.perf_counter()
    h = wl.gen_all()

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    d = {k: dev(v) for k, v in h.items()}
    t_gen = time.perf_counter() - t_gen
    spec = moe.LayerSpec(tokens=wl.T, d_model=wl.d, d_ff=wl.F, n_experts=wl.E, top_k=wl.K, gate=wl.gate,
                         capacity_factor=wl.capacity_factor, n_shared=wl.n_shared,
                         d_ff_shared=wl.Fs, dtype=wl.dtype, stats=args.stats, drop_policy=args.drop_policy,
                         expert_choice=args.expert_choice, renorm=wl.renorm and not args.expert_choice,
                         wdtype=wl.wdtype, packed=packing)
    # the weight layout is chosen once, when the weights are loaded: outside the timed region
    pack_names = {"none": (), "up": ("W1", "W3", "Ws1", "Ws3"), "down": ("W2", "Ws2")}
    pack_names["both"] = pack_names["up"] + pack_names["down"]
    torch.cuda.synchronize()
    t_pack = time.perf_counter()
    for k in pack_names[packing]:
        if d.get(k) is not None:
            packed = torch.empty_like(d[k])
            moe.moe_pack_weights(d[k], packed)
            d[k] = packed
    torch.cuda.synchronize()
    t_pack = time.perf_counter() - t_pack
    scales = None
    if args.fp8:
        scales = dict(w1=d["S1"], w3=d["S3"], w2=d["S2"], ws1=d["Ss1"], ws3=d["Ss3"], ws2=d["Ss2"])
    ws, _ = moe.alloc_workspace(spec)
    r = moe.Routing(spec)
    y = torch.empty((wl.T, wl.d), dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_forward(spec, d["x"], d["Wg"], d["logit_bias"], d["sel_bias"], d["W1"], d["W3"], d["W2"], d["Ws1"],
                        d["Ws3"], d["Ws2"], y, r, ws, stream, scales=scales)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps; in the last of every EVENT_EVERY
    # steps the dominant kernel is bracketed by HIP events on its launch stream
    # (a pair of event records costs a few microseconds of stream time, so
    # sampling keeps the measurement from inflating the step time)
    dominant = "gemm_gate_up"
    moe.profile_enable([])
    moe.profile_reset()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    timed = [i % EVENT_EVERY == EVENT_EVERY - 1 or args.steps < EVENT_EVERY for i in range(args.steps)]
    for i in range(args.steps):
        moe.profile_enable([dominant] if timed[i] else [])
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    moe.profile_enable([])
    prof = moe.profile_read()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    dom_ms, dom_n = prof[dominant]
    dom_avg_ms = dom_ms / max(dom_n, 1)

    breakdown = None
    if args.breakdown:
        moe.profile_reset()
        moe.profile_enable(None)
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        moe.profile_enable([])
        breakdown = {k: round(v[0] / v[1] * 1000.0, 2) for k, v in moe.profile_read().items() if v[1]}

    offsets = r.offsets.cpu().numpy()
    R = int(offsets[-1])
    touched = int(np.count_nonzero(np.diff(offsets)))
    acc, layer_flops, layer_bytes = kernel_accounting(wl, R, touched)
    a = acc[dominant]
    timed_steps = sum(timed)
    assert dom_n == timed_steps, f"{dominant}: {dom_n} launches timed in {timed_steps} steps"
    per_launch_bytes = a["bytes"]
    per_launch_flops = a["flops"]
    intensity = per_launch_flops / per_launch_bytes
    if intensity < RIDGE:
        achieved = per_launch_bytes / (dom_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = per_launch_flops / (dom_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = dominant
    roof["avg_launch_ms"] = round(dom_avg_ms, 4)
    roof["event_timed_launches"] = int(dom_n)  # in the last of every EVENT_EVERY timed steps
    roof["algorithmic_bytes_per_launch"] = per_launch_bytes
    roof["algorithmic_flops_per_launch"] = per_launch_flops
    roof["implementation_bytes_per_launch"] = a["impl_bytes"]
    roof["mfma_frac"] = round(per_launch_flops / (dom_avg_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    roof["hbm_frac"] = round(per_launch_bytes / (dom_avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    # HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    # summary, valid only for the kernel source the counters were taken on
    roof["traffic"] = None
    tpath = os.path.join(ROOT, "profiles", f"traffic__{dominant}__{wl.name}{'__fp8_weights' if args.fp8 else ''}.txt")
    if os.path.exists(tpath):
        kv = {}
        for ln in open(tpath):
            if "=" in ln and not ln.lstrip().startswith("#"):
                k, v = ln.split("=", 1)
                kv[k.strip()] = v.strip()
        if kv.get("source_sha256_16") == gemm_source_hash():
            roof["traffic"] = float(kv["bytes_per_launch"])

    line = {
        "metric": METRIC,
        "value": round(wl.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.T, "d_model": wl.d, "d_ff": wl.F, "n_experts": wl.E,
                   "top_k": wl.K, "gate": "sigmoid" if wl.gate else "softmax", "renorm": wl.renorm,
                   "capacity_factor": wl.capacity_factor, "n_shared": wl.n_shared, "d_ff_shared": wl.Fs,
                   "expert_weights": "fp8_e4m3" if args.fp8 else wl.dtype,
                   "packed_weights": packing, "weight_pack_ms": round(t_pack * 1e3, 2),
                   "router_stats": args.stats, "drop_policy": args.drop_policy,
                   "routing": "expert_choice" if args.expert_choice else "token_choice",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"tflops": round(layer_flops / (ms_per_step * 1e-3) / 1e12, 2),
                  "algorithmic_gbps": round(layer_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                  "mfma_frac": round(layer_flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                  "hbm_frac": round(layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  # max(flops / MFMA peak, bytes / HBM peak) / step time
                  "roofline_frac": round(max(layer_flops / (BF16_PEAK_TFLOPS * 1e12),
                                             layer_bytes / (HBM_PEAK_GBS * 1e9)) / (ms_per_step * 1e-3), 4),
                  "algorithmic_flops": layer_flops, "algorithmic_bytes": layer_bytes,
                  "kept_rows": R, "touched_experts": touched, "host_wall_s": round(wall, 3)},
    }
    if breakdown:
        line["kernels_us"] = breakdown
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, h, args.cpu_seconds, args.drop_policy, args.expert_choice)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    del lib


if __name__ == "__main__":
    main()
