"""Throughput of the routed MoE expert-FFN hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
    python bench.py --profile      # workload + copy calibration, for rocprofv3

Workload: the FP8 blockwise layer with clamped SwiGLU (H = 6144, I = 2048,
288 routed experts top-8 plus one shared expert, L = 10), at T = 4096 tokens
per step; T = 1 and T = 64 are reported in "sweep", and the router GEMM
fused with the gate epilogue (moe_gate_route, the 258-column gate of the
ep_lora_258 layer) at T = 1 .. 8192 in "gate_route". Inputs are seeded,
synthetic and resident in HBM before timing. A step is one moe_forward: route
-> permute -> activation quant -> grouped GEMM1 + SwiGLU -> grouped GEMM2 +
combine. Prints one JSON line. "value" is the back-to-back time of K steps
at T = 4096 (10.9 GB of touched weights per step, far beyond the 256 MB
MALL); the sweep and "configs" also time every step alone after a 512 MB
copy that evicts the MALL, and their rates use that median, so repeated
small-T weights count as HBM traffic only when they come from HBM.
"decode_graph" compares host-issued T = 1 steps with replays of the same
step captured in a HIP graph.

roofline: the dominant kernel is the FP8 GEMM1 (moe_gemm_fp8_kernel<128,
true>). "achieved" is its algorithmic bytes (touched W13 codes + scales, the
x codes + scales once, the h codes + scales written) over its average launch
time measured here with HIP events on the launching stream. "traffic" is the
HBM bytes per launch measured by rocprofv3 FETCH_SIZE + WRITE_SIZE (scaled by
the same counters on a plain copy of known size), read from the committed
summary profiles/gemm1_fp8_T4096_traffic.md -- and null when the kernel
sources no longer hash to the ones the counters were taken on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "fp8_clamp_288"
T_MAIN = 4096
T_SWEEP = (1, 64, 4096)
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5033.0
BF16_PEAK_TFLOPS = 2517.0
METRIC = ("MoE layer tokens/s + TFLOP/s (% MFMA peak) and weight GB/s (% HBM) "
          "at T=1..4096")
GEMM1_KERNEL = "moe_gemm_fp8_kernel<128, true> (moe_grouped_gemm1_act)"
CSRC = os.path.join(ROOT, "mixture_experts_expert_sigmoid_amd", "csrc")
KERNEL_SOURCES = ("gemm_fp8.hip", "gemm_common.h", "common.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm1_fp8_T4096_traffic.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="run only the forward at --profile-tokens (warmup + steps) and "
                         "a copy of known size, for rocprofv3 counter passes")
    ap.add_argument("--profile-tokens", type=int, default=T_MAIN)
    ap.add_argument("--profile-config", default=WORKLOAD,
                    help="seeded configuration the --profile run uses")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration array (every seeded layer at each "
                         "of its token counts)")
    return ap.parse_args()


def kernel_sources_sha256():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per GEMM1 launch from the committed counter summary, or
    None when it is missing or was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    sha = re.search(r"sources_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != kernel_sources_sha256():
        return None
    return float(val.group(1))


def algorithmic(spec, ids_np, T):
    """Pairs, touched experts, GEMM flops and bytes from the run's routing."""
    k, H, I = spec.top_k, spec.H, spec.I
    e_loc = ids_np.reshape(-1) - spec.offset
    local = (e_loc >= 0) & (e_loc < spec.n_local)
    touched = len(set(e_loc[local].tolist())) + (spec.shared if T > 0 else 0)
    P = int(local.sum()) + (T if spec.shared else 0)
    w13_b = 2 * I * H + 4 * (2 * I // 128) * (H // 128)
    w2_b = H * I + 4 * (H // 128) * (I // 128)
    return dict(
        P=P, touched=touched,
        flops=6.0 * P * H * I,
        gemm1_flops=4.0 * P * H * I,
        weight_bytes=touched * (w13_b + w2_b),
        # GEMM1 algorithmic bytes: touched W13 + scales, x codes + scales read
        # once, h codes + scales written
        gemm1_bytes=touched * w13_b + T * (H + 4 * H // 128) + P * (I + 4 * I // 128),
    )


class MallFlush:
    """Evicts the 256 MB Infinity Cache (MALL) between timed iterations: a
    copy of 512 MB (1 GB of traffic), itself not timed. Without it the
    weight bytes of small-T steps, which repeat every iteration, could be
    served from the MALL instead of HBM."""

    def __init__(self):
        import torch
        self.src = torch.ones(1 << 27, device="cuda")          # 512 MB
        self.dst = torch.empty_like(self.src)

    def __call__(self):
        self.dst.copy_(self.src)


def time_flushed(fn, steps, stream, flush):
    """Per-iteration times (HIP events on `stream`) with a MALL flush before
    every iteration; returns (median, min) in ms."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2], t[0]


def time_calls(fn, steps, stream):
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU's share of the layer; "
                                   "--gpus must be 1 (no multi-GPU runs)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_expert_sigmoid_amd as M
    from synth import CONFIGS, FP4_CONFIGS, make_batch, make_layer
    from tests.gpu_helpers import module_for

    assert torch.cuda.is_available(), "bench needs a GPU"
    spec = {**CONFIGS, **FP4_CONFIGS}[args.profile_config if args.profile else WORKLOAD]
    t0 = time.time()
    layer = make_layer(spec, device="cuda")
    torch.cuda.synchronize()
    print(f"# layer generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    mod = module_for(spec, layer)
    stream = torch.cuda.current_stream()

    if args.profile:
        # copy calibration: 1 GiB read + 1 GiB written by a plain copy kernel
        src = torch.ones(1 << 28, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        Tp = args.profile_tokens
        batch = make_batch(spec, None, Tp, device="cuda")
        outs = mod.alloc_outputs(Tp)
        for _ in range(args.warmup + args.steps):
            mod.forward(batch.x, batch.logits, outs)
        torch.cuda.synchronize()
        alg = algorithmic(spec, outs["topk_ids"].cpu().numpy(), Tp)
        print(f"# profile run done: copy 3 x 1 GiB, {spec.name} forward T={Tp} x "
              f"{args.warmup + args.steps}; pairs {alg['P']}, experts touched "
              f"{alg['touched']}", flush=True)
        return

    flush = MallFlush()
    results = {}
    for T in (T_SWEEP if not args.no_sweep else (T_MAIN,)):
        batch = make_batch(spec, None, T, device="cuda")
        x, lg = batch.x, batch.logits
        outs = mod.alloc_outputs(T)
        mod.workspace(T)
        for _ in range(args.warmup):
            mod.forward(x, lg, outs)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            mod.forward(x, lg, outs)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        ids = outs["topk_ids"].cpu().numpy()
        alg = algorithmic(spec, ids, T)
        fmed, fmin = time_flushed(lambda: mod.forward(x, lg, outs), args.steps, stream, flush)
        results[T] = dict(ms=ms, alg=alg, batch=batch, outs=outs, fmed=fmed, fmin=fmin)
        print(f"# T={T}: {ms:.3f} ms/step back to back; MALL flushed before each step: "
              f"median {fmed:.3f} min {fmin:.3f}", file=sys.stderr, flush=True)

    # ---- per-call timing of the path's steps at the main size ---------------
    T = T_MAIN
    r = results[T]
    x, lg = r["batch"].x, r["batch"].logits
    k, N, H, I, G = spec.top_k, spec.n_routed, spec.H, spec.I, spec.n_groups
    pc = T * k + T
    d32 = dict(device="cuda", dtype=torch.int32)
    ids = torch.empty(T, k, **d32)
    w = torch.empty(T, k, device="cuda")
    offsets = torch.empty(G + 1, **d32)
    sp = torch.empty(pc, **d32)
    pr = torch.empty(pc, **d32)
    err = torch.zeros(1, **d32)
    wsp = torch.empty(M.moe_permute_workspace_size(T, k, G), dtype=torch.uint8, device="cuda")
    xq = torch.empty(T, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(T, H // 128, device="cuda")
    h = torch.empty(pc, I, dtype=torch.uint8, device="cuda")
    hs = torch.empty(pc, I // 128, device="cuda")
    out = torch.empty(T, H, device="cuda")
    ws2 = torch.empty(M.moe_gemm2_workspace_size(mod.w2, pc), dtype=torch.uint8, device="cuda")
    calls = {
        "route": lambda: M.moe_route(lg, N, 0, k, 1.0, 1.0, ids, w, None),
        "permute": lambda: M.moe_permute(ids, k, N, 0, N, 1, offsets, sp, pr, err, wsp),
        "quant": lambda: M.moe_quantize_act_fp8(x, xq, xs),
        "gemm1": lambda: M.moe_grouped_gemm1_act(mod.w13, xq, xs, None, T, H, I, k, pc,
                                                  offsets, sp, mod.act, None, h, hs, None),
        "gemm2_combine": lambda: M.moe_grouped_gemm2_combine(
            mod.w2, h, hs, T, H, I, k, 1, pc, offsets, pr, w, 1.0, out, ws2),
    }
    for f in calls.values():      # warm and fill the intermediates in order
        f()
    torch.cuda.synchronize()
    per_call = {}
    for name, f in calls.items():
        for _ in range(2):
            f()
        per_call[name] = time_calls(f, args.steps, stream)
    assert torch.equal(out, r["outs"]["out"]), "step-wise path differs from moe_forward"

    alg = r["alg"]
    g1_ms = per_call["gemm1"]
    g1_gbs = alg["gemm1_bytes"] / (g1_ms * 1e-3) / 1e9
    roofline = {"kernel": GEMM1_KERNEL,
                "bound": "hbm", "achieved": round(g1_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(g1_gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(),
                "algorithmic_bytes": alg["gemm1_bytes"],
                "gemm1_ms": round(g1_ms, 4),
                "gemm1_tflops": round(alg["gemm1_flops"] / (g1_ms * 1e-3) / 1e12, 1)}

    # rates from the MALL-flushed median (weights really come from HBM)
    sweep = []
    for T_, rr in results.items():
        a = rr["alg"]
        s = rr["fmed"] * 1e-3
        sweep.append({"T": T_, "ms_per_step": round(rr["ms"], 4),
                      "ms_per_step_flushed_median": round(rr["fmed"], 4),
                      "ms_per_step_flushed_min": round(rr["fmin"], 4),
                      "tokens_per_s": round(T_ / s, 1),
                      "tflops": round(a["flops"] / s / 1e12, 2),
                      "pct_fp8_mfma_peak": round(100 * a["flops"] / s / 1e12 / FP8_PEAK_TFLOPS, 2),
                      "weight_gbs": round(a["weight_bytes"] / s / 1e9, 1),
                      "pct_hbm_peak": round(100 * a["weight_bytes"] / s / 1e9 / HBM_PEAK_GBS, 2),
                      # the attainable roofline min(peak, AI * BW) as a time:
                      # max(flops / FP8 peak, touched weight bytes / 8 TB/s)
                      "roofline_bound": ("hbm" if a["weight_bytes"] / (HBM_PEAK_GBS * 1e9) >=
                                         a["flops"] / (FP8_PEAK_TFLOPS * 1e12) else "mfma"),
                      "pct_attainable": round(100 * max(a["weight_bytes"] / (HBM_PEAK_GBS * 1e9),
                                                        a["flops"] / (FP8_PEAK_TFLOPS * 1e12)) / s, 2),
                      "pairs": a["P"], "experts_touched": a["touched"]})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, layer, r["batch"], T_MAIN)

    configs = None if args.no_configs else config_table(args, stream, flush)

    main_ms = results[T_MAIN]["ms"]
    line = {
        "metric": METRIC, "value": round(T_MAIN / (main_ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(main_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: FP8 blockwise 128x128, H=6144, I=2048, "
                               "288 routed top-8 + 1 shared, clamped SwiGLU L=10",
                   "T": T_MAIN, "H": spec.H, "I": spec.I, "experts": spec.n_routed,
                   "shared_experts": spec.shared, "top_k": spec.top_k},
        "roofline": roofline, "cpu_baseline": cpu,
        "per_call_ms": {k_: round(v, 4) for k_, v in per_call.items()},
        "sweep": sweep,
        "gate_route": gate_route_table(args.steps, stream) if not args.no_sweep else None,
        "decode_graph": (decode_graph(mod, results[1]["batch"], results[1]["outs"])
                         if 1 in results else None),
        "configs": configs,
    }
    print(json.dumps(line))


def decode_graph(mod, batch, outs, n=50):
    """A decode step (T = 1) issued by the host: wall time per step of n
    moe_forward calls from Python (each ~10 kernel launches through the C
    ABI) against n replays of the same forward captured once in a HIP graph
    (torch.cuda.graph), both ending in one synchronisation. The MALL is not
    flushed (the 340 MB of this step's weights partly stay in it), so the
    replay time is the launch-bound floor of a serving loop, not an HBM
    figure."""
    import torch
    x, lg = batch.x, batch.logits
    for _ in range(5):
        mod.forward(x, lg, outs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        mod.forward(x, lg, outs)
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / n
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mod.forward(x, lg, outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mod.forward(x, lg, outs)
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        g.replay()
    torch.cuda.synchronize()
    replay = (time.perf_counter() - t0) / n
    return {"T": 1, "eager_ms_per_step": round(eager * 1e3, 4),
            "graph_replay_ms_per_step": round(replay * 1e3, 4), "steps": n}


GATE_CFG = "ep_lora_258"
GATE_T = (1, 37, 512, 8192)


def gate_route_table(steps, stream):
    """moe_gate_route (router GEMM fused with the gate epilogue: selection
    bias, raw-logit carry, two sinks, packed output) on the 258-column gate
    of the ep_lora_258 layer (H = 2048). Per-call time (HIP events on the
    launching stream around each call, so host submission counts when the
    GPU outruns it), the GPU time per call from replays of a captured HIP
    graph of 20 calls (us_per_call_graph), algorithmic bytes (x once, the
    router weight once, ids / weights / packed / sink weights written) as
    GB/s and % of 8 TB/s, and 2 T C H flop as % of the bf16 MFMA peak; the
    rates use the per-call time."""
    import torch
    import mixture_experts_expert_sigmoid_amd as M
    from synth import CONFIGS, make_gate, make_tokens
    spec = CONFIGS[GATE_CFG]
    N, S, k, H = spec.n_routed, spec.n_sink, spec.top_k, spec.H
    gate = make_gate(spec)
    wg, bias = gate.wg.cuda(), gate.bias.cuda()
    out = []
    for T in GATE_T:
        x = make_tokens(spec, T, device="cuda")
        ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, k, device="cuda")
        sw = torch.empty(T, S, device="cuda")
        packed = torch.empty(T, k, dtype=torch.int32, device="cuda")
        nb = M.moe_gate_route_workspace_size(T, H, N, S)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        f = lambda: M.moe_gate_route(x, wg, N, S, k, 1.0, 1.0, ids, w, sw,
                                     sel_bias=bias, packed=packed, ws=ws)
        for _ in range(5):
            f()
        ms = time_calls(f, steps, stream)
        reps = 20
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                f()
        g.replay()
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(5):
            g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        us_graph = e0.elapsed_time(e1) / (5 * reps) * 1e3
        del g
        byts = T * H * 2 + (N + S) * H * 2 + T * (k * 12 + S * 4)
        flops = 2.0 * T * (N + S) * H
        gbs = byts / (ms * 1e-3) / 1e9
        tfl = flops / (ms * 1e-3) / 1e12
        out.append({"T": T, "us_per_call": round(ms * 1e3, 2),
                    "us_per_call_graph": round(us_graph, 2),
                    "tokens_per_s": round(T / (ms * 1e-3), 1),
                    "path": "fused" if nb == 0 else "split-K + epilogue kernel",
                    "algorithmic_bytes": byts, "gbs": round(gbs, 1),
                    "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                    "tflops": round(tfl, 2),
                    "pct_bf16_mfma_peak": round(100 * tfl / BF16_PEAK_TFLOPS, 2)})
        print(f"# gate_route T={T}: {ms * 1e3:.2f} us/call, {us_graph:.2f} us/call "
              f"from graph replays", file=sys.stderr, flush=True)
    return out


def _weight_bytes(layer):
    """Bytes of one group's W13 and W2 (codes + scales)."""
    b13 = layer.w13_q[0].numel() * layer.w13_q.element_size()
    b2 = layer.w2_q[0].numel() * layer.w2_q.element_size()
    if layer.w13_s is not None:
        b13 += layer.w13_s[0].numel() * layer.w13_s.element_size()
        b2 += layer.w2_s[0].numel() * layer.w2_s.element_size()
    return b13, b2


def _peak_tflops(fmt, gemm=0):
    """The dense MFMA peak a GEMM of the format runs against: FP8 layers and
    the W4A8 GEMM1 (fp4 x fp8 on the block-scaled instructions) the FP8
    rate, the others bf16 / f16; gemm 0 = the whole layer, where the W4A8
    layer takes the rate of its GEMMs' flop mix (2/3 at FP8, 1/3 at f16)."""
    if fmt == "fp8":
        return FP8_PEAK_TFLOPS
    if fmt == "mxfp4_a8":
        if gemm == 1:
            return FP8_PEAK_TFLOPS
        if gemm == 0:
            return 1.0 / (2.0 / 3.0 / FP8_PEAK_TFLOPS + 1.0 / 3.0 / BF16_PEAK_TFLOPS)
    return BF16_PEAK_TFLOPS


def config_table(args, stream, flush):
    """moe_forward on every seeded configuration at each of its token
    counts: back to back and MALL-flushed (median), tokens/s, useful TFLOP/s
    (6 P H I) against the format's MFMA peak (FP8 layers the FP8 peak, the
    others bf16), touched-weight GB/s against 8 TB/s, the attainable-roofline
    percentage, and the two GEMM entry points timed alone (MALL flushed)
    with their algorithmic bytes: GEMM1 = touched W13 + x + h written,
    GEMM2 + combine = touched W2 + h read + out written. Also printed as a
    table on stderr."""
    import torch
    from synth import CONFIGS, EXT_CONFIGS, FP4_CONFIGS, make_batch, make_layer
    from tests.gpu_helpers import StepCalls, module_for
    print("# config              T    ms/step  flushed-med  flushed-min    tokens/s"
          "    TFLOP/s  weight GB/s  gemm1 ms  gemm2+comb ms", file=sys.stderr)
    # C5 with the down LoRA too, and with a batch of eight rank-16 adapters
    # (tokens pick one or none), the page's multi-adapter serving case; the
    # C5 layer in NVFP4 (the page's own weight format) and the INT4 layer's
    # shape in MXFP4
    table = dict(CONFIGS)
    table.update(EXT_CONFIGS)
    table["ep_lora_258_x8"] = EXT_CONFIGS["ep_lora_258_down"].scaled(
        name="ep_lora_258_x8", cfg_id=15, n_adapters=8)
    table.update(FP4_CONFIGS)
    entries = []
    for name, spec in table.items():
        layer = make_layer(spec, device="cuda")
        mod = module_for(spec, layer)
        b13, b2 = _weight_bytes(layer)
        for T in spec.Ts:
            batch = make_batch(spec, layer, T, device="cuda")
            mod.set_adapters(batch.adapter_ids)
            outs = mod.alloc_outputs(T)
            mod.workspace(T)
            # warm up for >= 50 ms of wall time: a GPU left idle while the
            # host builds a layer needs that long to return to full clocks
            t_end = time.perf_counter() + 0.05
            n = 0
            while n < args.warmup or time.perf_counter() < t_end:
                mod.forward(batch.x, batch.logits, outs)
                n += 1
                if n % 16 == 0:
                    torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(args.steps):
                mod.forward(batch.x, batch.logits, outs)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / args.steps
            fmed, fmin = time_flushed(lambda: mod.forward(batch.x, batch.logits, outs),
                                      args.steps, stream, flush)
            ids = outs["topk_ids"].cpu().numpy()
            e_loc = ids.reshape(-1) - spec.offset
            local = (e_loc >= 0) & (e_loc < spec.n_local)
            touched = len(set(e_loc[local].tolist())) + (spec.shared if T > 0 else 0)
            P = int(local.sum()) + (T if spec.shared else 0)
            fl = 6.0 * P * spec.H * spec.I
            wbytes = touched * (b13 + b2)
            peak = _peak_tflops(spec.fmt)
            s_ = fmed * 1e-3
            # the two GEMM entry points alone, MALL flushed before each call
            st = StepCalls(spec, mod, batch.x, batch.logits, batch.adapter_ids)
            st.run()
            g1_med, _ = time_flushed(st.gemm1, args.steps, stream, flush)
            g2_med, _ = time_flushed(st.gemm2, args.steps, stream, flush)
            fp8 = spec.fmt == "fp8"
            xb = T * spec.H * ((1 + 4 / 128) if fp8 else (1 + 1 / 32)
                               if spec.fmt == "mxfp4_a8" else 2)
            hb = P * spec.I * ((1 + 4 / 128) if fp8 else 2)
            g1_bytes = touched * b13 + xb + hb
            g2_bytes = touched * b2 + hb + T * spec.H * 4

            def rate(ms_, byts, flops, pk):
                gbs = byts / (ms_ * 1e-3) / 1e9
                tfl = flops / (ms_ * 1e-3) / 1e12
                return {"ms": round(ms_, 4), "gbs": round(gbs, 1),
                        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                        "tflops": round(tfl, 2), "frac_mfma": round(tfl / pk, 4)}
            ent = {"config": name, "T": T, "fmt": spec.fmt,
                   "ms_per_step": round(ms, 4), "ms_flushed_median": round(fmed, 4),
                   "ms_flushed_min": round(fmin, 4), "tokens_per_s": round(T / s_, 1),
                   "tflops": round(fl / s_ / 1e12, 2),
                   "pct_mfma_peak": round(100 * fl / s_ / 1e12 / peak, 2),
                   "weight_gbs": round(wbytes / s_ / 1e9, 1),
                   "pct_hbm_peak": round(100 * wbytes / s_ / 1e9 / HBM_PEAK_GBS, 2),
                   "roofline_bound": ("hbm" if wbytes / (HBM_PEAK_GBS * 1e9) >=
                                      fl / (peak * 1e12) else "mfma"),
                   "pct_attainable": round(100 * max(wbytes / (HBM_PEAK_GBS * 1e9),
                                                     fl / (peak * 1e12)) / s_, 2),
                   "pairs": P, "experts_touched": touched,
                   "gemm1": rate(g1_med, g1_bytes, 4.0 * P * spec.H * spec.I,
                                 _peak_tflops(spec.fmt, 1)),
                   "gemm2_combine": rate(g2_med, g2_bytes, 2.0 * P * spec.H * spec.I,
                                         _peak_tflops(spec.fmt, 2))}
            entries.append(ent)
            print(f"# {name:18s} {T:5d} {ms:10.4f} {fmed:12.4f} {fmin:12.4f} "
                  f"{T / fmed * 1e3:11.1f} {fl / fmed / 1e9:10.2f} "
                  f"{wbytes / fmed / 1e6:12.1f} {g1_med:9.4f} {g2_med:14.4f}",
                  file=sys.stderr, flush=True)
            del st
        del layer, mod
        torch.cuda.empty_cache()
    return entries


def cpu_baseline(spec, layer, batch, T, n_experts=80):
    """The fp64 oracle as it stands on the host cores, on a bounded sample:
    routing, permutation and activation quantisation of all T tokens plus
    the expert FFNs of the first `n_experts` routed experts (all their
    pairs); the layer time is extrapolated by pair count."""
    import numpy as np
    from oracle import moe_oracle as O
    from synth import to_numpy_batch
    from tests.gpu_helpers import LazyExperts
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    nb = to_numpy_batch(batch)
    arr = LazyExperts(layer)
    t0 = time.time()
    ids, w, _ = O.route(nb["logits"], spec.n_routed, spec.n_sink, spec.top_k)
    offsets, sp, _, _ = O.permute(ids, spec.n_routed, spec.offset, spec.n_local, spec.shared)
    xhat, xb = O.gemm1_input(spec, nb["x_bits"])
    t_fixed = time.time() - t0
    k = spec.top_k
    done = 0
    t1 = time.time()
    for e in range(n_experts):
        rows = np.arange(offsets[e], offsets[e + 1])
        toks = sp[rows] // k
        O.expert_ffn(spec, arr, e, xhat[toks], xb[toks])
        done += len(rows)
    t_ffn = time.time() - t1
    P = int(offsets[-1])
    t_layer = t_fixed + t_ffn * P / max(done, 1)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(T / t_layer, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model,
            "gflops": round(6.0 * P * spec.H * spec.I / t_layer / 1e9, 2),
            "sample": f"fp64 oracle: route+permute+quant of all {T} tokens "
                      f"({t_fixed:.1f}s) + expert FFN of {n_experts} of {spec.n_groups} "
                      f"groups ({done} of {P} pairs, {t_ffn:.1f}s), layer time "
                      f"extrapolated by pair count to {t_layer:.0f}s"}


if __name__ == "__main__":
    main()
