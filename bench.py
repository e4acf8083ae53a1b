"""Benchmark of one GPU's share of the expert-parallel MoE layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode128_fp8]

A step is one whole layer (dispatch -> grouped GEMM with SwiGLU + requant -> combine)
over one batch of synthetic input already resident in HBM.  The default workload is
the 128-token decode layer: 8 simulated source ranks x 16 tokens, hidden 7168, 32
local experts, top-8, intermediate 2048, FP8 e4m3 weights (128x128 scales) and
activations (1x128 scales), bf16 output.

Prints ONE JSON line: value = layer latency in microseconds (lower is better), with
per-stage timings from HIP events recorded by the library on the launch stream,
dispatch/combine GB/s (inside the layer, and alone both warm and cold, cold meaning after
a 1 GiB fill that evicts the caches), the layer time's p10/p50/p90, grouped-GEMM TFLOP/s,
the roofline of the dominant kernel (GEMM1) and the CPU oracle timed on a bounded sample
of the same workload.  Weights smaller than 4x the 256 MB MALL are kept in two copies,
alternated from call to call, so that no call finds its weights in that cache.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer µs at 1–256 tok/GPU; dispatch/combine GB/s; grouped-GEMM TFLOP/s"
HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
# the GEMM1 kernel's source and the headers compiled into it
GEMM1_SRC = [os.path.join(ROOT, "combine_top_gate_amd", "csrc", f)
             for f in ("gemm_lowp.hip", "dispatch_chunk.h", "kernels.h", "common.h", "pack_layout.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm1_decode128_fp8_traffic.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode128_fp8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row-major", action="store_true",
                    help="stream the weights in their row-major layout instead of the packed one")
    ap.add_argument("--cpu-experts", type=int, default=32,
                    help="experts the CPU oracle evaluates in each timed sample")
    ap.add_argument("--cpu-repeats", type=int, default=3,
                    help="timed CPU oracle samples (the median is reported)")
    ap.add_argument("--sched", choices=["fence", "sentinel"], default="fence",
                    help="synchronisation between dispatch and GEMM1")
    ap.add_argument("--dispatch-cus", type=int, default=0,
                    help="SENTINEL: CUs of the dispatch stream (multiple of 8; 0 = library default)")
    ap.add_argument("--no-gate", action="store_true",
                    help="skip the separate timing of the gate (router + top-k) ahead of dispatch")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def algorithmic_bytes(inp, cnt):
    """HBM bytes each stage must move at least once (the per-unit figures are in the design notes)."""
    S, T_s, H, I, E, k = inp.S, inp.T_s, inp.H, inp.I, inp.E, inp.k
    T, R = S * T_s, int(cnt.sum())
    active = int((cnt.sum(axis=0) > 0).sum())
    Ish = inp.shared_I
    if inp.weight == "fp8":
        w13 = 2 * I * H + (2 * I // 128) * (H // 128) * 4
        w2 = H * I + (H // 128) * (I // 128) * 4
        w13_sh = w2_sh = 0
    else:  # MXFP4: packed nibbles + one e8m0 byte per 32
        w13 = 2 * I * H // 2 + 2 * I * H // 32
        w2 = H * I // 2 + H * I // 32
        w13_sh = 2 * Ish * H // 2 + 2 * Ish * H // 32
        w2_sh = H * Ish // 2 + H * Ish // 32
    if inp.act == "bf16":  # W4A16: x and h rows are bf16, no scales
        xrow, hrow, hrow_sh = 2 * H, 2 * I, 2 * Ish
    else:
        xrow = H + (H // 128) * 4
        hrow = I + (I // 128) * 4
        hrow_sh = Ish + (Ish // 128) * 4 if Ish else 0
    d = {}
    # dispatch: ids read, each source row read once, R window rows (+scales) written, control state
    d["dispatch"] = T * k * 4 + T * xrow + R * xrow + T * k * 4 + S * T_s * k * 4 + 2 * S * E * 4
    # GEMM1: weights of active experts once, window rows read, h rows written
    d["gemm1"] = active * w13 + R * xrow + R * hrow + (w13_sh + T * xrow + T * hrow_sh if Ish else 0)
    # GEMM2: weights once, h rows read, y rows (bf16) written
    d["gemm2"] = active * w2 + R * hrow + R * H * 2 + (w2_sh + T * hrow_sh + T * H * 2 if Ish else 0)
    # combine: y rows read, weights and rows read, token rows written
    d["combine"] = R * H * 2 + T * k * 8 + T * H * 2 + (T * H * 2 if Ish else 0)
    d["layer"] = sum(d.values())
    flops = 2 * R * (2 * I) * H + 2 * R * I * H + (6 * T * Ish * H if Ish else 0)
    return d, flops


def code_sha256(paths):
    """sha256 of source files' code (one path or a list, hashed in order): // comments,
    trailing blanks and blank lines removed, so that an edit of the comments alone keeps
    counters taken on the same code."""
    text = "".join(open(p).read() + "\n" for p in ([paths] if isinstance(paths, str) else paths))
    lines = (re.sub(r"//.*$", "", line).rstrip() for line in text.split("\n"))
    return hashlib.sha256("\n".join(line for line in lines if line.strip()).encode()).hexdigest()


def read_traffic():
    """GEMM1 HBM bytes per launch from the committed counter summary, if it is for this code."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_sha = re.search(r"kernel code sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic bytes per launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b:
        return None
    return float(m_b.group(1)) if code_sha256(GEMM1_SRC) == m_sha.group(1) else None


GATE_EXPERTS = 256  # the router scores every global expert (DeepSeek-V3 shape)
MALL_BYTES = 256 << 20  # MI355X last-level (Infinity) cache


def time_warm_cold(torch, fn, reps=50):
    """Microseconds per call of one stage: warm = back-to-back calls (mean, queued behind a
    GPU spin); cold = the median of calls each preceded by a 1 GiB fill, which evicts the
    L2s and the MALL (events around the call only)."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    e0, e1 = ev(), ev()
    torch.cuda._sleep(20_000_000)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    warm = e0.elapsed_time(e1) * 1e3 / reps
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    pairs = []
    for i in range(reps):
        scrub.fill_(i & 0xFF)
        a, b = ev(), ev()
        a.record()
        fn()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    cold = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)[reps // 2]
    del scrub
    return warm, cold


def layer_distribution(torch, run, steps=200, warm=20):
    """p10 / p50 / p90 of single layer calls (200 after 20 warm-up calls), HIP events
    between consecutive calls."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(warm):
        run(i)
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        run(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    t = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps))
    q = lambda f: round(t[min(steps - 1, int(f * steps))], 2)
    return {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9),
            "method": f"{steps} calls after {warm} warm-up calls, HIP events between consecutive calls "
                      "(each a queue barrier)"}


def time_graph(torch, moe, ds, steps):
    """Microseconds per layer call replayed from a captured HIP graph: one graph holds one
    call per weight copy (alternating as in the timed loop), replayed back to back behind
    a GPU spin, HIP events around all the replays."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for dd in ds:
            moe.run(dd)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // len(ds))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(ds))
    del g
    return {"us_per_call": round(us, 2), "calls": reps * len(ds),
            "method": "HIP graph of one layer call per weight copy, replayed back to back behind a GPU spin"}


def time_fused_combine(torch, binding, moe, run, steps):
    """The layer with the combine formed in GEMM2's epilogue (MOE_OPT_FUSED_COMBINE), over
    the same steps as the default loop (us per step)."""
    moe.set_option(binding.MOE_OPT_FUSED_COMBINE, 1)
    try:
        for i in range(5):
            run(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run(i)
        torch.cuda.synchronize()
        return round((time.perf_counter() - t0) * 1e6 / steps, 2)
    finally:
        moe.set_option(binding.MOE_OPT_FUSED_COMBINE, 0)


def time_combine_fp8(torch, moe, d, inp, nbytes_combine, calls=200):
    """Microseconds per FP8-output combine (the layer's output requantised 1x128 for the
    next layer) on the last layer's expert outputs, timed like the gate; its bytes are the
    plain combine's with the token rows written as e4m3 codes + scales instead of bf16."""
    T, H = inp.S * inp.T_s, inp.H
    q = torch.empty((inp.S, inp.T_s, H), dtype=torch.uint8, device="cuda")
    sc = torch.empty((inp.S, inp.T_s, H // 128), dtype=torch.float32, device="cuda")
    for _ in range(3):
        moe.combine_fp8(d.topk_w, q, sc)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(50_000_000)
    e0.record()
    for _ in range(calls):
        moe.combine_fp8(d.topk_w, q, sc)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    nbytes = nbytes_combine - T * H * 2 + T * H + T * (H // 128) * 4
    return {"us_per_call": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes": nbytes,
            "method": f"{calls} back-to-back calls queued behind a GPU spin, HIP events"}


def time_gate(torch, binding, synth, T, H, k, calls=200):
    """Microseconds per fused gate call (router + top-k softmax) for T tokens.

    The calls are plain stream launches, as the layer's are.  A GPU-side spin is queued
    first so that all the calls are enqueued before the first one starts: the events then
    time the GPU's back-to-back work, not the host's call overhead."""
    ri = synth.make_router_inputs(T, H, GATE_EXPERTS, seed=11)
    x = torch.from_numpy(ri.x_bits.view("int16")).cuda()
    wr = torch.from_numpy(ri.wr_bits.view("int16")).cuda()
    ws = torch.empty(binding.gate_workspace_bytes(T, H, GATE_EXPERTS) // 4, dtype=torch.float32, device="cuda")
    for _ in range(3):
        binding.gate(x, wr, k, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(50_000_000)
    e0.record()
    h0 = time.perf_counter()
    for _ in range(calls):
        binding.gate(x, wr, k, workspace=ws)
    h1 = time.perf_counter()
    e1.record()
    torch.cuda.synchronize()
    gpu_us = e0.elapsed_time(e1) * 1e3 / calls
    return {"tokens": T, "hidden": H, "experts": GATE_EXPERTS, "topk": k, "us_per_call": round(gpu_us, 2),
            "host_us_per_call": round((h1 - h0) * 1e6 / calls, 2),
            "method": f"{calls} back-to-back calls queued behind a GPU spin, HIP events"}


def measure_fp8_mfma(torch, binding, blocks=2048, iters=2000, reps=3):
    """Sustained FP8 MFMA rate (TFLOP/s) of the library's register-only MFMA probe, best
    of `reps` launches timed with HIP events on the launch stream."""
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    binding.mfma_fp8_probe(sink, blocks, 10)
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = binding.mfma_fp8_probe(sink, blocks, iters)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return round(best, 1)


def cpu_baseline(inp, n_experts, repeats):
    """The oracle as it stands, timed on a bounded sample of the same workload.

    Sample: the full dispatch and combine, and the expert FFN (dequantise, GEMM1,
    SwiGLU, requant, GEMM2) of n_experts of the E experts, the expert part scaled
    by E / n_experts to the whole layer; median of `repeats` samples."""
    runs = [_cpu_once(inp, n_experts) for _ in range(max(1, repeats))]
    runs.sort(key=lambda r: r[0])
    total, wall, n, cores = runs[len(runs) // 2]
    what = "the whole layer" if n == inp.E else f"dispatch + combine + the FFNs of {n} of {inp.E} experts (scaled by {inp.E}/{n})"
    return {"value": round(total * 1e6, 1), "unit": "us", "cores": int(cores), "kind": "oracle",
            "sample": f"{what}, one batch of the same workload; median of {len(runs)} runs of "
                      f"{wall:.1f} s wall each"}


def _cpu_once(inp, n_experts):
    from oracle import layer
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    route = layer.dispatch(inp.ids, inp.E)
    rows = layer.expert_rows(route["cnt"], route["off"], inp.T_s, inp.k)
    t1 = time.perf_counter()
    x = np.asarray(inp.x).reshape(inp.S * inp.T_s, inp.H)
    if inp.act == "bf16":
        from oracle import codecs
        xt = codecs.bf16_decode(x)
    else:
        xs = np.asarray(inp.x_scale).reshape(inp.S * inp.T_s, inp.H // 128)
        xt = layer.dequant_act_fp8(x, xs)
    R = inp.S * inp.T_s * inp.k
    y = np.zeros((R, inp.H))
    src = np.where(route["row_src"] >= 0, route["row_src"] // inp.k, -1)
    n = min(n_experts, inp.E)
    for e in range(n):
        r = rows[e]
        w13 = layer.dequant_weight(inp.weight, inp.w13[e], inp.s13[e])
        w2 = layer.dequant_weight(inp.weight, inp.w2[e], inp.s2[e])
        ye, _, _ = layer.expert_ffn(xt[src[r]], w13, w2, inp.I, layer.h_format(inp.act))
        y[r] = layer.round_out(ye, inp.out)
    t2 = time.perf_counter()
    layer.combine(y, route["dst_row"], inp.topk_w)
    t3 = time.perf_counter()
    total = (t1 - t0) + (t2 - t1) * inp.E / n + (t3 - t2)
    return total, t3 - t0, n, cores


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer on one GPU; it has no multi-GPU "
              "mode (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    from combine_top_gate_amd import binding, synth

    torch.cuda.set_device(0)
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(args.workload)
    d = binding.DeviceInputs(inp)
    sched = binding.MOE_SCHED_SENTINEL if args.sched == "sentinel" else binding.MOE_SCHED_FENCE
    moe = binding.Moe.for_inputs(inp, sched=sched, dispatch_cus=args.dispatch_cus)
    # fp32 weights have no packed form: the fp32 layer always reads them row-major
    row_major = args.row_major or inp.weight == "f32"
    if not row_major:
        # one-time weight preparation (as at model load), outside the timed region
        moe.pack(d)
        torch.cuda.synchronize()
    # weights under 4x the MALL could be partly served from it across calls: alternate two
    # copies of them (same inputs, same outputs) so that every call streams its weights
    wbytes = sum(t.numel() * t.element_size() for t in (d.w13, d.s13, d.w2, d.s2, *d.sh) if t is not None)
    ds = [d]
    if wbytes < 4 * MALL_BYTES:
        d2 = binding.DeviceInputs(inp)
        if not row_major:
            moe.pack(d2)
        ds.append(d2)
        torch.cuda.synchronize()
    run = lambda i: moe.run(ds[i % len(ds)])
    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    cnt = moe.routing(inp.S, inp.T_s, inp.k, inp.E)[0].cpu().numpy()
    # timed region 1: the layer alone (no timing events: each is a barrier packet
    # in the queue and would add its own gap to the step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # timed region 2: the same steps with HIP events at every stage boundary, on the
    # stream each kernel is launched on (stage times and the GEMM1 launch duration)
    print("[bench] stage timing", file=sys.stderr, flush=True)
    moe.set_timing(args.steps)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    stage_ms, ncalls = moe.read_timing()
    assert ncalls == args.steps
    moe.set_timing(0)
    if moe.device_error():
        raise RuntimeError("device error during the timed region")
    print("[bench] layer distribution, warm and cold dispatch / combine", file=sys.stderr, flush=True)
    dist = layer_distribution(torch, run)
    # the SENTINEL handshake's per-call epoch cannot be replayed from a graph
    graph = time_graph(torch, moe, ds, args.steps) if sched == binding.MOE_SCHED_FENCE else None
    # the decode GEMM2 can also form the combine (an option; the tiled prefill path cannot)
    fused_combine = (time_fused_combine(torch, binding, moe, run, args.steps)
                     if args.workload.startswith("decode") else None)
    disp_warm, disp_cold = time_warm_cold(torch, lambda: moe.dispatch(inp.T_s, d.x, d.x_scale, d.ids))
    comb_warm, comb_cold = time_warm_cold(torch, lambda: moe.combine(d.topk_w, d.out))
    if args.calib_copy_mib:
        a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    ms_step = (t1 - t0) * 1e3 / args.steps
    avg = [m / ncalls for m in stage_ms]  # dispatch, gemm1, gemm2, combine, layer (ms)
    nbytes, flops = algorithmic_bytes(inp, cnt)
    gbps = lambda b, ms: b / (ms * 1e-3) / 1e9
    g1_gbps = gbps(nbytes["gemm1"], avg[1])
    traffic = read_traffic()
    rec = {
        "metric": METRIC,
        "value": round(ms_step * 1e3, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8", "bf16": "bf16"}.get(inp.act, "f32"),
        "data": "synthetic",
        "config": {"workload": args.workload, "sources": inp.S, "tokens_per_source": inp.T_s,
                   "tokens": inp.S * inp.T_s, "hidden": inp.H, "inter": inp.I, "experts": inp.E,
                   "topk": inp.k, "weights": inp.weight, "shared_inter": inp.shared_I,
                   "routing": inp.extra.get("routing"), "schedule": args.sched,
                   "weight_layout": "row-major" if row_major else "packed"},
        "stages_us": {"dispatch": round(avg[0] * 1e3, 2), "gemm1": round(avg[1] * 1e3, 2),
                      "gemm2": round(avg[2] * 1e3, 2), "combine": round(avg[3] * 1e3, 2),
                      "layer_events": round(avg[4] * 1e3, 2)},
        "dispatch_GBps": round(gbps(nbytes["dispatch"], avg[0]), 1),
        "combine_GBps": round(gbps(nbytes["combine"], avg[3]), 1),
        "gemm_TFLOPs": round(flops / ((avg[1] + avg[2]) * 1e-3) / 1e12, 2),
        "layer_hbm_frac": round(gbps(nbytes["layer"], ms_step) / HBM_PEAK_GBPS, 4),
        "fractions": {"dispatch_of_hbm": round(gbps(nbytes["dispatch"], avg[0]) / HBM_PEAK_GBPS, 4),
                      "combine_of_hbm": round(gbps(nbytes["combine"], avg[3]) / HBM_PEAK_GBPS, 4),
                      "gemm_of_fp8_peak": round(flops / ((avg[1] + avg[2]) * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)},
        "us_per_step_with_stage_events": round((t3 - t2) * 1e6 / args.steps, 2),
        "layer_us_dist": dist,
        "layer_us_graph": graph,
        "layer_us_fused_combine": fused_combine,
        "weight_copies": len(ds),
        "dispatch_alone": {"warm_us": round(disp_warm, 2), "cold_us": round(disp_cold, 2),
                           "warm_GBps": round(gbps(nbytes["dispatch"], disp_warm * 1e-3), 1),
                           "cold_GBps": round(gbps(nbytes["dispatch"], disp_cold * 1e-3), 1)},
        "combine_alone": {"warm_us": round(comb_warm, 2), "cold_us": round(comb_cold, 2),
                          "warm_GBps": round(gbps(nbytes["combine"], comb_warm * 1e-3), 1),
                          "cold_GBps": round(gbps(nbytes["combine"], comb_cold * 1e-3), 1),
                          "method": "moe_dispatch / moe_combine alone: warm = back-to-back calls, "
                                    "cold = median of calls each after a 1 GiB fill"},
        "algorithmic_bytes": nbytes,
        "roofline": {"kernel": "gemm1 (FP8 grouped GEMM + SwiGLU + requant)", "bound": "hbm",
                     "achieved": round(g1_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(g1_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": nbytes["gemm1"]},
    }
    mfma = measure_fp8_mfma(torch, binding)
    rec["fp8_mfma_measured_TFLOPs"] = mfma
    rec["fractions"]["gemm_of_measured_fp8_mfma"] = round(rec["gemm_TFLOPs"] / mfma, 4)
    if inp.out == "bf16":
        print("[bench] FP8-output combine timing", file=sys.stderr, flush=True)
        rec["combine_fp8_out"] = time_combine_fp8(torch, moe, d, inp, nbytes["combine"])
    if not args.no_gate:
        print("[bench] gate timing", file=sys.stderr, flush=True)
        rec["gate_us"] = time_gate(torch, binding, synth, inp.S * inp.T_s, inp.H, inp.k)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_experts, args.cpu_repeats)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
