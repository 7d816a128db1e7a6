#!/usr/bin/env python3
"""Benchmark of the W8A8 INT8 linear layer on one MI355X.

Headline workload: the decode-shaped Llama-3-8B-like linears -- M in
{1, 8, 32, 64} tokens x (K, N) in {(4096, 6144) fused QKV, (4096, 4096),
(4096, 28672) gate_up, (14336, 4096) down} -- with dynamic per-token
symmetric activation quantisation, per-channel int8 weights and a bf16 bias.
One step runs the whole hot path on all 16 shapes: w8a8_linear_dyn_sym for
each, which is w8a8_quantize_act then w8a8_scaled_mm_int8 (one fused launch
for the shapes where that is faster: M = 1 with N = 4096). Every call reads its own copy of the weight,
and each shape's copies add up to >= 1 GiB, so no call finds its weight in
the 256 MB Infinity Cache and the figure is HBM bandwidth. Inputs are seeded
synthetic data already resident in HBM when timing starts.

Steps are captured once as HIP graphs (one graph per step of the weight
rotation) and replayed, so the timed region holds GPU work only, not the
host's per-call launch cost.

value = algorithmic bytes of one step / step time (GB/s). The same line
carries the dominant kernel's roofline -- its average launch duration taken
with HIP events on the launch stream around a graph of back-to-back launches
-- and the CPU oracle timed on a bounded sample. The other workloads (prefill
TOPS, the static per-tensor scheme, the MoE grouped GEMM and the FP8 weight
conversion) are reported in their own sections, each kernel against its own
roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-prefill] [--no-extra]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
HBM_STREAM_GBS = 6450.0      # what a plain streaming read of HBM reaches on this GPU (measured)
NODE_US = 1.6                # a kernel node of a HIP graph, empty (measured)
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOPS
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, TFLOP/s
ROTATE_BYTES = 1 << 30       # weight bytes cycled between reuses of one copy, per shape
GRAPH_STEPS = 16             # distinct step graphs (weight-rotation period)
SECTIONS = ("decode", "prefill", "static", "moe", "fp8", "rmsnorm")


def gemm_bytes(M, K, N, bias=False, asym=False):
    """Algorithmic HBM bytes of one scaled GEMM: weight, activation codes,
    scales, output (and bias / zero points / column sums when present)."""
    b = K * N + M * K + 4 * M + 4 * N + 2 * M * N
    if bias:
        b += 2 * N
    if asym:
        b += 4 * M + 4 * N
    return b


def vendor_int32(torch, W, timer, xq, w, s_x, s_w, R):
    """Context for the prefill figure: the plain int8 x int8 -> int32 product
    (no epilogue) by this library and by PyTorch's own int8 matrix product
    (hipBLASLt on ROCm) on the same codes, with whether the two agree."""
    M, N = xq.shape[0], w.shape[0]
    i32 = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    g = capture(torch, lambda: [W.scaled_mm_int8(xq, w, s_x, s_w, out_dtype=W.OUT_I32, out=i32)
                                for _ in range(R)])
    ours = timer.graph_us(g, R)
    del g
    res = {"us": round(ours, 1)}
    try:
        wt = w.t()
        equal = bool(torch.equal(torch._int_mm(xq, wt), i32))
        g = capture(torch, lambda: [torch._int_mm(xq, wt) for _ in range(R)])
        res.update(torch_int_mm_us=round(timer.graph_us(g, R), 1), torch_int_mm_equal=equal)
        del g
    except (RuntimeError, AttributeError) as e:
        res["torch_int_mm"] = f"unavailable: {type(e).__name__}"
    return res


def quant_bytes(M, K, asym=False):
    return 3 * M * K + 4 * M + (4 * M if asym else 0)


def grouped_bytes(E, T, K, N, rows_read):
    return E * N * K + rows_read * K + 4 * T + 4 * E * N + 2 * T * N + 4 * (E + 1)


def launch_floor_us(nbytes):
    """The time no launch of a kernel moving nbytes can beat here: an empty
    graph node plus the bytes at the plain streaming-read rate. floor_frac =
    this / the measured time (1.0 = at the floor), beside hbm_frac against
    the 8 TB/s peak."""
    return NODE_US + nbytes / (HBM_STREAM_GBS * 1e3)


def rmsnorm_quant_bytes(M, K, residual):
    """x in, codes and scales out, gamma once; the residual read and written."""
    return 3 * M * K + 4 * M + 2 * K + (4 * M * K if residual else 0)


def fp8_convert_bytes(E, N, K):
    return 2 * E * N * K + 4 * E * (-(-N // 128)) * (-(-K // 128)) + 4 * E * N


# Sources the decode kernels are compiled from (the kernels whose HBM traffic
# profiles/traffic.json records).
DECODE_SOURCES = ("gemv.hip", "gemm_common.h", "device_common.h", "launch.h", "quant_common.h", "rounding.h")


def kernel_source_hash():
    """sha256 over the decode kernels' sources, to tell whether recorded
    counters were taken on the kernels being run."""
    import hashlib
    csrc = os.path.join(ROOT, "int8_w8a8_quantized_amd", "csrc")
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from profiles/traffic.json (rocprofv3
    FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known size), or None if
    none was recorded for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path, encoding="utf-8") as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else int(k["bytes_per_launch"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill TOPS section")
    p.add_argument("--no-extra", action="store_true", help="skip the static / MoE / FP8 sections")
    p.add_argument("--sections", default=",".join(SECTIONS),
                   help="comma-separated subset of %s (a run without decode reports no value; "
                        "for profiling one part)" % ",".join(SECTIONS))
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time of the oracle sample")
    p.add_argument("--calib-copy", action="store_true",
                   help="first copy 256 MiB device-to-device once (the known-size reference for "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = p.parse_args()
    args.sections = {x.strip() for x in args.sections.split(",") if x.strip()}
    unknown = args.sections - set(SECTIONS)
    if unknown:
        p.error(f"unknown sections {sorted(unknown)}")
    if args.no_prefill:
        args.sections.discard("prefill")
    if args.no_extra:
        args.sections -= {"static", "moe", "fp8"}
    return args


class Timer:
    """HIP events on one stream around a region of already-enqueued work."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def graph_us(self, graph, launches, reps=5, warm_ms=20.0):
        """Microseconds per launch of a graph holding `launches` launches, in
        steady state: the graph is first replayed until at least warm_ms of
        GPU time has passed (the first replays after a capture, or after other
        work, run at a lower clock), then `reps` replays are timed back to
        back, each between its own pair of events, and the median is taken."""
        torch = self.torch
        done = 0.0
        while True:
            w0 = torch.cuda.Event(enable_timing=True)
            w1 = torch.cuda.Event(enable_timing=True)
            w0.record(self.stream)
            graph.replay()
            w1.record(self.stream)
            w1.synchronize()
            done += w0.elapsed_time(w1)
            if done >= warm_ms:
                break
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(self.stream)
        for i in range(reps):
            graph.replay()
            ev[i + 1].record(self.stream)
        ev[-1].synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
        return 1e3 * per[reps // 2] / launches


def progress(msg):
    """One line on stderr per finished section (the JSON line stays alone on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fresh_cache(torch):
    """Each section starts from an empty allocator cache: the decode
    section's 4 GiB of weight copies, once freed, otherwise stay cached, and
    the prefill GEMMs measured 10-20% slower on tensors carved out of them."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def decode_section(args, torch, W, synth, to_dev, timer, dev):
    """The headline decode step (16 linears, each the quantiser and the scaled
    GEMM), timed as whole-step graph replays, then each shape on its own."""
    shapes = [(M, K, N) for M in synth.DECODE_M for (K, N) in synth.DECODE_KN]
    pools = {}
    for (K, N) in synth.DECODE_KN:
        d = synth.decode(64, K, N)
        w0 = to_dev(d["w"])
        n_copies = max(2, -(-ROTATE_BYTES // (K * N)))
        pools[(K, N)] = dict(w=[w0] + [w0.clone() for _ in range(n_copies - 1)],
                             s_w=to_dev(d["s_w"]), bias=to_dev(d["bias"]))
    acts = {}
    for (M, K, N) in shapes:
        d = synth.decode(M, K, N)
        acts[(M, K, N)] = dict(x=to_dev(d["x"]), xq=torch.empty((M, K), dtype=torch.int8, device=dev),
                               s_x=torch.empty(M, dtype=torch.float32, device=dev),
                               out=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
    step_bytes = sum(gemm_bytes(M, K, N, bias=True) + quant_bytes(M, K) for (M, K, N) in shapes)
    ws_bytes = max(W.scaled_mm_workspace_size(M, N, K) for (M, K, N) in shapes)
    workspace = torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def gemm(shape, copy):
        M, K, N = shape
        a, p = acts[shape], pools[(K, N)]
        W.scaled_mm_int8(a["xq"], p["w"][copy % len(p["w"])], a["s_x"], p["s_w"], bias=p["bias"],
                         out=a["out"], workspace=workspace)

    def quant(shape):
        a = acts[shape]
        W.quantize_act(a["x"], W.QUANT_DYN_SYM, xq=a["xq"], s_x=a["s_x"])

    def linear(shape, copy):
        # the quantiser and the scaled GEMM in one call: one fused launch
        # where that is faster (M <= 2, N <= 4096), else the two launches
        M, K, N = shape
        a, p = acts[shape], pools[(K, N)]
        W.linear_dyn_sym(a["x"], p["w"][copy % len(p["w"])], p["s_w"], bias=p["bias"], out=a["out"],
                         xq=a["xq"], s_x=a["s_x"], workspace=workspace)

    def fused(shape):
        M, K, N = shape
        return W.linear_dyn_sym_kernel_name(M, N, K) != W.scaled_mm_kernel_name(M, N, K)

    def step(s):
        # call j of a (K, N) pair in step s reads weight copy 4*s + j of its pool
        j_of = {}
        for shape in shapes:
            kn = shape[1:]
            j = j_of.get(kn, 0)
            j_of[kn] = j + 1
            linear(shape, 4 * s + j)

    for s in range(2):   # eager warm-up (also checks every call returns OK)
        step(s)
    torch.cuda.synchronize()
    graphs = [capture(torch, lambda s=s: step(s)) for s in range(GRAPH_STEPS)]
    torch.cuda.synchronize()

    # ------------------------------------------------------ timed region
    for i in range(args.warmup):
        graphs[i % GRAPH_STEPS].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % GRAPH_STEPS].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = step_bytes / (elapsed / args.steps) / 1e9

    progress(f"decode step: {value:.1f} GB/s")
    # ---------------------------------------- per-kernel launch durations
    # One graph per shape of back-to-back launches over that shape's weight
    # copies; HIP events on the launch stream around its replays.
    per_shape, per_kernel = {}, {}
    for shape in shapes:
        M, K, N = shape
        n = len(pools[(K, N)]["w"])
        R = n * max(1, -(-64 // n))
        if fused(shape):  # one launch does both: its time and bytes include the quantiser's
            g = capture(torch, lambda: [linear(shape, c) for c in range(R)])
            us = timer.graph_us(g, R)
            del g
            kname = W.linear_dyn_sym_kernel_name(M, N, K)
            b = gemm_bytes(M, K, N, bias=True) + quant_bytes(M, K)
            per_shape[f"{M}x{K}x{N}"] = {"kernel": kname, "fused_us": round(us, 3),
                                         "GBs": round(b / (us * 1e-6) / 1e9, 1),
                                         "hbm_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                         "floor_frac": round(launch_floor_us(b) / us, 4)}
        else:
            g = capture(torch, lambda: [gemm(shape, c) for c in range(R)])
            us = timer.graph_us(g, R)
            gq = capture(torch, lambda: [quant(shape) for _ in range(32)])
            qus = timer.graph_us(gq, 32)
            del g, gq
            kname = W.scaled_mm_kernel_name(M, N, K)
            b = gemm_bytes(M, K, N, bias=True)
            per_shape[f"{M}x{K}x{N}"] = {"kernel": kname, "gemm_us": round(us, 3),
                                         "GBs": round(b / (us * 1e-6) / 1e9, 1),
                                         "hbm_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                         "floor_frac": round(launch_floor_us(b) / us, 4),
                                         "quant_us": round(qus, 3)}
            qname = "quant_kernel (dynamic symmetric)"
            agg = per_kernel.setdefault(qname, dict(launches=0, us=0.0, bytes=0))
            agg["launches"] += 1
            agg["us"] += qus
            agg["bytes"] += quant_bytes(M, K)
        agg = per_kernel.setdefault(kname, dict(launches=0, us=0.0, bytes=0))
        agg["launches"] += 1
        agg["us"] += us
        agg["bytes"] += b
    dom_name, dom = max(per_kernel.items(), key=lambda kv: kv[1]["us"])
    avg_us = dom["us"] / dom["launches"]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    # frac is the dominant kernel's (achieved / peak); step_frac is the whole
    # step's (value / peak), the figure to read against the decode target
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(dom_name),
                "kernel": dom_name, "avg_launch_us": round(avg_us, 3),
                "bytes_per_launch": int(dom["bytes"] / dom["launches"]),
                "step_frac": round(value / HBM_PEAK_GBS, 4)}
    kernels = {k: {"launches_per_step": v["launches"], "avg_us": round(v["us"] / v["launches"], 3),
                   "GBs": round(v["bytes"] / (v["us"] * 1e-6) / 1e9, 1)} for k, v in per_kernel.items()}
    del graphs

    progress("decode per-kernel durations done")
    return dict(value=value, ms_per_step=ms_per_step, step_bytes=step_bytes, roofline=roofline,
                kernels=kernels, per_shape=per_shape, shapes=shapes)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(across GPUs the layer would shard by output columns)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from int8_w8a8_quantized_amd import lib as W
    from int8_w8a8_quantized_amd import synth

    W.init(0)
    dev = "cuda:0"

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Graph capture runs on a side stream; all timing happens on this one.
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    timer = Timer(torch, stream)

    # ---------------------------------------------------------------- decode
    shapes = [(M, K, N) for M in synth.DECODE_M for (K, N) in synth.DECODE_KN]
    dec = decode_section(args, torch, W, synth, to_dev, timer, dev) if "decode" in args.sections else None
    fresh_cache(torch)
    # ------------------------------------------------------------ prefill TOPS
    prefill = None
    if "prefill" in args.sections:
        prefill = {}
        for M in synth.PREFILL_M:
            for (K, N) in synth.DECODE_KN:
                d = synth.prefill(M, K, N)
                x, w = to_dev(d["x"]), to_dev(d["w"])
                s_w = to_dev(d["s_w"])
                xq, s_x, zp = W.quantize_act(x, W.QUANT_DYN_ASYM)
                cs = W.prepare_colsum(w)
                out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                R = 5
                g = capture(torch, lambda: [W.scaled_mm_int8(xq, w, s_x, s_w, zp=zp, colsum=cs,
                                                             azp_mode=W.AZP_PER_TOKEN, out=out)
                                            for _ in range(R)])
                us = timer.graph_us(g, R)
                gq = capture(torch, lambda: [W.quantize_act(x, W.QUANT_DYN_ASYM, xq=xq, s_x=s_x, zp=zp)
                                             for _ in range(R)])
                qus = timer.graph_us(gq, R)
                del g, gq
                tops = 2.0 * M * N * K / (us * 1e-6) / 1e12
                prefill[f"{M}x{K}x{N}"] = {"kernel": W.scaled_mm_kernel_name(M, N, K),
                                           "gemm_us": round(us, 1), "TOPS": round(tops, 1),
                                           "frac": round(tops / INT8_PEAK_TOPS, 4),
                                           "quant_us": round(qus, 1),
                                           "quant_GBs": round(quant_bytes(M, K, True) / (qus * 1e-6) / 1e9, 1)}
                prefill[f"{M}x{K}x{N}"]["plain_int32"] = vendor_int32(torch, W, timer, xq, w, s_x, s_w, R)
                del x, w, xq, out
                progress(f"prefill {M}x{K}x{N} done")
        torch.cuda.synchronize()

    extra = None
    if args.sections & {"static", "moe", "fp8", "rmsnorm"}:
        fresh_cache(torch)
        extra = extra_sections(torch, np, W, synth, to_dev, timer, dev, args.sections)
        if "fp8" in args.sections:
            fresh_cache(torch)
            extra["fp8_prefill"] = fp8_section(torch, W, synth, to_dev, timer, dev)
            progress("fp8 section done")
        if "rmsnorm" in args.sections:
            fresh_cache(torch)
            extra["rmsnorm_quant"] = rmsnorm_section(torch, W, synth, to_dev, timer, dev)
            progress("rmsnorm section done")

    progress("prefill and extra sections done")
    # ------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(np, synth, shapes, args.cpu_seconds)

    dec = dec or dict(value=None, ms_per_step=None, step_bytes=None, roofline=None, kernels=None,
                      per_shape=None)
    line = {
        "metric": "INT8 scaled-GEMM TOPS (prefill) and GB/s (decode), % of MI355X roofline",
        "value": None if dec["value"] is None else round(dec["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None if dec["ms_per_step"] is None else round(dec["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded), resident in HBM; each shape's weight rotated over >= 1 GiB of copies",
        "config": {"workload": "decode: M in {1,8,32,64} x (K,N) in {(4096,6144),(4096,4096),"
                               "(4096,28672),(14336,4096)}; dynamic per-token symmetric quant + "
                               "scaled int8 GEMM with bf16 bias",
                   "shapes": len(shapes), "step_bytes": dec["step_bytes"], "timing": "HIP graph replay",
                   "parallelism": "single GPU"},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "kernels": dec["kernels"],
        "decode_shapes": dec["per_shape"],
        "prefill": prefill,
        "extra": extra,
    }
    print(json.dumps(line))
    return 0


def extra_sections(torch, np, W, synth, to_dev, timer, dev, sections):
    """The static per-tensor scheme, the MoE grouped GEMM and the FP8 weight
    conversion, each timed as a graph of back-to-back launches."""
    out = {}
    if "static" in sections:
        out.update(static_section(torch, np, W, synth, to_dev, timer, dev))
    if "moe" in sections:
        fresh_cache(torch)
        out.update(moe_section(torch, np, W, synth, to_dev, timer, dev))
    return out


def static_section(torch, np, W, synth, to_dev, timer, dev):
    out = {}

    # Static per-tensor scheme: fused QKV, M=512, K=4096, N=6144.
    d = synth.static_qkv()
    M, K = d["x"].shape
    N = d["w"].shape[0]
    x, w = to_dev(d["x"]), to_dev(d["w"])
    ps = to_dev(d["part_scales"])
    s_in = to_dev(np.array([d["s_in"]], np.float32))
    zp_in = to_dev(np.array([d["zp_in"]], np.int32))
    s_max = W.prepare_requant_max(w, ps, d["widths"])
    adj = W.prepare_colsum(w, zp_in=zp_in)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    o = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    R = 20
    g = capture(torch, lambda: [W.quantize_act(x, W.QUANT_STATIC_ASYM, s_in=s_in, zp_in=zp_in, xq=xq)
                                for _ in range(R)])
    qus = timer.graph_us(g, R)
    g = capture(torch, lambda: [W.scaled_mm_int8(xq, w, s_in, s_max, colsum=adj, azp_mode=W.AZP_STATIC,
                                                 out=o) for _ in range(R)])
    us = timer.graph_us(g, R)
    # the lossless alternative to requantising: the partitions' own scales per
    # channel on the original weight
    w0 = to_dev(d["w"])
    s_ch = W.prepare_expand_scales(ps, d["widths"])
    adj0 = W.prepare_colsum(w0, zp_in=zp_in)
    g = capture(torch, lambda: [W.prepare_expand_scales(ps, d["widths"], s_w=s_ch) for _ in range(R)])
    eus = timer.graph_us(g, R)
    g = capture(torch, lambda: [W.scaled_mm_int8(xq, w0, s_in, s_ch, colsum=adj0, azp_mode=W.AZP_STATIC,
                                                 out=o) for _ in range(R)])
    us_ch = timer.graph_us(g, R)
    del g
    tops = 2.0 * M * N * K / (us * 1e-6) / 1e12
    gb = gemm_bytes(M, K, N, asym=True)
    out["static_qkv_512x4096x6144"] = {
        "kernel": W.scaled_mm_kernel_name(M, N, K), "gemm_us": round(us, 2), "TOPS": round(tops, 1),
        "mfma_frac": round(tops / INT8_PEAK_TOPS, 4), "GBs": round(gb / (us * 1e-6) / 1e9, 1),
        "hbm_frac": round(gb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "quant_us": round(qus, 2),
        "per_channel_scales": {"expand_us": round(eus, 2), "gemm_us": round(us_ch, 2)}}
    del x, w, w0, xq, o, one
    progress("static fused QKV done")
    return out


def moe_section(torch, np, W, synth, to_dev, timer, dev):
    """MoE: FP8 -> int8 conversion of the expert weights, the two grouped
    GEMMs, then the whole expert block."""
    out = {}
    m = synth.moe()
    E, topk = synth.MOE_E, m["topk"]
    tokens = m["x13"].shape[0]
    T = tokens * topk
    logits = to_dev(m["logits"])
    # the routing and expert sort on the device (the block's own first step)
    _, _, rows, offs, _ = W.moe_route(logits, topk)
    conv = {}
    qw = {}
    for name in ("w13", "w2"):
        codes, S = to_dev(m[name + "_fp8"]), to_dev(m[name + "_scales"])
        _, Nn, Kk = codes.shape
        Wq, s, flag = W.prepare_fp8_block_to_int8(codes, S)
        g = capture(torch, lambda: [W.prepare_fp8_block_to_int8(codes, S, Wq=Wq, s=s, err_flag=flag)
                                    for _ in range(3)])
        us = timer.graph_us(g, 3)
        del g
        b = fp8_convert_bytes(E, Nn, Kk)
        conv[f"{name}_{E}x{Nn}x{Kk}"] = {"us": round(us, 1), "GBs": round(b / (us * 1e-6) / 1e9, 1),
                                         "hbm_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        qw[name] = (Wq, s)
        del codes, S
    out["fp8_block_to_int8"] = conv
    progress("fp8 conversion done")

    x13 = to_dev(m["x13"])
    x2 = to_dev(m["x2"])
    xq13, sx13, _ = W.quantize_act(x13, W.QUANT_DYN_SYM)
    xq2, sx2, _ = W.quantize_act(x2, W.QUANT_DYN_SYM)
    moe = {}
    for name, xq_, sx_, rid, Kk in (("w13", xq13, sx13, rows, synth.MOE_HIDDEN),
                                     ("w2", xq2, sx2, None, synth.MOE_INTER)):
        Wq, s = qw[name]
        Nn = Wq.shape[1]
        o = torch.empty((T, Nn), dtype=torch.bfloat16, device=dev)
        R = 5
        g = capture(torch, lambda: [W.grouped_scaled_mm_int8(xq_, offs, Wq, sx_, s, row_ids=rid, T=T, out=o)
                                    for _ in range(R)])
        us = timer.graph_us(g, R)
        del g
        tops = 2.0 * T * Nn * Kk / (us * 1e-6) / 1e12
        b = grouped_bytes(E, T, Kk, Nn, T)
        moe[f"{name}_T{T}_K{Kk}_N{Nn}"] = {
            "gemm_us": round(us, 1), "TOPS": round(tops, 1), "mfma_frac": round(tops / INT8_PEAK_TOPS, 4),
            "GBs": round(b / (us * 1e-6) / 1e9, 1), "hbm_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del o
    R = 5
    g = capture(torch, lambda: [W.quantize_act(x2, W.QUANT_DYN_SYM, xq=xq2, s_x=sx2) for _ in range(R)])
    qus = timer.graph_us(g, R)
    del g
    moe["quant_w2_input_32768x1536"] = {"us": round(qus, 1),
                                         "GBs": round(quant_bytes(T, 1536) / (qus * 1e-6) / 1e9, 1)}
    out["moe_grouped"] = moe
    progress("grouped GEMMs done")
    del xq2, sx2, x2
    out["moe_block"] = moe_block_section(torch, W, timer, dev, x13, logits, topk, qw)
    torch.cuda.synchronize()
    return out


def fp8_section(torch, W, synth, to_dev, timer, dev):
    """The W8A8 FP8 GEMM on the prefill shapes: E4M3 activations quantised on
    the device (per token, or per token in groups of 128), E4M3 weights of
    N(0, 1) values scaled to the format's range, per-channel or 128 x 128
    block scales; TFLOP/s against the fp8 peak, plus the quantiser's time."""
    res = {}
    for M in synth.PREFILL_M:
        for (K, N) in synth.DECODE_KN:
            d = synth.prefill(M, K, N)
            x = to_dev(d["x"])
            g = torch.Generator(device=dev)
            g.manual_seed(M * 7 + K * 3 + N)
            w8 = (torch.randn((N, K), device=dev, generator=g) * 100).clamp(-448, 448).to(
                torch.float8_e4m3fn).view(torch.uint8)
            sw_ch = torch.rand(N, device=dev, generator=g) * 1e-4 + 1e-5
            G, NB = -(-K // 128), -(-N // 128)
            sw_blk = torch.rand((NB, G), device=dev, generator=g) * 1e-4 + 1e-5
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            row = {}
            for name, act, wm, sw in (("channel", W.FP8_ACT_TOKEN, W.FP8_W_CHANNEL, sw_ch),
                                      ("block128", W.FP8_ACT_GROUP128, W.FP8_W_BLOCK128, sw_blk)):
                xq, sx = W.quantize_act_fp8(x, act)
                R = 5
                gq = capture(torch, lambda: [W.quantize_act_fp8(x, act, xq=xq, s_x=sx) for _ in range(R)])
                qus = timer.graph_us(gq, R)
                gg = capture(torch, lambda: [W.scaled_mm_fp8(xq, w8, sx, sw, act, wm, out=out) for _ in range(R)])
                us = timer.graph_us(gg, R)
                del gq, gg
                tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
                row[name] = {"kernel": W.scaled_mm_fp8_kernel_name(M, N, K, wm), "gemm_us": round(us, 1),
                             "TFLOPS": round(tf, 1), "frac": round(tf / FP8_PEAK_TFLOPS, 4),
                             "quant_us": round(qus, 1)}
            res[f"{M}x{K}x{N}"] = row
            progress(f"fp8 {M}x{K}x{N} done")
            del x, w8, out
    torch.cuda.synchronize()
    return res


def rmsnorm_section(torch, W, synth, to_dev, timer, dev):
    """The quantiser fused into the RMS normalisation before it (with the
    residual add) on the hidden rows (K = 4096) of the decode and prefill
    batches; against the plain quantiser on the same rows (the launch the
    fusion removes from a layer that normalises anyway) and the read + write
    HBM roof."""
    res = {}
    R = 16
    for M in synth.DECODE_M + synth.PREFILL_M:
        for K in (4096,):
            d = synth.decode(M, K, 16)
            x = to_dev(d["x"])
            g = torch.ones(K, dtype=torch.bfloat16, device=dev)
            r = x.clone()
            xq = torch.empty((M, K), dtype=torch.int8, device=dev)
            sx = torch.empty(M, dtype=torch.float32, device=dev)
            gf = capture(torch, lambda: [W.rmsnorm_quant(x, g, 1e-6, residual=r, xq=xq, s_x=sx) for _ in range(R)])
            us = timer.graph_us(gf, R)
            gq = capture(torch, lambda: [W.quantize_act(x, W.QUANT_DYN_SYM, xq=xq, s_x=sx) for _ in range(R)])
            qus = timer.graph_us(gq, R)
            del gf, gq
            b = rmsnorm_quant_bytes(M, K, True)
            res[f"{M}x{K}"] = {"us": round(us, 2), "GBs": round(b / (us * 1e-6) / 1e9, 1),
                               "hbm_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                               "quant_only_us": round(qus, 2)}
            del x, r, xq
    torch.cuda.synchronize()
    return res


def moe_block_section(torch, W, timer, dev, x, logits, topk, qw):
    """The whole int8 MoE expert block on the MoE workload (4096 tokens, top-8
    of 64 experts, hidden 3072, intermediate 1536, the converted expert
    weights): one w8a8_moe_block_int8 call, and each of its steps alone."""
    (w13, s13), (w2, s2) = qw["w13"], qw["w2"]
    tokens, H = x.shape
    E = logits.shape[1]
    I = w2.shape[2]
    T = tokens * topk
    ws = torch.empty(W.moe_block_workspace_size(tokens, E, topk, H, I), dtype=torch.uint8, device=dev)
    o = torch.empty((tokens, H), dtype=torch.bfloat16, device=dev)
    R = 5
    g = capture(torch, lambda: [W.moe_block_int8(x, logits, topk, w13, s13, w2, s2, out=o, workspace=ws)
                                for _ in range(R)])
    us = timer.graph_us(g, R)
    del g
    ops = 2.0 * T * (2 * I) * H + 2.0 * T * H * I
    res = {"block_us": round(us, 1), "TOPS": round(ops / (us * 1e-6) / 1e12, 1),
           "mfma_frac": round(ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)}
    # the steps around the grouped GEMMs, each as a graph of back-to-back launches
    rws = torch.empty(max(16, int(W.load().w8a8_moe_route_workspace_size(tokens, E))), dtype=torch.uint8,
                      device=dev)
    routed = W.moe_route(logits, topk, workspace=rws)
    g = capture(torch, lambda: [W.moe_route(logits, topk, workspace=rws, out=routed) for _ in range(R)])
    res["route_us"] = round(timer.graph_us(g, R), 2)
    h = torch.randn((T, 2 * I), device=dev).to(torch.bfloat16)
    aq = torch.empty((T, I), dtype=torch.int8, device=dev)
    sa = torch.empty(T, dtype=torch.float32, device=dev)
    g = capture(torch, lambda: [W.silu_mul_quant(h, I, aq=aq, s_a=sa) for _ in range(R)])
    sus = timer.graph_us(g, R)
    sb = T * 2 * I * 2 + T * I + 4 * T
    res["silu_mul_quant_us"] = round(sus, 1)
    res["silu_mul_quant_GBs"] = round(sb / (sus * 1e-6) / 1e9, 1)
    del h, aq
    y = torch.randn((T, H), device=dev).to(torch.bfloat16)
    _, wts, _, _, pos = routed
    g = capture(torch, lambda: [W.moe_combine(y, pos, wts, out=o) for _ in range(R)])
    cus = timer.graph_us(g, R)
    cb = T * H * 2 + tokens * H * 2 + T * 8
    res["combine_us"] = round(cus, 1)
    res["combine_GBs"] = round(cb / (cus * 1e-6) / 1e9, 1)
    del g, y, ws
    return res


def cpu_baseline(np, synth, shapes, min_seconds):
    """The oracle, as written, on the decode workload: whole steps (all 16
    shapes, quantise + GEMM + epilogue) until at least min_seconds of CPU
    time have passed. Input generation is outside the timing."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    data = {s: synth.decode(*s) for s in shapes}
    nbytes = 0
    steps = 0
    t0 = time.perf_counter()
    while True:
        for (M, K, N) in shapes:
            d = data[(M, K, N)]
            O.linear_forward(d["x"], d["w"], d["s_w"], O.MODE_DYN_SYM, bias_bits=d["bias"])
            nbytes += gemm_bytes(M, K, N, bias=True) + quant_bytes(M, K)
        steps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    cpu_s = time.perf_counter() - t0
    return {"value": round(nbytes / cpu_s / 1e9, 3), "unit": "GB/s",
            "cores": blas_threads or len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{steps} whole decode step(s) of the oracle (all 16 shapes: quantise + GEMM + "
                      f"epilogue); input generation excluded",
            "seconds": round(cpu_s, 2), "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    sys.exit(main())
