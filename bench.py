#!/usr/bin/env python3
"""Benchmark of the W8A8 INT8 linear layer on one MI355X.

Headline workload: the decode-shaped Llama-3-8B-like linears -- M in
{1, 8, 32, 64} tokens x (K, N) in {(4096, 6144) fused QKV, (4096, 4096),
(4096, 28672) gate_up, (14336, 4096) down} -- with dynamic per-token
symmetric activation quantisation, per-channel int8 weights and a bf16 bias.
One step runs the whole hot path on all 16 shapes: w8a8_quantize_act then
w8a8_scaled_mm_int8 for each. The weights rotate through enough copies
(>= 1 GiB) that no call finds its weight in the 256 MB Infinity Cache, so the
figure is HBM bandwidth. Inputs are seeded synthetic data already resident
in HBM when timing starts.

value = algorithmic bytes of one step / step time (GB/s); the same line
carries the dominant kernel's roofline (HIP events around each of its
launches on the launch stream) and the CPU oracle timed on a bounded sample.
Prefill-shaped GEMMs (M in {2048, 8192}) are reported in "prefill" as TOPS.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-prefill]
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
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOPS
ROTATE_BYTES = 1 << 30       # weight bytes cycled between reuses of one copy


def gemm_bytes(M, K, N, bias=False, asym=False):
    """Algorithmic HBM bytes of one scaled GEMM: weight, activation codes,
    scales, output (and bias / zero points / column sums when present)."""
    b = K * N + M * K + 4 * M + 4 * N + 2 * M * N
    if bias:
        b += 2 * N
    if asym:
        b += 4 * M + 4 * N
    return b


def quant_bytes(M, K, asym=False):
    return 3 * M * K + 4 * M + (4 * M if asym else 0)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill TOPS section")
    p.add_argument("--prefill-steps", type=int, default=5)
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the layer would shard by output columns across GPUs; see DESIGN.md)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from int8_w8a8_quantized_amd import lib as W
    from int8_w8a8_quantized_amd import synth

    W.init(0)
    dev = "cuda:0"
    stream = torch.cuda.current_stream()

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # ---------------------------------------------------------------- inputs
    shapes = [(M, K, N) for M in synth.DECODE_M for (K, N) in synth.DECODE_KN]
    weights = {}
    for (K, N) in synth.DECODE_KN:
        d = synth.decode(64, K, N)
        weights[(K, N)] = dict(w=to_dev(d["w"]), s_w=to_dev(d["s_w"]), bias=to_dev(d["bias"]))
    set_bytes = sum(K * N for (K, N) in synth.DECODE_KN)
    copies = max(2, -(-ROTATE_BYTES // set_bytes))
    rot = {kn: [v["w"]] + [v["w"].clone() for _ in range(copies - 1)] for kn, v in weights.items()}
    acts = {}
    for (M, K, N) in shapes:
        d = synth.decode(M, K, N)
        x = to_dev(d["x"])
        acts[(M, K, N)] = dict(x=x, xq=torch.empty((M, K), dtype=torch.int8, device=dev),
                               s_x=torch.empty(M, dtype=torch.float32, device=dev),
                               out=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
    step_bytes = sum(gemm_bytes(M, K, N, bias=True) + quant_bytes(M, K) for (M, K, N) in shapes)
    ws_bytes = max(W.scaled_mm_workspace_size(M, N, K) for (M, K, N) in shapes)
    workspace = torch.zeros(max(1, ws_bytes // 4), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    call = [0]
    ev_log = []

    def step(events=False):
        for (M, K, N) in shapes:
            a = acts[(M, K, N)]
            wv = weights[(K, N)]
            w = rot[(K, N)][call[0] % copies]
            W.quantize_act(a["x"], W.QUANT_DYN_SYM, xq=a["xq"], s_x=a["s_x"])
            if events:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            W.scaled_mm_int8(a["xq"], w, a["s_x"], wv["s_w"], bias=wv["bias"], out=a["out"],
                             workspace=workspace)
            if events:
                e1.record(stream)
                ev_log.append(((M, K, N), e0, e1))
        call[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = step_bytes / (elapsed / args.steps) / 1e9

    # Per-launch GEMM durations with HIP events on the launch stream, over a
    # second pass of the same steps (the events sit between launches, so this
    # pass is kept out of the headline timing).
    ev_log.clear()
    for _ in range(args.steps):
        step(events=True)
    torch.cuda.synchronize()
    per_kernel = {}
    for (M, K, N), e0, e1 in ev_log:
        kname = "gemv_i8_kernel<MF=%d>" % (1 if M <= 16 else 2 if M <= 32 else 3 if M <= 48 else 4)
        ms = e0.elapsed_time(e1)
        agg = per_kernel.setdefault(kname, dict(launches=0, ms=0.0, bytes=0))
        agg["launches"] += 1
        agg["ms"] += ms
        agg["bytes"] += gemm_bytes(M, K, N, bias=True)
    dom_name, dom = max(per_kernel.items(), key=lambda kv: kv[1]["ms"])
    avg_us = 1e3 * dom["ms"] / dom["launches"]
    achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": dom_name, "avg_launch_us": round(avg_us, 3),
                "bytes_per_launch": int(dom["bytes"] / dom["launches"])}
    kernels = {k: {"launches_per_step": v["launches"] // args.steps,
                   "avg_us": round(1e3 * v["ms"] / v["launches"], 3),
                   "GBs": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1)} for k, v in per_kernel.items()}
    per_shape = {}
    for (M, K, N), e0, e1 in ev_log:
        per_shape.setdefault(f"{M}x{K}x{N}", []).append(e0.elapsed_time(e1))
    shapes_out = {k: {"us": round(1e3 * float(np.median(v)), 2),
                      "GBs": round(gemm_bytes(*map(int, k.split("x")), bias=True) / (np.median(v) * 1e-3) / 1e9, 1)}
                  for k, v in per_shape.items()}

    # ------------------------------------------------------------ prefill TOPS
    prefill = None
    if not args.no_prefill:
        prefill = {}
        for M in synth.PREFILL_M:
            for (K, N) in synth.DECODE_KN:
                d = synth.prefill(M, K, N)
                x, w = to_dev(d["x"]), to_dev(d["w"])
                s_w = to_dev(d["s_w"])
                xq, s_x, zp = W.quantize_act(x, W.QUANT_DYN_ASYM)
                cs = W.prepare_colsum(w)
                out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                for _ in range(2):
                    W.scaled_mm_int8(xq, w, s_x, s_w, zp=zp, colsum=cs, azp_mode=W.AZP_PER_TOKEN, out=out)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(args.prefill_steps):
                    W.scaled_mm_int8(xq, w, s_x, s_w, zp=zp, colsum=cs, azp_mode=W.AZP_PER_TOKEN, out=out)
                e1.record(stream)
                q0 = torch.cuda.Event(enable_timing=True)
                q1 = torch.cuda.Event(enable_timing=True)
                q0.record(stream)
                for _ in range(args.prefill_steps):
                    W.quantize_act(x, W.QUANT_DYN_ASYM, xq=xq, s_x=s_x, zp=zp)
                q1.record(stream)
                torch.cuda.synchronize()
                us = 1e3 * e0.elapsed_time(e1) / args.prefill_steps
                qus = 1e3 * q0.elapsed_time(q1) / args.prefill_steps
                tops = 2.0 * M * N * K / (us * 1e-6) / 1e12
                prefill[f"{M}x{K}x{N}"] = {"gemm_us": round(us, 1), "TOPS": round(tops, 1),
                                           "frac": round(tops / INT8_PEAK_TOPS, 4),
                                           "quant_us": round(qus, 1),
                                           "quant_GBs": round(quant_bytes(M, K, True) / (qus * 1e-6) / 1e9, 1)}
                del x, w, xq, out
        torch.cuda.synchronize()

    # ------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu:
        import oracle as O
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            blas_threads = None
        sample = [(M, K, N) for (M, K, N) in shapes if M in (1, 64)]
        t0 = time.perf_counter()
        nbytes = 0
        for (M, K, N) in sample:
            d = synth.decode(M, K, N)
            O.linear_forward(d["x"], d["w"], d["s_w"], O.MODE_DYN_SYM, bias_bits=d["bias"])
            nbytes += gemm_bytes(M, K, N, bias=True) + quant_bytes(M, K)
        cpu_s = time.perf_counter() - t0
        cpu = {"value": round(nbytes / cpu_s / 1e9, 3), "unit": "GB/s",
               "cores": blas_threads or len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": "oracle linear_forward (quantize + GEMM + epilogue) on the 8 decode shapes "
                         "with M in {1, 64}, once each; input generation excluded",
               "seconds": round(cpu_s, 2), "host_cpus": len(os.sched_getaffinity(0))}

    line = {
        "metric": "INT8 scaled-GEMM TOPS (prefill) and GB/s (decode), % of MI355X roofline",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded), resident in HBM; weights rotated over >=1 GiB",
        "config": {"workload": "decode: M in {1,8,32,64} x (K,N) in {(4096,6144),(4096,4096),"
                               "(4096,28672),(14336,4096)}; dynamic per-token symmetric quant + "
                               "scaled int8 GEMM with bf16 bias",
                   "shapes": len(shapes), "weight_copies": copies, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "decode_shapes": shapes_out,
        "prefill": prefill,
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
