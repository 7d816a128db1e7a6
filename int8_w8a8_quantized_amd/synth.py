"""Seeded synthetic inputs for the W8A8 INT8 linear layer.

This module only *draws* inputs: activations, int8 weights, scales, FP8 block
weights and MoE router logits. It holds none of the layer's arithmetic
(quantisation, GEMM, epilogue, weight preparation), so the tests, the benchmark
and the CPU checker can all feed the same bytes to both sides.

Every generator seeds ``numpy.random.default_rng`` with a list that starts
with the workload id and its sizes, so one (workload, shape) always yields the
same data. Workloads (shapes from the Llama-3-8B linears that the
"vLLM INT8 W8A8 量化实战" page quantises, and the MiniMax-M2 expert shapes of
"MiniMax-M2.7 FP8 转昆仑芯 INT8"):

1. tiny       M=16, K=256, N=512; x ~ N(0,1) with 2 outlier channels x50.
2. decode     M in {1,8,32,64}, (K,N) in DECODE_KN; x ~ N(0,1) with
              round(0.005 K) outlier channels x30; bias ~ N(0, 0.02).
3. prefill    M in {2048, 8192}, same (K,N); x ~ N(0.3, 1).
4. static     M=512, K=4096, N=4096+1024+1024 with three per-tensor scales.
5. moe        64 experts, router logits N(0,1) for 4096 tokens (top-8),
              hidden 3072, w13 (K=3072,N=3072) and w2 (K=1536,N=3072) as
              OCP FP8 E4M3FN N(0, 0.02) with 128x128 block scales.

Int8 weights are uniform integers in [-127, 127]; per-channel weight scales
are U(1e-3, 1e-2) float32.
"""

from __future__ import annotations

import numpy as np

DECODE_M = (1, 8, 32, 64)
PREFILL_M = (2048, 8192)
DECODE_KN = ((4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096))
STATIC_WIDTHS = (4096, 1024, 1024)

MOE_E, MOE_TOPK, MOE_TOKENS, MOE_HIDDEN, MOE_INTER = 64, 8, 4096, 3072, 1536


def rng_for(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bits with round-to-nearest-even (finite inputs only).

    Used only to encode drawn samples as bf16 inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def activations(rng, M, K, mean=0.0, n_outliers=0, outlier_scale=1.0):
    """bf16 bits [M,K]: N(mean, 1) with n_outliers channels multiplied."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    if mean:
        x += np.float32(mean)
    if n_outliers:
        ch = rng.choice(K, size=n_outliers, replace=False)
        x[:, ch] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


def int8_weight(rng, N, K):
    return rng.integers(-127, 128, size=(N, K), dtype=np.int8)


def channel_scales(rng, N):
    return rng.uniform(1e-3, 1e-2, size=N).astype(np.float32)


def bias_bits(rng, N, std=0.02):
    return f32_to_bf16_bits(rng.normal(0.0, std, size=N).astype(np.float32))


def tiny(M=16, K=256, N=512):
    """Workload 1 (any sizes accepted for ragged-shape tests)."""
    rng = rng_for(1, M, K, N)
    return dict(x=activations(rng, M, K, 0.0, min(2, K), 50.0),
                w=int8_weight(rng, N, K), s_w=channel_scales(rng, N))


def decode(M, K, N):
    """Workload 2: dynamic symmetric quant, per-channel weights, bf16 bias."""
    rng = rng_for(2, M, K, N)
    return dict(x=activations(rng, M, K, 0.0, int(round(0.005 * K)), 30.0),
                w=int8_weight(rng, N, K), s_w=channel_scales(rng, N),
                bias=bias_bits(rng, N))


def prefill(M, K, N):
    """Workload 3: shifted activations for the asymmetric (zero point) path."""
    rng = rng_for(3, M, K, N)
    return dict(x=activations(rng, M, K, 0.3), w=int8_weight(rng, N, K),
                s_w=channel_scales(rng, N))


def static_qkv(M=512, K=4096, widths=STATIC_WIDTHS):
    """Workload 4: fused QKV, one per-tensor scale per partition, and a static
    input scale / zero point.

    The static input parameters stand in for an offline calibration: a
    separate batch of the same distribution is drawn, and its range [lo, hi]
    (widened to contain 0) is spread over the 256 int8 codes, the zero point
    being the code nearest to where 0 lands.
    """
    N = int(sum(widths))
    rng = rng_for(4, M, K, N)
    x = activations(rng, M, K, 0.3)
    w = int8_weight(rng, N, K)
    part_scales = rng.uniform(1e-3, 1e-2, size=len(widths)).astype(np.float32)
    cal = rng_for(4, M, K, N, 1).standard_normal((M, K), dtype=np.float32) + np.float32(0.3)
    lo = min(0.0, float(cal.min()))
    hi = max(0.0, float(cal.max()))
    s_in = np.float32((hi - lo) / 255.0)
    zp_in = int(np.clip(-128 - round(lo / float(s_in)), -128, 127))
    return dict(x=x, w=w, part_scales=part_scales, widths=tuple(int(v) for v in widths),
                s_in=s_in, zp_in=np.int32(zp_in))


def fp8_e4m3fn_codes(values_f32) -> np.ndarray:
    """Encode float32 values (|v| <= 448) as OCP E4M3FN codes via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    t = t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def fp8_block_weight(rng, E, N, K, std=0.02, block=128):
    """FP8 E4M3FN weights [E,N,K] ~ N(0, std) with float32 block scales
    [E, ceil(N/128), ceil(K/128)] equal to the block's absmax / 448."""
    w = rng.normal(0.0, std, size=(E, N, K)).astype(np.float32)
    nb, kb = -(-N // block), -(-K // block)
    pad = np.zeros((E, nb * block, kb * block), np.float32)
    pad[:, :N, :K] = np.abs(w)
    amax = pad.reshape(E, nb, block, kb, block).max(axis=(2, 4))
    scales = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    full = np.repeat(np.repeat(scales, block, axis=1), block, axis=2)[:, :N, :K]
    codes = fp8_e4m3fn_codes(w / full)
    return codes, scales


def router_logits(rng, tokens, E):
    """Router logits [tokens, E] ~ N(0, 1), float32 (the routing itself is a
    step of the MoE block, not drawn here)."""
    return rng.standard_normal((tokens, E), dtype=np.float32)


def moe(tokens=MOE_TOKENS, E=MOE_E, topk=MOE_TOPK, hidden=MOE_HIDDEN, inter=MOE_INTER,
        with_weights=True):
    """Workload 5. w13 has N = 2*inter (gate and up fused), K = hidden; w2 has
    K = inter, N = hidden. The w2 input is an N(0,1) stand-in for the
    activated gate*up product, already in expert-sorted order."""
    rng = rng_for(5, tokens, E, topk, hidden, inter)
    logits = router_logits(rng, tokens, E)
    T = tokens * topk
    d = dict(logits=logits, topk=topk,
             x13=activations(rng, tokens, hidden),
             x2=activations(rng_for(5, tokens, E, topk, hidden, inter, 2), T, inter))
    if with_weights:
        d["w13_fp8"], d["w13_scales"] = fp8_block_weight(
            rng_for(5, tokens, E, topk, hidden, inter, 13), E, 2 * inter, hidden)
        d["w2_fp8"], d["w2_scales"] = fp8_block_weight(
            rng_for(5, tokens, E, topk, hidden, inter, 2, 2), E, hidden, inter)
    return d
