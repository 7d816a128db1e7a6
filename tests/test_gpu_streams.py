"""Calls on two streams at once (both at the default priority): the library
keeps no state between calls beyond what the caller passes, and the binding
gives each stream its own split-K workspace, so two sequences of GEMMs that
run concurrently -- each with the quantiser in front and the K-range
reduction behind -- must each match the oracle exactly (codes, scales and
the int32 products) and reproduce the same bits on every repetition."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_equal, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPS = 6


def _problem(seed, M, K, N):
    rng = synth.rng_for(991, seed, M, K, N)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    return x, w, sw


@pytest.mark.parametrize("M,K,N", [(32, 14336, 4096), (64, 8192, 2048), (8, 4096, 28672)])
def test_two_streams_concurrently(M, K, N):
    """Stream A and stream B each quantise their own activation and run the
    int32 GEMM REPS times into fresh outputs, enqueued alternately so that
    their kernels overlap on the GPU."""
    assert W.scaled_mm_workspace_size(M, N, K) > 0 or N > 8192  # split-K on the first two shapes
    probs = [_problem(s, M, K, N) for s in (0, 1)]
    dev = [(to_dev(x), to_dev(w), to_dev(sw)) for x, w, sw in probs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    note(f"two streams M={M} K={K} N={N} kernel={W.scaled_mm_kernel_name(M, N, K)}")
    results = [[], []]
    for _ in range(REPS):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                x, w, sw = dev[i]
                xq, sx, _ = W.quantize_act(x, W.QUANT_DYN_SYM)
                acc = W.scaled_mm_int8(xq, w, sx, sw, out_dtype=W.OUT_I32)
                results[i].append((xq, sx, acc))
    torch.cuda.synchronize()
    for i, (x, w, _) in enumerate(probs):
        q_ref, s_ref = O.quant_dyn_sym(x)
        acc_ref = O.int_gemm(q_ref, w).astype(np.int32)
        for r, (xq, sx, acc) in enumerate(results[i]):
            what = f"stream {i} repetition {r}"
            assert_equal(host(xq), q_ref, what + " codes")
            assert_equal(host(sx).view(np.uint32), s_ref.view(np.uint32), what + " scales")
            assert_equal(host(acc), acc_ref, what + " int32 products")
