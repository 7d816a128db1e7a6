"""w8a8_scaled_mm_int8_noalloc, the GEMM entry point that allocates nothing
(its split-K partials live in the library's static per-GPU scratch array),
through the C ABI: its outputs equal those of w8a8_scaled_mm_int8 given a
workspace, bit for bit, and the oracle's (int32 exact, bf16 within 1e-2), on
two calls in a row with the second one smaller (the array keeps the first
call's contents)."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_bf16_close, assert_equal, bf16_bits, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, seed):
    rng = synth.rng_for(960, M, K, N, seed)
    return dict(xq=rng.integers(-128, 128, (M, K), dtype=np.int8),
                w=rng.integers(-127, 128, (N, K), dtype=np.int8),
                sx=rng.uniform(1e-3, 5e-2, M).astype(np.float32),
                sw=rng.uniform(1e-3, 1e-2, N).astype(np.float32),
                zp=rng.integers(-128, 128, M).astype(np.int32),
                bias=synth.bias_bits(rng, N))


def _one(M, K, N, seed):
    d = _inputs(M, K, N, seed)
    note(f"noalloc M={M} K={K} N={N} kernel={W.scaled_mm_kernel_name(M, N, K)} "
         f"scratch={W.scaled_mm_workspace_size(M, N, K)}")
    xq, w, sx, sw = to_dev(d["xq"]), to_dev(d["w"]), to_dev(d["sx"]), to_dev(d["sw"])
    zp, cs, b = to_dev(d["zp"]), to_dev(O.colsum(d["w"])), to_dev(d["bias"])
    ws = torch.empty(max(16, W.scaled_mm_workspace_size(M, N, K)), dtype=torch.uint8, device="cuda:0")
    kw = dict(zp=zp, colsum=cs, azp_mode=W.AZP_PER_TOKEN)
    got32 = W.scaled_mm_int8_noalloc(xq, w, sx, sw, out_dtype=W.OUT_I32, **kw)
    gotbf = W.scaled_mm_int8_noalloc(xq, w, sx, sw, bias=b, **kw)
    ref32 = W.scaled_mm_int8(xq, w, sx, sw, out_dtype=W.OUT_I32, workspace=ws, **kw)
    refbf = W.scaled_mm_int8(xq, w, sx, sw, bias=b, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert_equal(host(got32), host(ref32), "int32, against the workspace entry point")
    assert_equal(bf16_bits(gotbf), bf16_bits(refbf), "bf16, against the workspace entry point")
    c = O.corrected_acc(O.int_gemm(d["xq"], d["w"]), zp=d["zp"], col_sum=O.colsum(d["w"]))
    assert_equal(host(got32), c.astype(np.int32), "int32, against the oracle")
    assert_bf16_close(bf16_bits(gotbf), O.epilogue_bf16(c, d["sx"], d["sw"], d["bias"]))


# (first call, second smaller call): split-K decode shapes with 4 and 6 token
# blocks, a one-range shape and an MFMA-tile shape, which use no scratch
@pytest.mark.parametrize("first,second", [
    ((64, 14336, 4096), (32, 8192, 1000)),
    ((96, 14336, 4096), (70, 2048, 300)),
    ((64, 4096, 28672), (17, 8192, 100)),
    ((300, 1024, 520), (48, 8192, 1000)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    assert W.scaled_mm_workspace_size(*[first[0], first[2], first[1]]) <= W.NOALLOC_SCRATCH_BYTES
    _one(*first, seed=1)
    _one(*second, seed=2)
