"""The entry points under HIP graph capture, as the benchmark replays them:
each call is run eagerly for a reference, captured into a graph on the same
buffers, and the graph is replayed several times with the outputs cleared
and unrelated eager work in between; every replay must reproduce the eager
result bit for bit (every kernel here is deterministic: no atomic decides an
order or a sum)."""

import numpy as np
import pytest
import torch

from gpu_util import note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _replays(name, call, outs, n=3):
    """call() writes the tensors in outs; capture it, then replay n times."""
    note(f"graph replay: {name}")
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    junk = torch.randn((512, 512), device=DEV)
    for i in range(n):
        for o in outs:
            o.zero_()
        junk = junk @ junk.t() * 1e-3  # unrelated eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.uint8) if o.dtype == torch.bfloat16 else o,
                               r.view(torch.uint8) if r.dtype == torch.bfloat16 else r), \
                f"{name}: replay {i} output {j} differs from the eager call"
    del g


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (8, 4096, 6144), (64, 14336, 4096), (32, 4096, 28672)])
def test_linear_dyn_sym_graph(M, K, N):
    """The decode step's call: fused kernel, register kernel, split-K shared
    kernel with its reduction (workspace), shared kernel over the whole K."""
    d = synth.decode(M, K, N)
    x, w, sw, b = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["s_w"]), to_dev(d["bias"])
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    sx = torch.empty(M, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(16, W.scaled_mm_workspace_size(M, N, K)), dtype=torch.uint8, device=DEV)
    _replays(f"linear_dyn_sym {M}x{K}x{N}",
             lambda: W.linear_dyn_sym(x, w, sw, bias=b, out=out, xq=xq, s_x=sx, workspace=ws), [out, xq, sx])


def test_prefill_asym_graph():
    """Asymmetric quantiser, column sums and the tile GEMM with per-token AZP."""
    M, K, N = 600, 2048, 1536
    d = synth.prefill(M, K, N)
    x, w, sw = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["s_w"])
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    sx = torch.empty(M, dtype=torch.float32, device=DEV)
    zp = torch.empty(M, dtype=torch.int32, device=DEV)
    cs = torch.empty(N, dtype=torch.int32, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def call():
        W.quantize_act(x, W.QUANT_DYN_ASYM, xq=xq, s_x=sx, zp=zp)
        W.prepare_colsum(w, out=cs)
        W.scaled_mm_int8(xq, w, sx, sw, zp=zp, colsum=cs, azp_mode=W.AZP_PER_TOKEN, out=out)
    _replays("prefill asym", call, [xq, sx, zp, cs, out])


def test_moe_block_graph():
    """The whole int8 MoE block (routing, sort, both grouped GEMMs, SiLU
    requant, combine) in one captured call."""
    tokens, E, k, H, I = 96, 8, 2, 256, 128
    rng = np.random.default_rng(5)
    x = to_dev(synth.f32_to_bf16_bits(rng.standard_normal((tokens, H)).astype(np.float32)))
    logits = to_dev(rng.standard_normal((tokens, E)).astype(np.float32))
    w13 = to_dev(rng.integers(-127, 128, (E, 2 * I, H), dtype=np.int8))
    s13 = to_dev(rng.uniform(1e-3, 1e-2, (E, 2 * I)).astype(np.float32))
    w2 = to_dev(rng.integers(-127, 128, (E, H, I), dtype=np.int8))
    s2 = to_dev(rng.uniform(1e-3, 1e-2, (E, H)).astype(np.float32))
    out = torch.empty((tokens, H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(W.moe_block_workspace_size(tokens, E, k, H, I), dtype=torch.uint8, device=DEV)
    _replays("moe block", lambda: W.moe_block_int8(x, logits, k, w13, s13, w2, s2, out=out, workspace=ws), [out])


@pytest.mark.parametrize("w_mode", [W.FP8_W_CHANNEL, W.FP8_W_BLOCK128])
def test_fp8_graph(w_mode):
    """FP8 activation quantisation and the FP8 GEMM, both scale layouts."""
    M, K, N = 512, 1024, 768
    rng = np.random.default_rng(6)
    x = to_dev(synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    wq = to_dev((rng.integers(0, 256, (N, K)) & 0xF7).astype(np.uint8))  # no NaN codes
    act = W.FP8_ACT_TOKEN if w_mode == W.FP8_W_CHANNEL else W.FP8_ACT_GROUP128
    sw = to_dev(rng.uniform(1e-4, 1e-2, N if w_mode == W.FP8_W_CHANNEL else (N // 128, K // 128))
                .astype(np.float32))
    xq, sx = W.quantize_act_fp8(x, act)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def call():
        W.quantize_act_fp8(x, act, xq=xq, s_x=sx)
        W.scaled_mm_fp8(xq, wq, sx, sw, act, w_mode, out=out)
    _replays(f"fp8 w_mode={w_mode}", call, [xq, sx, out])


def test_rmsnorm_and_silu_graph():
    """The two quantisers fused into the op before them."""
    M, K = 48, 4096
    rng = np.random.default_rng(7)
    x = to_dev(synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    g = to_dev(synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, K).astype(np.float32)))
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    sx = torch.empty(M, dtype=torch.float32, device=DEV)
    y = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    aq = torch.empty((M, K // 2), dtype=torch.int8, device=DEV)
    sa = torch.empty(M, dtype=torch.float32, device=DEV)

    def call():
        W.rmsnorm_quant(x, g, 1e-6, xq=xq, s_x=sx, y=y)
        W.silu_mul_quant(x, K // 2, aq=aq, s_a=sa)
    _replays("rmsnorm + silu", call, [xq, sx, y, aq, sa])
