"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark times, through the C ABI.

Each workload runs at its real shape on the same seeded inputs the benchmark
draws; the oracle then computes the outputs it can afford one by one: every
output of the decode linears and of the static fused-QKV scheme, sampled rows
(all their columns) of the prefill and MoE products, and sampled 128-row
blocks of the FP8 expert-weight conversion. Codes, scales, zero points,
int32 sums and converted weights are compared bit for bit, bf16 outputs
within the stated 1e-2 relative bar.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_bf16_close, assert_equal, bf16_bits, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth

pytestmark = pytest.mark.gpu


def _sample_rows(M, tile, n_random, seed):
    """Rows spread over the tiles: the first and last rows, both sides of
    every few tile boundaries, and random ones."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, M // 2, M - 2, M - 1}
    for b in range(tile, M, max(tile, (M // 8) // tile * tile)):
        rows.update((b - 1, b))
    rows.update(int(r) for r in rng.choice(M, size=min(n_random, M), replace=False))
    return np.array(sorted(r for r in rows if 0 <= r < M), np.int64)


@pytest.mark.parametrize("M", synth.DECODE_M)
@pytest.mark.parametrize("K,N", synth.DECODE_KN)
def test_decode_linears_full(M, K, N):
    """The headline decode step's call (quantiser + scaled GEMM with bias, one
    call, with a workspace) on each of its 16 shapes; every output compared."""
    d = synth.decode(M, K, N)
    note(f"fullsize decode M={M} K={K} N={N} kernel={W.linear_dyn_sym_kernel_name(M, N, K)}")
    ws = torch.empty(max(16, W.scaled_mm_workspace_size(M, N, K)), dtype=torch.uint8, device="cuda:0")
    out, xq, sx = W.linear_dyn_sym(to_dev(d["x"]), to_dev(d["w"]), to_dev(d["s_w"]), bias=to_dev(d["bias"]),
                                   workspace=ws)
    torch.cuda.synchronize()
    q_ref, s_ref = O.quant_dyn_sym(d["x"])
    assert_equal(host(xq), q_ref, "codes")
    assert_equal(host(sx).view(np.uint32), s_ref.view(np.uint32), "scales")
    want, _ = O.scaled_mm(q_ref, d["w"], s_ref, d["s_w"], bias_bits=d["bias"])
    assert_bf16_close(bf16_bits(out), want)


@pytest.mark.parametrize("M", synth.PREFILL_M)
@pytest.mark.parametrize("K,N", synth.DECODE_KN)
def test_prefill_full(M, K, N):
    """Dynamic asymmetric quantisation, column sums and the scaled GEMM with
    per-token zero-point correction at the prefill shapes; the tile kernels
    (256 x 256 / 192 / 128) run over the whole K. Sampled rows compared."""
    d = synth.prefill(M, K, N)
    note(f"fullsize prefill M={M} K={K} N={N} kernel={W.scaled_mm_kernel_name(M, N, K)}")
    x, w, sw = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["s_w"])
    xq, sx, zp = W.quantize_act(x, W.QUANT_DYN_ASYM)
    cs = W.prepare_colsum(w)
    i32 = W.scaled_mm_int8(xq, w, sx, sw, zp=zp, colsum=cs, azp_mode=W.AZP_PER_TOKEN, out_dtype=W.OUT_I32)
    bf = W.scaled_mm_int8(xq, w, sx, sw, zp=zp, colsum=cs, azp_mode=W.AZP_PER_TOKEN)
    torch.cuda.synchronize()
    rows = _sample_rows(M, 256, 24, seed=M + K + N)
    rt = torch.from_numpy(rows).to("cuda:0")
    q_ref, s_ref, zp_ref = O.quant_dyn_asym(d["x"][rows])
    assert_equal(host(xq[rt]), q_ref, "codes")
    assert_equal(host(sx[rt]).view(np.uint32), s_ref.view(np.uint32), "scales")
    assert_equal(host(zp[rt]), zp_ref, "zero points")
    col = O.colsum(d["w"])
    assert_equal(host(cs), col, "column sums")
    c = O.corrected_acc(O.int_gemm(q_ref, d["w"]), zp=zp_ref, col_sum=col)
    assert_equal(host(i32[rt]), c.astype(np.int32), "int32 accumulator")
    assert_bf16_close(bf16_bits(bf[rt]), O.epilogue_bf16(c, s_ref, d["s_w"]))
    del x, w, xq, i32, bf


def test_static_qkv_full():
    """The static per-tensor scheme end to end: requantise the fused QKV to
    the largest partition scale, azp_adj, static asymmetric quantisation and
    the GEMM with the static correction. Every output compared."""
    d = synth.static_qkv()
    M, K = d["x"].shape
    N = d["w"].shape[0]
    note(f"fullsize static qkv M={M} K={K} N={N} kernel={W.scaled_mm_kernel_name(M, N, K)}")
    w = to_dev(d["w"])
    s_in = to_dev(np.array([d["s_in"]], np.float32))
    zp_in = to_dev(np.array([d["zp_in"]], np.int32))
    s_max = W.prepare_requant_max(w, to_dev(d["part_scales"]), d["widths"])
    adj = W.prepare_colsum(w, zp_in=zp_in)
    xq, _, _ = W.quantize_act(to_dev(d["x"]), W.QUANT_STATIC_ASYM, s_in=s_in, zp_in=zp_in)
    i32 = W.scaled_mm_int8(xq, w, s_in, s_max, colsum=adj, azp_mode=W.AZP_STATIC, out_dtype=W.OUT_I32)
    bf = W.scaled_mm_int8(xq, w, s_in, s_max, colsum=adj, azp_mode=W.AZP_STATIC)
    torch.cuda.synchronize()
    rw, rs = O.requant_max(d["w"], d["part_scales"], d["widths"])
    assert_equal(host(w), rw, "requantised weight")
    assert host(s_max)[0] == rs
    radj = O.azp_adj_static(rw, int(d["zp_in"]))
    assert_equal(host(adj), radj, "azp_adj")
    rq = O.quant_static(d["x"], d["s_in"], int(d["zp_in"]), symmetric=False)
    assert_equal(host(xq), rq, "codes")
    c = O.corrected_acc(O.int_gemm(rq, rw), azp_adj=radj)
    assert_equal(host(i32), c.astype(np.int32), "int32 accumulator")
    assert_bf16_close(bf16_bits(bf), O.epilogue_bf16(c, np.float32(d["s_in"]), rs))


@pytest.fixture(scope="module")
def moe_inputs():
    return synth.moe()


@pytest.mark.parametrize("name", ["w13", "w2"])
def test_moe_fp8_conversion_full(moe_inputs, name):
    """The MoE expert weights (64 experts, FP8 E4M3FN with 128 x 128 block
    scales) converted on the device in one launch; sampled 128-row blocks
    (first and last expert, the last block row, random ones) compared with the
    oracle's conversion of the same blocks."""
    codes, S = moe_inputs[name + "_fp8"], moe_inputs[name + "_scales"]
    E, N, K = codes.shape
    note(f"fullsize fp8 conversion {name} E={E} N={N} K={K}")
    q, s, flag = W.prepare_fp8_block_to_int8(to_dev(codes), to_dev(S))
    torch.cuda.synchronize()
    assert int(host(flag)[0]) == 0
    nb = -(-N // 128)
    rng = np.random.default_rng(17)
    picks = {(0, 0), (E - 1, nb - 1), (E // 2, nb // 2)}
    picks.update((int(e), int(b)) for e, b in zip(rng.integers(0, E, 5), rng.integers(0, nb, 5)))
    for e, b in sorted(picks):
        r0, r1 = 128 * b, min(128 * b + 128, N)
        rq, rs, rf = O.fp8_block_to_int8(codes[e, r0:r1], S[e, b:b + 1])
        assert rf == 0
        assert_equal(host(q[e, r0:r1]), rq, f"int8 weight expert {e} block {b}")
        assert_equal(host(s[e, r0:r1]).view(np.uint32), rs.view(np.uint32), f"row scales expert {e} block {b}")


@pytest.mark.parametrize("name", ["w13", "w2"])
def test_moe_grouped_full(moe_inputs, name):
    """The grouped GEMMs at the MoE workload's size: 32768 routed rows over 64
    experts (w13 gathers token rows through row_ids, w2 reads sorted rows),
    int8 expert weights, per-token symmetric activations. Sampled rows (every
    expert's first and last row among them) compared."""
    m = moe_inputs
    E = synth.MOE_E
    rid, off, _ = O.moe_sort(O.moe_topk(m["logits"], m["topk"])[0], E)
    T = int(off[-1])
    if name == "w13":
        K, N, x, gather = synth.MOE_HIDDEN, 2 * synth.MOE_INTER, m["x13"], True
    else:
        K, N, x, gather = synth.MOE_INTER, synth.MOE_HIDDEN, m["x2"], False
    rng = synth.rng_for(930, E, N, K)
    w = rng.integers(-127, 128, (E, N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, (E, N)).astype(np.float32)
    note(f"fullsize grouped {name} T={T} E={E} K={K} N={N}")
    q_ref, s_ref = O.quant_dyn_sym(x)  # the oracle's codes feed both sides
    xq, sxd = to_dev(q_ref), to_dev(s_ref)
    args = dict(row_ids=to_dev(rid) if gather else None, T=T)
    i32 = W.grouped_scaled_mm_int8(xq, to_dev(off), to_dev(w), sxd, to_dev(sw), out_dtype=W.OUT_I32, **args)
    bf = W.grouped_scaled_mm_int8(xq, to_dev(off), to_dev(w), sxd, to_dev(sw), **args)
    torch.cuda.synchronize()
    rows = set(_sample_rows(T, 256, 16, seed=31).tolist())
    for e in range(0, E, 7):
        if off[e + 1] > off[e]:
            rows.update((int(off[e]), int(off[e + 1]) - 1))
    rows = np.array(sorted(rows), np.int64)
    rt = torch.from_numpy(rows).to("cuda:0")
    g32, gbf = host(i32[rt]), bf16_bits(bf[rt])
    expert = np.searchsorted(off, rows, side="right") - 1
    for i, r in enumerate(rows):
        src = int(rid[r]) if gather else int(r)
        e = int(expert[i])
        acc = O.int_gemm(q_ref[src:src + 1], w[e])
        assert_equal(g32[i:i + 1], acc.astype(np.int32), f"int32 row {r} (expert {e})")
        assert_bf16_close(gbf[i:i + 1], O.epilogue_bf16(acc, s_ref[src:src + 1], sw[e]))
