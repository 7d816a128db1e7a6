"""The C ABI on the host (CPU only): the library loads, exports every function
the header declares, validates schemes, and rejects bad arguments before any
device work. No call here reaches a kernel."""

import ctypes

import pytest

from int8_w8a8_quantized_amd import lib as W


@pytest.fixture(scope="module")
def L():
    return W.load()


def test_exports_every_declared_function(L):
    names = W.header_functions()
    assert len(names) == 26, names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert W.status_string(W.OK) == "W8A8_OK"
    assert W.status_string(W.ERR_NOT_IMPLEMENTED) == "W8A8_ERR_NOT_IMPLEMENTED"
    assert W.status_string(99) == "W8A8_UNKNOWN_STATUS"


@pytest.mark.parametrize("wstrat,istrat,idyn,isym,mode,chan", [
    (W.STRATEGY_CHANNEL, W.STRATEGY_TOKEN, 1, 1, W.QUANT_DYN_SYM, True),
    (W.STRATEGY_CHANNEL, W.STRATEGY_TOKEN, 1, 0, W.QUANT_DYN_ASYM, True),
    (W.STRATEGY_TENSOR, W.STRATEGY_TOKEN, 1, 1, W.QUANT_DYN_SYM, False),
    (W.STRATEGY_TENSOR, W.STRATEGY_TENSOR, 0, 0, W.QUANT_STATIC_ASYM, False),
    (W.STRATEGY_CHANNEL, W.STRATEGY_TENSOR, 0, 1, W.QUANT_STATIC_SYM, True),
])
def test_legal_schemes(wstrat, istrat, idyn, isym, mode, chan):
    """The dispatch table of "vLLM INT8 W8A8 量化实战" 4.1: 8-bit weights
    (tensor or channel, static, symmetric) with static per-tensor or dynamic
    per-token 8-bit input, symmetric or not."""
    assert W.check_scheme(weight_strategy=wstrat, input_strategy=istrat, input_dynamic=idyn,
                          input_symmetric=isym) == (mode, chan)


@pytest.mark.parametrize("kw,field", [
    (dict(weight_bits=4), "weight_bits"),
    (dict(input_bits=16), "input_bits"),
    (dict(weight_strategy=W.STRATEGY_BLOCK), "weight_strategy"),
    (dict(weight_strategy=W.STRATEGY_GROUP), "weight_strategy"),
    (dict(weight_symmetric=0), "weight_symmetric"),
    (dict(weight_dynamic=1), "weight_dynamic"),
    (dict(input_strategy=W.STRATEGY_TOKEN, input_dynamic=0), "input_dynamic"),
    (dict(input_strategy=W.STRATEGY_TENSOR, input_dynamic=1), "input_strategy"),
    (dict(input_strategy=W.STRATEGY_CHANNEL), "input_strategy"),
])
def test_illegal_schemes_raise_not_implemented(kw, field):
    with pytest.raises(NotImplementedError, match=field):
        W.check_scheme(**kw)


FAKE = 1 << 20  # a 16-byte aligned address that is never dereferenced


def test_quantize_act_rejects_before_device_work(L):
    def q(M=4, K=64, ldx=64, mode=0, x=FAKE, xq=FAKE, ldq=64, s_x=FAKE, zp=FAKE, s_in=None, zp_in=None):
        return L.w8a8_quantize_act(x, M, K, ldx, mode, s_in, zp_in, xq, ldq, s_x, zp, None)
    assert q(K=40) == W.ERR_INVALID_ARG            # K % 16
    assert q(K=0) == W.ERR_INVALID_ARG
    assert q(K=W.MAX_K + 16, ldx=W.MAX_K + 16, ldq=W.MAX_K + 16) == W.ERR_INVALID_ARG
    assert q(M=-1) == W.ERR_INVALID_ARG
    assert q(mode=7) == W.ERR_INVALID_ARG
    assert q(x=None) == W.ERR_INVALID_ARG
    assert q(x=FAKE + 8) == W.ERR_INVALID_ARG      # alignment
    assert q(ldx=60) == W.ERR_INVALID_ARG
    assert q(ldq=72) == W.ERR_INVALID_ARG          # ldq % 16
    assert q(s_x=None) == W.ERR_INVALID_ARG
    assert q(mode=W.QUANT_DYN_ASYM, zp=None) == W.ERR_INVALID_ARG
    assert q(mode=W.QUANT_STATIC_SYM) == W.ERR_INVALID_ARG   # s_in missing
    assert q(mode=W.QUANT_STATIC_ASYM, s_in=FAKE) == W.ERR_INVALID_ARG  # zp_in missing
    assert "ldq" in W.last_error() or "zp_in" in W.last_error()
    assert q(M=0) == W.OK                           # empty problem: nothing to do


def test_gemm_rejects_before_device_work(L):
    def mm(M=8, K=64, N=32, ldx=64, ldw=64, ldo=32, xq=FAKE, wq=FAKE, out=FAKE, sx=FAKE, sw=FAKE,
           zp=None, cs=None, azp=0, dt=0):
        return L.w8a8_scaled_mm_int8(xq, M, K, ldx, wq, N, ldw, sx, 1, sw, 1, zp, cs, azp, None, out,
                                     dt, ldo, None, 0, None)
    assert mm(K=24) == W.ERR_INVALID_ARG
    assert mm(ldx=48) == W.ERR_INVALID_ARG
    assert mm(ldw=72) == W.ERR_INVALID_ARG
    assert mm(ldo=20) == W.ERR_INVALID_ARG
    assert mm(out=FAKE + 4) == W.ERR_INVALID_ARG
    assert mm(azp=1) == W.ERR_INVALID_ARG          # per-token AZP needs zp and colsum
    assert mm(azp=2) == W.ERR_INVALID_ARG          # static AZP needs azp_adj
    assert mm(azp=5) == W.ERR_INVALID_ARG
    assert mm(dt=3) == W.ERR_INVALID_ARG
    assert mm(sw=None) == W.ERR_INVALID_ARG
    assert mm(M=1 << 26) == W.ERR_INVALID_ARG
    assert mm(M=0) == W.OK and mm(N=0) == W.OK

    # decode (M <= 64) shapes with 64+ steps of K and fewer than 16384 weight
    # rows split K over workgroups: int32 tiles [splits][row blocks of 64][4
    # waves][16*MF x 16], splits = min(256 / row blocks, 8, steps / 16)
    assert W.scaled_mm_workspace_size(64, 4096, 14336) == 4 * 64 * 4 * 4 * 256 * 4
    assert W.scaled_mm_workspace_size(32, 4096, 14336) == 4 * 64 * 4 * 2 * 256 * 4
    assert W.scaled_mm_workspace_size(48, 1000, 8192) == 4 * 16 * 4 * 3 * 256 * 4
    assert W.scaled_mm_workspace_size(17, 100, 8192) == 4 * 2 * 4 * 2 * 256 * 4
    assert W.scaled_mm_workspace_size(8, 4096, 14336) == 0      # M <= 16: register kernel
    assert W.scaled_mm_workspace_size(64, 4096, 4096) == 0      # fewer than 64 steps
    assert W.scaled_mm_workspace_size(64, 28672, 14336) == 0    # 16384+ weight rows
    assert W.scaled_mm_workspace_size(40, 4096, 8200) == 0      # K % 128 != 0
    # 65 - 128 rows: ranges of at least 8 steps, splits = min(256 / row blocks, 8, steps / 8)
    assert W.scaled_mm_workspace_size(65, 4096, 14336) == 4 * 64 * 4 * 5 * 256 * 4
    assert W.scaled_mm_workspace_size(128, 2048, 8192) == 8 * 32 * 4 * 8 * 256 * 4
    assert W.scaled_mm_workspace_size(128, 8200, 4096) == 0     # N > 8192: MFMA tiles
    assert W.scaled_mm_workspace_size(129, 4096, 14336) == 0    # not the decode path


def test_linear_rejects_before_device_work(L):
    def lin(M=1, K=128, N=32, ldx=128, ldw=128, ldo=32, ldq=128, x=FAKE, wq=FAKE, out=FAKE, xq=FAKE,
            sx=FAKE, sw=FAKE):
        return L.w8a8_linear_dyn_sym(x, M, K, ldx, wq, N, ldw, sw, 1, None, out, ldo, xq, ldq, sx, None, 0,
                                     None)
    assert lin(K=24) == W.ERR_INVALID_ARG
    assert lin(ldx=132) == W.ERR_INVALID_ARG       # not a multiple of 8
    assert lin(ldq=136) == W.ERR_INVALID_ARG       # not a multiple of 16
    assert lin(ldw=136) == W.ERR_INVALID_ARG
    assert lin(ldo=20) == W.ERR_INVALID_ARG
    assert lin(x=FAKE + 4) == W.ERR_INVALID_ARG
    for kw in ("x", "xq", "sx", "sw", "out", "wq"):
        assert lin(**{kw: None}) == W.ERR_INVALID_ARG, kw
    assert lin(M=-1) == W.ERR_INVALID_ARG
    assert lin(M=0) == W.OK


def test_linear_kernel_names():
    """The fused kernel for M <= 2, N <= 4096, K % 128 == 0, M * K <= 16384,
    in the register kernel's launch shape; otherwise the separate GEMM's."""
    assert W.linear_dyn_sym_kernel_name(1, 4096, 4096) == "gemv_fused_kernel<1, 8, 2>"
    assert W.linear_dyn_sym_kernel_name(2, 4096, 4096) == "gemv_fused_kernel<1, 8, 2>"
    assert W.linear_dyn_sym_kernel_name(1, 4096, 14336) == "gemv_fused_kernel<1, 4, 4>"
    assert W.linear_dyn_sym_kernel_name(1, 2048, 4096) == "gemv_fused_kernel<1, 4, 4>"
    for (M, N, K) in [(1, 6144, 4096), (1, 28672, 4096), (3, 4096, 4096), (2, 4096, 14336),
                      (1, 300, 4112), (64, 4096, 4096)]:
        assert W.linear_dyn_sym_kernel_name(M, N, K) == W.scaled_mm_kernel_name(M, N, K), (M, N, K)
    assert W.linear_dyn_sym_kernel_name(0, 300, 4096) == ""


def test_grouped_rejects_before_device_work(L):
    def g(T=16, E=4, K=64, N=32, rows=FAKE, msrc=8, off=FAKE, ldo=32):
        return L.w8a8_grouped_scaled_mm_int8(FAKE, 64, msrc, rows, off, T, E, K, N, FAKE, FAKE, FAKE,
                                             None, FAKE, 0, ldo, None)
    assert g(K=8) == W.ERR_INVALID_ARG
    assert g(off=None) == W.ERR_INVALID_ARG
    assert g(msrc=0) == W.ERR_INVALID_ARG
    assert g(ldo=16) == W.ERR_INVALID_ARG
    assert g(T=0) == W.OK and g(E=0) == W.OK


def test_prepare_rejects_before_device_work(L):
    widths = (ctypes.c_int64 * 3)(4096, 1024, 1024)
    assert L.w8a8_prepare_requant_max(FAKE, 6000, 64, 64, FAKE, widths, 3, FAKE, None, None) == W.ERR_INVALID_ARG
    assert "sum" in W.last_error()
    assert L.w8a8_prepare_requant_max(FAKE, 6144, 64, 64, FAKE, widths, 0, FAKE, None, None) == W.ERR_INVALID_ARG
    assert L.w8a8_prepare_requant_max(FAKE, 6144, 64, 64, FAKE, widths, 17, FAKE, None, None) == W.ERR_INVALID_ARG
    neg = (ctypes.c_int64 * 2)(-1, 6145)
    assert L.w8a8_prepare_requant_max(FAKE, 6144, 64, 64, FAKE, neg, 2, FAKE, None, None) == W.ERR_INVALID_ARG
    assert L.w8a8_prepare_expand_scales(FAKE, widths, 3, 6000, FAKE, None, None) == W.ERR_INVALID_ARG
    assert L.w8a8_prepare_expand_scales(FAKE, widths, 0, 6144, FAKE, None, None) == W.ERR_INVALID_ARG
    assert L.w8a8_prepare_expand_scales(FAKE, widths, 17, 6144, FAKE, None, None) == W.ERR_INVALID_ARG
    assert L.w8a8_prepare_expand_scales(FAKE, neg, 2, 6144, FAKE, None, None) == W.ERR_INVALID_ARG
    assert L.w8a8_prepare_expand_scales(None, widths, 3, 6144, FAKE, None, None) == W.ERR_INVALID_ARG
    zero = (ctypes.c_int64 * 2)(0, 0)
    assert L.w8a8_prepare_expand_scales(None, zero, 2, 0, None, None, None) == W.OK
    assert L.w8a8_prepare_fp8_block_to_int8(FAKE, FAKE, 2, 64, 72, FAKE, FAKE, FAKE, None) == W.ERR_INVALID_ARG
    assert L.w8a8_prepare_fp8_block_to_int8(FAKE, FAKE, 2, 64, 64, FAKE, FAKE, None, None) == W.ERR_INVALID_ARG
    assert L.w8a8_prepare_fp8_block_to_int8(FAKE, FAKE, 0, 64, 64, FAKE, FAKE, FAKE, None) == W.OK
    assert L.w8a8_prepare_colsum(FAKE, 16, 48, 40, None, FAKE, None) == W.ERR_INVALID_ARG
    assert L.w8a8_prepare_colsum(FAKE, 0, 48, 48, None, FAKE, None) == W.OK


def test_noalloc_scratch_covers_every_workspace():
    """No shape asks the no-allocation GEMM for more split-K scratch than its
    static array holds: the workspace sizes (host arithmetic only) over the
    decode range of M, N up to past the split limit and K up to the maximum."""
    worst = 0
    for M in range(1, 129):
        for N in (16, 100, 1000, 4096, 6144, 8064, 8192, 8200, 16384):
            for K in (128, 1024, 8192, 14336, 65536):
                worst = max(worst, W.scaled_mm_workspace_size(M, N, K))
    assert 0 < worst <= W.NOALLOC_SCRATCH_BYTES


def test_workspace_cache_keeps_replaced_buffers():
    """The binding's per-stream workspace (host tensors stand in for device
    ones): a request it covers reuses the buffer; a larger one replaces it
    with one at least twice as large and keeps the old one alive, since a
    captured graph may still use its address."""
    import torch
    dev, stream = torch.device("cpu"), 0x5EED
    W._ws_cache.pop((dev.index, stream), None)
    kept = len(W._ws_retired)
    a = W._workspace(dev, stream, 1000)
    assert a.numel() == 1000 and W._workspace(dev, stream, 600) is a
    b = W._workspace(dev, stream, 1200)
    assert b.numel() == 2000 and W._ws_retired[-1] is a
    c = W._workspace(dev, stream, 9000)
    assert c.numel() == 9000 and W._ws_retired[-1] is b
    assert len(W._ws_retired) == kept + 2
    W._ws_cache.pop((dev.index, stream))
    del W._ws_retired[kept:]


def test_noalloc_rejects_before_device_work(L):
    def mm(M=4, K=64, N=8, ldx=64, ldw=64, ldo=8, azp=0, out_dtype=0, xq=FAKE, w=FAKE, out=FAKE):
        return L.w8a8_scaled_mm_int8_noalloc(xq, M, K, ldx, w, N, ldw, FAKE, 1, FAKE, 1, None, None, azp,
                                             None, out, out_dtype, ldo, None)
    assert mm(K=40, ldx=48, ldw=48) == W.ERR_INVALID_ARG    # K % 16
    assert mm(xq=None) == W.ERR_INVALID_ARG
    assert mm(ldo=4) == W.ERR_INVALID_ARG
    assert mm(azp=W.AZP_PER_TOKEN) == W.ERR_INVALID_ARG     # zp / colsum missing
    assert mm(out_dtype=5) == W.ERR_INVALID_ARG
    assert mm(M=0) == W.OK


def test_moe_calls_reject_before_device_work(L):
    """The MoE block's calls: sizes, limits and missing buffers are refused on
    the host; empty problems are no-ops."""
    def route(tokens=8, E=64, k=8, ldl=64, ws=FAKE, nbytes=1 << 20, logits=FAKE):
        return L.w8a8_moe_route(logits, ldl, tokens, E, k, FAKE, FAKE, FAKE, FAKE, FAKE, ws, nbytes, None)
    assert route(E=0) == W.ERR_INVALID_ARG
    assert route(E=513) == W.ERR_INVALID_ARG
    assert route(k=0) == W.ERR_INVALID_ARG
    assert route(k=17) == W.ERR_INVALID_ARG
    assert route(E=4, k=5, ldl=4) == W.ERR_INVALID_ARG   # more experts asked for than exist
    assert route(ldl=32) == W.ERR_INVALID_ARG
    assert route(ws=None) == W.ERR_INVALID_ARG
    assert route(nbytes=8) == W.ERR_INVALID_ARG
    assert route(logits=None) == W.ERR_INVALID_ARG
    assert route(tokens=0) == W.OK
    assert L.w8a8_moe_route_workspace_size(4096, 64) == 128 * 64 * 8  # one 64-bit mask per expert and 32 tokens
    assert L.w8a8_moe_route_workspace_size(0, 64) == 0

    def smq(T=4, I=64, ldh=128, ldq=64, h=FAKE, act=None, ld_act=0):
        return L.w8a8_silu_mul_quant(h, T, I, ldh, FAKE, ldq, FAKE, act, ld_act, None)
    assert smq(I=40) == W.ERR_INVALID_ARG
    assert smq(I=16400, ldh=32800, ldq=16400) == W.ERR_INVALID_ARG
    assert smq(ldh=120) == W.ERR_INVALID_ARG
    assert smq(ldq=72) == W.ERR_INVALID_ARG
    assert smq(h=FAKE + 8) == W.ERR_INVALID_ARG
    assert smq(act=FAKE, ld_act=60) == W.ERR_INVALID_ARG
    assert smq(T=0) == W.OK

    def rnq(M=4, K=64, ldx=64, eps=1e-6, res=None, ldr=0, y=None, ldy=0, ldq=64, x=FAKE, g=FAKE):
        return L.w8a8_rmsnorm_quant(x, M, K, ldx, g, eps, res, ldr, y, ldy, FAKE, ldq, FAKE, None)
    assert rnq(K=40, ldx=40, ldq=48) == W.ERR_INVALID_ARG
    assert rnq(eps=0.0) == W.ERR_INVALID_ARG
    assert rnq(eps=-1e-6) == W.ERR_INVALID_ARG
    assert rnq(eps=float("inf")) == W.ERR_INVALID_ARG
    assert rnq(eps=float("nan")) == W.ERR_INVALID_ARG
    assert rnq(ldx=60) == W.ERR_INVALID_ARG
    assert rnq(ldq=72) == W.ERR_INVALID_ARG
    assert rnq(res=FAKE, ldr=56) == W.ERR_INVALID_ARG
    assert rnq(y=FAKE, ldy=60) == W.ERR_INVALID_ARG
    assert rnq(x=FAKE + 8) == W.ERR_INVALID_ARG
    assert rnq(g=None) == W.ERR_INVALID_ARG
    assert rnq(res=FAKE + 2, ldr=64) == W.ERR_INVALID_ARG
    assert rnq(res=FAKE + 4096, ldr=64, y=FAKE + 4096, ldy=64) == W.ERR_INVALID_ARG  # y is the residual
    assert rnq(M=0) == W.OK

    def comb(tokens=4, k=8, N=64, ldy=64, ldo=64, y=FAKE):
        return L.w8a8_moe_combine(y, ldy, FAKE, FAKE, tokens, k, N, FAKE, ldo, None)
    assert comb(k=17) == W.ERR_INVALID_ARG
    assert comb(N=60, ldy=60, ldo=60) == W.ERR_INVALID_ARG
    assert comb(ldo=32) == W.ERR_INVALID_ARG
    assert comb(y=None) == W.ERR_INVALID_ARG
    assert comb(tokens=0) == W.OK

    def block(tokens=8, E=8, k=2, H=64, I=32, ws=FAKE, nbytes=1 << 30):
        return L.w8a8_moe_block_int8(FAKE, H, FAKE, E, tokens, E, k, H, I, FAKE, FAKE, FAKE, FAKE, FAKE, H,
                                     ws, nbytes, None)
    assert block(H=40) == W.ERR_INVALID_ARG
    assert block(I=24) == W.ERR_INVALID_ARG
    assert block(k=9) == W.ERR_INVALID_ARG
    assert block(nbytes=1024) == W.ERR_INVALID_ARG
    assert block(ws=None) == W.ERR_INVALID_ARG
    assert block(tokens=0) == W.OK
    need = L.w8a8_moe_block_workspace_size(4096, 64, 8, 3072, 1536)
    T = 4096 * 8
    # codes, scales, routing, the int8 w2 input and one bf16 [T, 3072] buffer shared by h and y
    assert need >= 4096 * 3072 + T * 1536 + T * 3072 * 2 and need < 300 << 20
