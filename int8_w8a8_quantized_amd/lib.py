"""ctypes binding of libw8a8.so: argument marshalling only.

Every function here has the name of the C entry point without its ``w8a8_``
prefix, takes torch tensors that already live on the GPU, passes their device
pointers and the current HIP stream to the library, and turns a status code
into an exception: ``NotImplementedError`` for W8A8_ERR_NOT_IMPLEMENTED (an
undefined scheme), ``ValueError`` for W8A8_ERR_INVALID_ARG and
``RuntimeError`` otherwise. Output tensors are allocated here with torch when
the caller does not pass them; the library itself allocates nothing. All
arithmetic runs in the library's HIP kernels; there is no other path, and a
missing library raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw8a8.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "w8a8.h")

# enums of include/w8a8.h
OK, ERR_INVALID_ARG, ERR_NOT_IMPLEMENTED, ERR_UNSUPPORTED_DEVICE, ERR_HIP = range(5)
STRATEGY_TENSOR, STRATEGY_CHANNEL, STRATEGY_TOKEN, STRATEGY_BLOCK, STRATEGY_GROUP = range(5)
QUANT_DYN_SYM, QUANT_DYN_ASYM, QUANT_STATIC_SYM, QUANT_STATIC_ASYM = range(4)
AZP_NONE, AZP_PER_TOKEN, AZP_STATIC = range(3)
OUT_BF16, OUT_I32, OUT_F32 = range(3)
FP8_ACT_TOKEN, FP8_ACT_TENSOR, FP8_ACT_GROUP128 = range(3)
FP8_W_TENSOR, FP8_W_CHANNEL, FP8_W_BLOCK128 = range(3)
FLAG_NAN_CODE, FLAG_BAD_SCALE, FLAG_NONFINITE = 1, 2, 4
MAX_K = 65536
MAX_PARTITIONS = 16
NOALLOC_SCRATCH_BYTES = 8 << 20


class Scheme(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "weight_bits", "input_bits", "weight_strategy", "input_strategy",
        "weight_symmetric", "input_symmetric", "weight_dynamic", "input_dynamic")]


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_SIGS = {
    "w8a8_init": (_i32, [ctypes.c_int]),
    "w8a8_check_scheme": (_i32, [ctypes.POINTER(Scheme), ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "w8a8_quantize_act": (_i32, [_p, _i64, _i64, _i64, _i32, _p, _p, _p, _i64, _p, _p, _p]),
    "w8a8_prepare_colsum": (_i32, [_p, _i64, _i64, _i64, _p, _p, _p]),
    "w8a8_prepare_requant_max": (_i32, [_p, _i64, _i64, _i64, _p, ctypes.POINTER(_i64), _i32, _p, _p, _p]),
    "w8a8_prepare_expand_scales": (_i32, [_p, ctypes.POINTER(_i64), _i32, _i64, _p, _p, _p]),
    "w8a8_prepare_fp8_block_to_int8": (_i32, [_p, _p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "w8a8_scaled_mm_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "w8a8_scaled_mm_int8": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _i64, _p, _i32, _p, _i32,
                                   _p, _p, _i32, _p, _p, _i32, _i64, _p, ctypes.c_size_t, _p]),
    "w8a8_scaled_mm_int8_noalloc": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _i64, _p, _i32, _p, _i32,
                                           _p, _p, _i32, _p, _p, _i32, _i64, _p]),
    "w8a8_grouped_scaled_mm_int8": (_i32, [_p, _i64, _i64, _p, _p, _i64, _i64, _i64, _i64, _p,
                                           _p, _p, _p, _p, _i32, _i64, _p]),
    "w8a8_linear_dyn_sym": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _i64, _p, _i32, _p, _p, _i64,
                                   _p, _i64, _p, _p, ctypes.c_size_t, _p]),
    "w8a8_quantize_act_fp8": (_i32, [_p, _i64, _i64, _i64, _i32, _p, _p, _i64, _p, _p]),
    "w8a8_scaled_mm_fp8": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _i64, _p, _i32, _p, _i32, _p, _p, _i32,
                                  _i64, _p]),
    "w8a8_scaled_mm_fp8_kernel_name": (ctypes.c_char_p, [_i64, _i64, _i64, _i32]),
    "w8a8_moe_route_workspace_size": (ctypes.c_size_t, [_i64, _i64]),
    "w8a8_moe_route": (_i32, [_p, _i64, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]),
    "w8a8_silu_mul_quant": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p]),
    "w8a8_rmsnorm_quant": (_i32, [_p, _i64, _i64, _i64, _p, ctypes.c_float, _p, _i64, _p, _i64, _p, _i64, _p,
                                  _p]),
    "w8a8_moe_combine": (_i32, [_p, _i64, _p, _p, _i64, _i32, _i64, _p, _i64, _p]),
    "w8a8_moe_block_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i32, _i64, _i64]),
    "w8a8_moe_block_int8": (_i32, [_p, _i64, _p, _i64, _i64, _i64, _i32, _i64, _i64, _p, _p, _p, _p,
                                   _p, _i64, _p, ctypes.c_size_t, _p]),
    "w8a8_scaled_mm_kernel_name": (ctypes.c_char_p, [_i64, _i64, _i64]),
    "w8a8_linear_dyn_sym_kernel_name": (ctypes.c_char_p, [_i64, _i64, _i64]),
    "w8a8_status_string": (ctypes.c_char_p, [_i32]),
    "w8a8_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Open libw8a8.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m int8_w8a8_quantized_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions() -> list:
    """Names of the functions include/w8a8.h declares."""
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:w8a8_status|size_t|const char\*)\s+(w8a8_\w+)\s*\(", text, re.M)))


def _raise(status: int, what: str):
    if status == OK:
        return
    L = load()
    msg = f"{what}: {L.w8a8_status_string(status).decode()}: {L.w8a8_last_error().decode()}"
    if status == ERR_NOT_IMPLEMENTED:
        raise NotImplementedError(msg)
    if status == ERR_INVALID_ARG:
        raise ValueError(msg)
    raise RuntimeError(msg)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def status_string(status: int) -> str:
    return load().w8a8_status_string(status).decode()


def last_error() -> str:
    return load().w8a8_last_error().decode()


def init(device: int = 0) -> None:
    _raise(load().w8a8_init(device), "w8a8_init")


def check_scheme(weight_bits=8, input_bits=8, weight_strategy=STRATEGY_CHANNEL,
                 input_strategy=STRATEGY_TOKEN, weight_symmetric=1, input_symmetric=1,
                 weight_dynamic=0, input_dynamic=1):
    """Returns (quant_mode, is_channelwise) or raises NotImplementedError."""
    s = Scheme(weight_bits, input_bits, weight_strategy, input_strategy, weight_symmetric,
               input_symmetric, weight_dynamic, input_dynamic)
    mode, chan = _i32(-1), _i32(-1)
    _raise(load().w8a8_check_scheme(ctypes.byref(s), ctypes.byref(mode), ctypes.byref(chan)),
           "w8a8_check_scheme")
    return mode.value, bool(chan.value)


def quantize_act(x, mode: int = QUANT_DYN_SYM, s_in=None, zp_in=None, xq=None, s_x=None, zp=None):
    """x: bf16 [M,K] on the GPU. Returns (xq int8 [M,K], s_x float [M] or None, zp int32 [M] or None)."""
    import torch
    M, K = x.shape
    dev = x.device
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    dyn = mode in (QUANT_DYN_SYM, QUANT_DYN_ASYM)
    if dyn and s_x is None:
        s_x = torch.empty(M, dtype=torch.float32, device=dev)
    if mode == QUANT_DYN_ASYM and zp is None:
        zp = torch.empty(M, dtype=torch.int32, device=dev)
    st = load().w8a8_quantize_act(_ptr(x), M, K, x.stride(0), mode, _ptr(s_in), _ptr(zp_in),
                                  _ptr(xq), M and xq.stride(0) or K, _ptr(s_x) if dyn else None,
                                  _ptr(zp) if mode == QUANT_DYN_ASYM else None, _stream())
    _raise(st, "w8a8_quantize_act")
    return xq, (s_x if dyn else None), (zp if mode == QUANT_DYN_ASYM else None)


def prepare_colsum(W, zp_in=None, out=None):
    """W: int8 [N,K]. Returns int32 [N] (times *zp_in when given)."""
    import torch
    N, K = W.shape
    if out is None:
        out = torch.empty(N, dtype=torch.int32, device=W.device)
    _raise(load().w8a8_prepare_colsum(_ptr(W), N, K, W.stride(0), _ptr(zp_in), _ptr(out), _stream()),
           "w8a8_prepare_colsum")
    return out


def prepare_requant_max(W, part_scales, logical_widths: Sequence[int], err_flag=None, s_max=None):
    """Requantises W (int8 [N,K]) in place. Returns the device scalar s_max (float [1])."""
    import torch
    N, K = W.shape
    if s_max is None:
        s_max = torch.empty(1, dtype=torch.float32, device=W.device)
    widths = (_i64 * len(logical_widths))(*[int(v) for v in logical_widths])
    _raise(load().w8a8_prepare_requant_max(_ptr(W), N, K, W.stride(0), _ptr(part_scales), widths,
                                           len(logical_widths), _ptr(s_max), _ptr(err_flag), _stream()),
           "w8a8_prepare_requant_max")
    return s_max


def prepare_expand_scales(part_scales, logical_widths: Sequence[int], err_flag=None, s_w=None):
    """Per-channel scales float [N] from one scale per fused partition."""
    import torch
    N = int(sum(int(v) for v in logical_widths))
    if s_w is None:
        s_w = torch.empty(N, dtype=torch.float32, device=part_scales.device)
    widths = (_i64 * len(logical_widths))(*[int(v) for v in logical_widths])
    _raise(load().w8a8_prepare_expand_scales(_ptr(part_scales), widths, len(logical_widths), N,
                                             _ptr(s_w), _ptr(err_flag), _stream()),
           "w8a8_prepare_expand_scales")
    return s_w


def prepare_fp8_block_to_int8(W8, S, Wq=None, s=None, err_flag=None):
    """W8: uint8 [E,N,K] (or [N,K]) E4M3FN codes, S: float block scales.
    Returns (Wq int8, s float [E,N] (or [N]), err_flag int32 [1])."""
    import torch
    squeeze = W8.dim() == 2
    W8v = W8.unsqueeze(0) if squeeze else W8
    E, N, K = W8v.shape
    if Wq is None:
        Wq = torch.empty((E, N, K), dtype=torch.int8, device=W8.device)
    if s is None:
        s = torch.empty((E, N), dtype=torch.float32, device=W8.device)
    if err_flag is None:
        err_flag = torch.zeros(1, dtype=torch.int32, device=W8.device)
    _raise(load().w8a8_prepare_fp8_block_to_int8(_ptr(W8v), _ptr(S), E, N, K, _ptr(Wq), _ptr(s),
                                                 _ptr(err_flag), _stream()),
           "w8a8_prepare_fp8_block_to_int8")
    if squeeze:
        return Wq.view(N, K), s.view(N), err_flag
    return Wq, s, err_flag


def scaled_mm_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace scaled_mm_int8 can use for this shape (0: none)."""
    return int(load().w8a8_scaled_mm_workspace_size(M, N, K))


_ws_cache = {}
_ws_retired = []


def _workspace(device, stream: int, nbytes: int):
    """A workspace of at least nbytes kept per (device, stream); the library
    keeps no state in it, so calls ordered on one stream can share it. A
    buffer that a larger request replaces is kept alive (never freed), since
    a HIP graph captured with it may still write there on replay; a
    replacement is at least twice the size it replaces, so the buffers kept
    alive add up to less than the largest one."""
    import torch
    key = (device.index, stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _ws_retired.append(ws)
            nbytes = max(nbytes, 2 * ws.numel())
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def scaled_mm_kernel_name(M: int, N: int, K: int) -> str:
    """Name of the kernel instance scaled_mm_int8 launches for this shape."""
    return load().w8a8_scaled_mm_kernel_name(M, N, K).decode()


def scaled_mm_int8(xq, Wq, s_x, s_w, zp=None, colsum=None, azp_mode: int = AZP_NONE, bias=None,
                   out_dtype: int = OUT_BF16, out=None, workspace=None):
    """xq int8 [M,K], Wq int8 [N,K], s_x float [M] or [1], s_w float [N] or [1],
    zp int32 [M] / colsum int32 [N] (AZP_PER_TOKEN) or azp_adj int32 [N] as
    colsum (AZP_STATIC), bias bf16 [N]. Returns bf16 (or int32) [M,N].
    workspace: None = a buffer cached per device and stream, sized by
    scaled_mm_workspace_size; a tensor = that buffer; False = none (unsplit)."""
    import torch
    M, K = xq.shape
    N = Wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.int32,
                          device=xq.device)
    if workspace is None:
        need = scaled_mm_workspace_size(M, N, K)
        workspace = _workspace(xq.device, _stream(), need) if need else False
    if workspace is False:
        workspace = None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().w8a8_scaled_mm_int8(_ptr(xq), M, K, xq.stride(0), _ptr(Wq), N, Wq.stride(0),
                                    _ptr(s_x), int(s_x.numel() != 1 or M == 1), _ptr(s_w),
                                    int(s_w.numel() != 1 or N == 1), _ptr(zp), _ptr(colsum), azp_mode,
                                    _ptr(bias), _ptr(out), out_dtype, out.stride(0) if M else N,
                                    _ptr(workspace), ws_bytes, _stream())
    _raise(st, "w8a8_scaled_mm_int8")
    return out


def scaled_mm_int8_noalloc(xq, Wq, s_x, s_w, zp=None, colsum=None, azp_mode: int = AZP_NONE, bias=None,
                           out_dtype: int = OUT_BF16, out=None):
    """scaled_mm_int8 through the entry point that allocates nothing: split-K
    partials live in the library's static per-GPU scratch array (calls that
    overlap on one GPU race). `out` is allocated here when not given; pass it
    where nothing may be allocated."""
    import torch
    M, K = xq.shape
    N = Wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.int32,
                          device=xq.device)
    st = load().w8a8_scaled_mm_int8_noalloc(_ptr(xq), M, K, xq.stride(0), _ptr(Wq), N, Wq.stride(0),
                                            _ptr(s_x), int(s_x.numel() != 1 or M == 1), _ptr(s_w),
                                            int(s_w.numel() != 1 or N == 1), _ptr(zp), _ptr(colsum),
                                            azp_mode, _ptr(bias), _ptr(out), out_dtype,
                                            out.stride(0) if M else N, _stream())
    _raise(st, "w8a8_scaled_mm_int8_noalloc")
    return out


def linear_dyn_sym(x, Wq, s_w, bias=None, out=None, xq=None, s_x=None, workspace=None):
    """The dynamic per-token symmetric linear layer in one call: x bf16 [M,K],
    Wq int8 [N,K], s_w float [N] or [1], bias bf16 [N]. Returns (out bf16
    [M,N], xq int8 [M,K], s_x float [M]), identical to quantize_act(x,
    QUANT_DYN_SYM) followed by scaled_mm_int8. workspace as for
    scaled_mm_int8."""
    import torch
    M, K = x.shape
    N = Wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_x is None:
        s_x = torch.empty((M,), dtype=torch.float32, device=x.device)
    if workspace is None:
        need = scaled_mm_workspace_size(M, N, K)
        workspace = _workspace(x.device, _stream(), need) if need else False
    if workspace is False:
        workspace = None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().w8a8_linear_dyn_sym(_ptr(x), M, K, x.stride(0) if M else K, _ptr(Wq), N,
                                    Wq.stride(0) if N else K, _ptr(s_w), int(s_w.numel() != 1 or N == 1),
                                    _ptr(bias), _ptr(out), out.stride(0) if M else N, _ptr(xq),
                                    xq.stride(0) if M else K, _ptr(s_x), _ptr(workspace), ws_bytes,
                                    _stream())
    _raise(st, "w8a8_linear_dyn_sym")
    return out, xq, s_x


def linear_dyn_sym_kernel_name(M: int, N: int, K: int) -> str:
    """Kernel that linear_dyn_sym runs for the GEMM of an M x N x K shape."""
    return load().w8a8_linear_dyn_sym_kernel_name(M, N, K).decode()


def grouped_scaled_mm_int8(xq, expert_offsets, Wq, s_x, s_w, row_ids=None, bias=None, T=None,
                           out_dtype: int = OUT_BF16, out=None):
    """xq int8 [M_src,K] (gathered through row_ids [T]) or [T,K]; expert_offsets
    int32 [E+1] on the device; Wq int8 [E,N,K]; s_x float per row of xq;
    s_w float [E,N]; bias bf16 [E,N]. T (host int) defaults to row_ids' length
    or xq's rows. Returns bf16 (or int32) [T,N] in expert-sorted order."""
    import torch
    E, N, K = Wq.shape
    if T is None:
        T = row_ids.shape[0] if row_ids is not None else xq.shape[0]
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.int32,
                          device=xq.device)
    st = load().w8a8_grouped_scaled_mm_int8(_ptr(xq), xq.stride(0), xq.shape[0], _ptr(row_ids),
                                            _ptr(expert_offsets), T, E, K, N, _ptr(Wq), _ptr(s_x),
                                            _ptr(s_w), _ptr(bias), _ptr(out), out_dtype,
                                            out.stride(0) if T else N, _stream())
    _raise(st, "w8a8_grouped_scaled_mm_int8")
    return out


def moe_route(logits, topk: int, workspace=None, out=None):
    """Top-k routing and the expert sort of float router logits [tokens, E].
    Returns (topk_ids int32 [tokens, k], topk_w float [tokens, k], row_ids
    int32 [tokens*k], expert_offsets int32 [E+1], pos int32 [tokens, k]);
    `out` may pass those five tensors in."""
    import torch
    tokens, E = logits.shape
    dev = logits.device
    if out is None:
        out = (torch.empty((tokens, topk), dtype=torch.int32, device=dev),
               torch.empty((tokens, topk), dtype=torch.float32, device=dev),
               torch.empty(tokens * topk, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty((tokens, topk), dtype=torch.int32, device=dev))
    ids, w, rows, off, pos = out
    if workspace is None:
        workspace = torch.empty(max(16, int(load().w8a8_moe_route_workspace_size(tokens, E))),
                                dtype=torch.uint8, device=dev)
    st = load().w8a8_moe_route(_ptr(logits), logits.stride(0) if tokens else E, tokens, E, topk, _ptr(ids),
                               _ptr(w), _ptr(rows), _ptr(off), _ptr(pos), _ptr(workspace),
                               workspace.numel(), _stream())
    _raise(st, "w8a8_moe_route")
    return ids, w, rows, off, pos


def silu_mul_quant(h, inter: int, aq=None, s_a=None, act=None, want_act=False):
    """h bf16 [T, 2*inter] (gate, then up). Returns (aq int8 [T, inter], s_a
    float [T], act bf16 [T, inter] or None)."""
    import torch
    T = h.shape[0]
    dev = h.device
    if aq is None:
        aq = torch.empty((T, inter), dtype=torch.int8, device=dev)
    if s_a is None:
        s_a = torch.empty(T, dtype=torch.float32, device=dev)
    if act is None and want_act:
        act = torch.empty((T, inter), dtype=torch.bfloat16, device=dev)
    st = load().w8a8_silu_mul_quant(_ptr(h), T, inter, h.stride(0) if T else 2 * inter, _ptr(aq),
                                    aq.stride(0) if T else inter, _ptr(s_a), _ptr(act),
                                    act.stride(0) if act is not None and T else inter, _stream())
    _raise(st, "w8a8_silu_mul_quant")
    return aq, s_a, act


def rmsnorm_quant(x, gamma, eps: float, residual=None, xq=None, s_x=None, y=None, want_y=False):
    """x bf16 [M, K], gamma bf16 [K]; residual (bf16 [M, K], updated in place
    to x + residual) optional. Returns (xq int8 [M, K], s_x float [M], y bf16
    [M, K] or None)."""
    import torch
    M, K = x.shape
    dev = x.device
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    if s_x is None:
        s_x = torch.empty(M, dtype=torch.float32, device=dev)
    if y is None and want_y:
        y = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    st = load().w8a8_rmsnorm_quant(_ptr(x), M, K, x.stride(0) if M else K, _ptr(gamma), eps, _ptr(residual),
                                   residual.stride(0) if residual is not None and M else K, _ptr(y),
                                   y.stride(0) if y is not None and M else K, _ptr(xq), xq.stride(0) if M else K,
                                   _ptr(s_x), _stream())
    _raise(st, "w8a8_rmsnorm_quant")
    return xq, s_x, y


def moe_combine(y, pos, topk_w, out=None):
    """out[t] = sum_j topk_w[t, j] * y[pos[t, j]]: y bf16 [T, N] (sorted rows),
    pos int32 / topk_w float [tokens, k]. Returns bf16 [tokens, N]."""
    import torch
    tokens, k = pos.shape
    N = y.shape[1]
    if out is None:
        out = torch.empty((tokens, N), dtype=torch.bfloat16, device=y.device)
    st = load().w8a8_moe_combine(_ptr(y), y.stride(0) if y.shape[0] else N, _ptr(pos), _ptr(topk_w), tokens, k,
                                 N, _ptr(out), out.stride(0) if tokens else N, _stream())
    _raise(st, "w8a8_moe_combine")
    return out


def moe_block_workspace_size(tokens: int, E: int, topk: int, H: int, inter: int) -> int:
    return int(load().w8a8_moe_block_workspace_size(tokens, E, topk, H, inter))


def moe_block_int8(x, logits, topk: int, w13, s13, w2, s2, out=None, workspace=None):
    """The int8 MoE expert block: x bf16 [tokens, H], logits float [tokens, E],
    w13 int8 [E, 2I, H] with s13 float [E, 2I], w2 int8 [E, H, I] with s2
    float [E, H]. Returns bf16 [tokens, H]."""
    import torch
    tokens, H = x.shape
    E = logits.shape[1]
    inter = w2.shape[2]
    if out is None:
        out = torch.empty((tokens, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(16, moe_block_workspace_size(tokens, E, topk, H, inter)),
                                dtype=torch.uint8, device=x.device)
    st = load().w8a8_moe_block_int8(_ptr(x), x.stride(0) if tokens else H, _ptr(logits),
                                    logits.stride(0) if tokens else E, tokens, E, topk, H, inter, _ptr(w13),
                                    _ptr(s13), _ptr(w2), _ptr(s2), _ptr(out), out.stride(0) if tokens else H,
                                    _ptr(workspace), workspace.numel(), _stream())
    _raise(st, "w8a8_moe_block_int8")
    return out


def quantize_act_fp8(x, mode: int = FP8_ACT_TOKEN, s_in=None, xq=None, s_x=None):
    """E4M3 codes of bf16 x [M, K] (as uint8). Returns (xq uint8 [M, K],
    s_x: float [M] (TOKEN), float [G, M] (GROUP128) or None (TENSOR))."""
    import torch
    M, K = x.shape
    dev = x.device
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if s_x is None and mode != FP8_ACT_TENSOR:
        s_x = torch.empty(M if mode == FP8_ACT_TOKEN else (-(-K // 128), M), dtype=torch.float32, device=dev)
    st = load().w8a8_quantize_act_fp8(_ptr(x), M, K, x.stride(0) if M else K, mode, _ptr(s_in), _ptr(xq),
                                      xq.stride(0) if M else K, _ptr(s_x) if mode != FP8_ACT_TENSOR else None,
                                      _stream())
    _raise(st, "w8a8_quantize_act_fp8")
    return xq, (s_x if mode != FP8_ACT_TENSOR else None)


def scaled_mm_fp8(xq, Wq, s_x, s_w, act_mode: int, w_mode: int, bias=None, out_dtype: int = OUT_BF16, out=None):
    """The W8A8 FP8 GEMM on E4M3 codes (uint8): xq [M, K], Wq [N, K]; scales as
    w8a8_scaled_mm_fp8 documents. Returns bf16 (or float32) [M, N]."""
    import torch
    M, K = xq.shape
    N = Wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32,
                          device=xq.device)
    st = load().w8a8_scaled_mm_fp8(_ptr(xq), M, K, xq.stride(0) if M else K, _ptr(Wq), N,
                                   Wq.stride(0) if N else K, _ptr(s_x), act_mode, _ptr(s_w), w_mode, _ptr(bias),
                                   _ptr(out), out_dtype, out.stride(0) if M else N, _stream())
    _raise(st, "w8a8_scaled_mm_fp8")
    return out


def scaled_mm_fp8_kernel_name(M: int, N: int, K: int, w_mode: int) -> str:
    return load().w8a8_scaled_mm_fp8_kernel_name(M, N, K, w_mode).decode()
