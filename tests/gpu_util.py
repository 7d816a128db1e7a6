"""Host <-> device helpers for the GPU parity tests (no arithmetic of the layer)."""

import sys

import numpy as np
import torch

DEV = "cuda:0"


def note(msg):
    """Name the case on stdout before a GPU step, so a failure is attributable."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    t = torch.from_numpy(a)
    return t.to(DEV) if dtype is None else t.to(DEV, dtype)


def bf16_bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


def bf16_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bf16_close(got_bits, want_bits, rtol=1e-2):
    """The stated bar for the bf16 output: |g - o| <= rtol*|o| + 1e-6*max|o|
    element by element (the absolute term covers outputs that cancel to ~0)."""
    g = bf16_f64(got_bits)
    o = bf16_f64(want_bits)
    assert g.shape == o.shape
    if o.size == 0:
        return
    tol = rtol * np.abs(o) + 1e-6 * np.max(np.abs(o))
    bad = np.abs(g - o) > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} of {bad.size} outside tolerance, e.g. "
                             + ", ".join(f"{tuple(i)}: got {g[tuple(i)]} want {o[tuple(i)]}" for i in idx))


def assert_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]} want {want[i]}")
