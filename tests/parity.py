"""Comparison helpers for GPU-vs-oracle parity tests.

Bars (from the project's stated targets): integer codes, fp8 bytes, packed
nibbles and u8 scales bit-exact; binary32 outputs within 1 ulp with +0 == -0
and NaN == NaN; binary32 scales within 1e-6 relative.
"""
import numpy as np


def to_np(t):
    """Host numpy copy of a torch tensor (bf16 as uint16 bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    a = t.detach().cpu().numpy()
    return a


def assert_bits(actual, expected, what=""):
    a = np.ascontiguousarray(actual).reshape(-1)
    e = np.ascontiguousarray(expected).reshape(-1)
    assert a.shape == e.shape, (what, a.shape, e.shape)
    av = a.view(np.uint8) if a.dtype.itemsize == 1 else a.view(f"u{a.dtype.itemsize}")
    ev = e.view(np.uint8) if e.dtype.itemsize == 1 else e.view(f"u{e.dtype.itemsize}")
    bad = np.nonzero(av != ev)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first {[(int(i), a[i].item(), e[i].item()) for i in bad[:8]]}"


def _ordered(x):
    i = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.int32).astype(np.int64)
    return np.where(i < 0, -(2 ** 31) - i, i)


def assert_f32(actual, expected, what="", max_ulp=1, exact=True):
    """binary32 parity: within max_ulp (the stated bar, +0 == -0, NaN == NaN) and,
    with exact=True (the default; both sides run the same binary32 operations),
    bit-identical apart from NaN payloads."""
    a = np.ascontiguousarray(actual, dtype=np.float32).reshape(-1)
    e = np.ascontiguousarray(expected, dtype=np.float32).reshape(-1)
    assert a.shape == e.shape, (what, a.shape, e.shape)
    an, en = np.isnan(a), np.isnan(e)
    bad_nan = np.nonzero(an != en)[0]
    assert bad_nan.size == 0, f"{what}: NaN mismatch at {bad_nan[:8]}"
    keep = ~an
    if exact:
        ne = np.nonzero(keep & (a.view(np.uint32) != e.view(np.uint32)))[0]
        assert ne.size == 0, f"{what}: {ne.size} not bit-identical, first {[(int(i), float(a[i]), float(e[i])) for i in ne[:8]]}"
    d = np.abs(_ordered(a[keep]) - _ordered(e[keep]))
    idx = np.nonzero(keep)[0]
    bad = idx[d > max_ulp]
    assert bad.size == 0, f"{what}: {bad.size} beyond {max_ulp} ulp, first {[(int(i), float(a[i]), float(e[i])) for i in bad[:8]]}"


def assert_scale(actual, expected, what="", rel=1e-6):
    a = np.ascontiguousarray(actual, dtype=np.float64).reshape(-1)
    e = np.ascontiguousarray(expected, dtype=np.float64).reshape(-1)
    assert a.shape == e.shape
    err = np.abs(a - e)
    bad = np.nonzero(err > rel * np.abs(e))[0]
    assert bad.size == 0, f"{what}: {bad.size} scales beyond {rel} rel, first {[(int(i), a[i], e[i]) for i in bad[:8]]}"
