"""ctypes front-end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  It holds no
arithmetic of the method: every value is computed by the C oracle, this file
only allocates numpy buffers and marshals pointers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FLAG_NONFINITE = 1
FLAG_DEGENERATE = 2
SYM, AFFINE = 0, 1
E4M3, E5M2, E2M1, E2M3, E3M2 = 0, 1, 2, 3, 4
F32, BF16 = 0, 1

# Strict binary32: no FMA contraction, no fast-math, no re-association.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (always recompiles)."""
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_F = ctypes.c_float
_U32 = ctypes.c_uint32
_U8 = ctypes.c_uint8

_SIGS = {
    "orc_q_range": (_INT, [_INT, _INT, _P, _P]),
    "orc_finite_min_max": (_U32, [_P, _INT, _I64, _I64, _P, _P]),
    "orc_params_from_minmax": (_U32, [_F, _F, _INT, _INT, _P, _P]),
    "orc_quantize": (_I32, [_F, _F, _I32, _I32, _I32]),
    "orc_dequantize": (_F, [_I32, _F, _I32]),
    "orc_real_bounds": (None, [_F, _I32, _I32, _I32, _P, _P]),
    "orc_tensor_params_int": (_U32, [_P, _I64, _INT, _INT, _P, _P, _P, _P]),
    "orc_fake_quant_int": (None, [_P, _I64, _INT, _INT, _F, _I32, _P, _P]),
    "orc_dequantize_int": (None, [_P, _I64, _F, _I32, _P]),
    "orc_ste_backward": (None, [_P, _P, _I64, _F, _F, _P]),
    "orc_quant_rows": (_U32, [_P, _INT, _I64, _I64, _INT, _INT, _P, _P, _P, _P]),
    "orc_percentile_params": (_U32, [_P, _I64, _INT, _INT, ctypes.c_double, _P, _P, _P, _P, _P, _P]),
    "orc_quant_cols": (_U32, [_P, _INT, _I64, _I64, _INT, _INT, _P, _P, _P, _P]),
    "orc_quant_groups": (_U32, [_P, _INT, _I64, _I64, _I64, _INT, _INT, _P, _P, _P, _P]),
    "orc_narrow_encode": (ctypes.c_uint8, [ctypes.c_float, _INT]),
    "orc_narrow_decode": (ctypes.c_float, [ctypes.c_uint8, _INT]),
    "orc_mx_rows": (None, [_P, _INT, _I64, _I64, _INT, _P, _P, _P]),
    "orc_nvfp4": (None, [_P, _I64, _P, _P, _P, _P]),
    "orc_fp8_encode": (_U8, [_F, _INT]),
    "orc_fp8_decode": (_F, [_U8, _INT]),
    "orc_fp8_encode_n": (None, [_P, _I64, _INT, _P]),
    "orc_fp8_decode_n": (None, [_P, _I64, _INT, _P]),
    "orc_amax_finite": (_F, [_P, _I64]),
    "orc_fp8_scale": (_U32, [_F, _INT, _P]),
    "orc_fp8_quantize": (None, [_P, _I64, _INT, _F, _P, _P]),
    "orc_fp8_dequantize": (None, [_P, _I64, _INT, _F, _P]),
    "orc_q4dq_quantize": (_U32, [_P, _I64, _P, _P, _P, _P, _P]),
    "orc_q4dq_dequantize": (None, [_P, _P, _P, _I64, _P]),
    "orc_mxfp8_rows": (None, [_P, _INT, _I64, _I64, _P, _P, _P]),
    "orc_bf16_to_f32": (_F, [ctypes.c_uint16]),
    "orc_philox4x32_10": (None, [_P, _P, _P]),
    "orc_sr_uniform": (_F, [ctypes.c_uint64, ctypes.c_uint64]),
    "orc_sr_uniform_n": (None, [ctypes.c_uint64, ctypes.c_uint64, _I64, _P]),
    "orc_quantize_sr": (_I32, [_F, _F, _I32, _I32, _I32, _F]),
    "orc_fake_quant_int_sr": (None, [_P, _I64, _INT, _INT, _F, _I32, ctypes.c_uint64, ctypes.c_uint64,
                                     _P, _P]),
    "orc_fp8_encode_sr": (_U8, [_F, _INT, _F]),
    "orc_fp8_quantize_sr": (None, [_P, _I64, _INT, _F, ctypes.c_uint64, ctypes.c_uint64, _P, _P]),
    "orc_adamw_bias_corrections": (None, [_F, _F, _I64, _P, _P]),
    "orc_adamw_update": (None, [_P, _P, _P, _P, _I64, _F, _F, _F, _F, _F, _F, _F]),
    "orc_qat_step_int": (_U32, [_P, _P, _P, _P, _I64, _F, _F, _F, _F, _F, _I64, _INT, _INT, _INT,
                                ctypes.c_uint64, ctypes.c_uint64, _P, _P, _P, _P, _P, _P]),
    "orc_qat_step_fp8": (None, [_P, _P, _P, _P, _I64, _F, _F, _F, _F, _F, _I64, _INT, _INT, ctypes.c_uint64,
                                ctypes.c_uint64, _P, _P]),
}


def lib():
    """Load liboracle.so, building it first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        handle = ctypes.CDLL(LIB)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def _scalar_out(ctype):
    return ctype()


def _out(a, shape, dtype):
    """A caller's output array (C-contiguous, of this shape and dtype), or a new one."""
    if a is None:
        return np.empty(shape, dtype)
    shape = tuple(shape) if isinstance(shape, (tuple, list)) else (shape,)
    assert a.dtype == np.dtype(dtype) and a.shape == shape and a.flags["C_CONTIGUOUS"], (a.dtype, a.shape, shape)
    return a


# --- scalar helpers -----------------------------------------------------------

def q_range(bits: int, scheme: int):
    lo, hi = _I32(), _I32()
    st = lib().orc_q_range(bits, scheme, ctypes.byref(lo), ctypes.byref(hi))
    if st != 0:
        raise ValueError(f"unsupported width {bits}")
    return lo.value, hi.value


def params_from_minmax(mn: float, mx: float, bits: int, scheme: int):
    s, z = _F(), _I32()
    flags = lib().orc_params_from_minmax(mn, mx, bits, scheme, ctypes.byref(s), ctypes.byref(z))
    return s.value, z.value, flags


def quantize(x: float, scale: float, zp: int, qmin: int, qmax: int) -> int:
    return lib().orc_quantize(x, scale, zp, qmin, qmax)


def dequantize(q: int, scale: float, zp: int) -> float:
    return lib().orc_dequantize(q, scale, zp)


def fp8_encode(y: float, fmt: int) -> int:
    return lib().orc_fp8_encode(y, fmt)


def fp8_decode(b: int, fmt: int) -> float:
    return lib().orc_fp8_decode(b, fmt)


# --- array entry points ------------------------------------------------------

def finite_min_max(x):
    x = _f32(x)
    mn, mx = _F(), _F()
    flags = lib().orc_finite_min_max(_ptr(x), F32, x.size, 1, ctypes.byref(mn), ctypes.byref(mx))
    return mn.value, mx.value, flags


def tensor_params_int(x, bits: int, scheme: int):
    """Returns dict(scale, zp, lo, hi, flags) of per_tensor_minmax calibration."""
    x = _f32(x).ravel()
    s, z, lo, hi = _F(), _I32(), _F(), _F()
    flags = lib().orc_tensor_params_int(_ptr(x), x.size, bits, scheme, ctypes.byref(s),
                                        ctypes.byref(z), ctypes.byref(lo), ctypes.byref(hi))
    return dict(scale=np.float32(s.value), zp=z.value, lo=np.float32(lo.value),
                hi=np.float32(hi.value), flags=flags)


def fake_quant_int(x, bits: int, scheme: int, scale: float, zp: int, codes=None, fq=None):
    x = _f32(x).ravel()
    codes = _out(codes, x.size, np.int8)
    fq = _out(fq, x.size, np.float32)
    lib().orc_fake_quant_int(_ptr(x), x.size, bits, scheme, scale, zp, _ptr(codes), _ptr(fq))
    return codes, fq


def dequantize_int(codes, scale: float, zp: int):
    codes = np.ascontiguousarray(codes, dtype=np.int8).ravel()
    out = np.empty(codes.size, np.float32)
    lib().orc_dequantize_int(_ptr(codes), codes.size, scale, zp, _ptr(out))
    return out


def ste_backward(g, x, b0: float, b1: float, out=None):
    g = _f32(g).ravel()
    x = _f32(x).ravel()
    assert g.size == x.size
    out = _out(out, x.size, np.float32)
    lib().orc_ste_backward(_ptr(g), _ptr(x), x.size, b0, b1, _ptr(out))
    return out


def quant_rows(x, bits: int, scheme: int, dtype: int = F32, want_fq: bool = True, codes=None, fq=None, scale=None,
               zp=None):
    """x: [rows, cols] float32 array, or uint16 array of bfloat16 bits (dtype=BF16)."""
    if dtype == BF16:
        x = np.ascontiguousarray(x, dtype=np.uint16)
    else:
        x = _f32(x)
    rows, cols = x.shape
    if bits == 8:
        codes = _out(codes, (rows, cols), np.int8)
    else:
        codes = _out(codes, (rows, (cols + 1) // 2), np.uint8)
    fq = _out(fq, (rows, cols), np.float32) if want_fq else None
    scale = _out(scale, rows, np.float32)
    zp = _out(zp, rows, np.int32)
    flags = lib().orc_quant_rows(_ptr(x), dtype, rows, cols, bits, scheme, _ptr(codes), _ptr(fq),
                                 _ptr(scale), _ptr(zp))
    return dict(codes=codes, fq=fq, scale=scale, zp=zp, flags=flags)


def percentile_params(x, bits: int, scheme: int, clip_fraction: float):
    x = _f32(x).ravel()
    s, z, lo, hi, a, b = _F(), _I32(), _F(), _F(), _F(), _F()
    flags = lib().orc_percentile_params(_ptr(x), x.size, bits, scheme, clip_fraction, ctypes.byref(s), ctypes.byref(z),
                                        ctypes.byref(lo), ctypes.byref(hi), ctypes.byref(a), ctypes.byref(b))
    return dict(scale=np.float32(s.value), zp=z.value, lo=np.float32(lo.value), hi=np.float32(hi.value),
                sel_min=np.float32(a.value), sel_max=np.float32(b.value), flags=flags)


def quant_cols(x, bits: int, scheme: int, dtype: int = F32, want_fq: bool = True):
    """Per-column (axis 1) calibration + fake-quant; x as for quant_rows."""
    if dtype == BF16:
        x = np.ascontiguousarray(x, dtype=np.uint16)
    else:
        x = _f32(x)
    rows, cols = x.shape
    if bits == 8:
        codes = np.empty((rows, cols), np.int8)
    else:
        codes = np.empty((rows, (cols + 1) // 2), np.uint8)
    fq = np.empty((rows, cols), np.float32) if want_fq else None
    scale = np.empty(cols, np.float32)
    zp = np.empty(cols, np.int32)
    flags = lib().orc_quant_cols(_ptr(x), dtype, rows, cols, bits, scheme, _ptr(codes), _ptr(fq), _ptr(scale),
                                 _ptr(zp))
    return dict(codes=codes, fq=fq, scale=scale, zp=zp, flags=flags)


def quant_groups(x, group: int, bits: int, scheme: int, dtype: int = F32, want_fq: bool = True):
    """Group-wise calibration + fake-quant along the last dimension; x as for
    quant_rows; scale / zp: [rows, ceil(cols / group)]."""
    if dtype == BF16:
        x = np.ascontiguousarray(x, dtype=np.uint16)
    else:
        x = _f32(x)
    rows, cols = x.shape
    ng = (cols + group - 1) // group
    if bits == 8:
        codes = np.empty((rows, cols), np.int8)
    else:
        codes = np.empty((rows, (cols + 1) // 2), np.uint8)
    fq = np.empty((rows, cols), np.float32) if want_fq else None
    scale = np.empty((rows, ng), np.float32)
    zp = np.empty((rows, ng), np.int32)
    flags = lib().orc_quant_groups(_ptr(x), dtype, rows, cols, group, bits, scheme, _ptr(codes), _ptr(fq),
                                   _ptr(scale), _ptr(zp))
    return dict(codes=codes, fq=fq, scale=scale, zp=zp, flags=flags)


def narrow_encode(y, elem: int) -> int:
    return int(lib().orc_narrow_encode(float(np.float32(y)), elem))


def narrow_decode(code: int, elem: int) -> np.float32:
    return np.float32(lib().orc_narrow_decode(code, elem))


def mx_rows(x, elem: int, dtype: int = F32, want_fq: bool = True):
    """Block-scaled E2M1 / E2M3 / E3M2 (E8M0 scale per 32 elements along rows)."""
    if dtype == BF16:
        x = np.ascontiguousarray(x, dtype=np.uint16)
    else:
        x = _f32(x)
    rows, cols = x.shape
    q = np.empty((rows, (cols + 1) // 2) if elem == E2M1 else (rows, cols), np.uint8)
    e8m0 = np.empty((rows, (cols + 31) // 32), np.uint8)
    fq = np.empty((rows, cols), np.float32) if want_fq else None
    lib().orc_mx_rows(_ptr(x), dtype, rows, cols, elem, _ptr(q), _ptr(e8m0), _ptr(fq))
    return dict(q=q, e8m0=e8m0, fq=fq)


def nvfp4(x, want_fq: bool = True):
    """E2M1 elements, E4M3 scale per 16 elements, fp32 tensor scale (flattened x)."""
    x = _f32(x).ravel()
    n = x.size
    q = np.empty((n + 1) // 2, np.uint8)
    sb = np.empty((n + 15) // 16, np.uint8)
    g = _F()
    fq = np.empty(n, np.float32) if want_fq else None
    lib().orc_nvfp4(_ptr(x), n, _ptr(q), _ptr(sb), ctypes.byref(g), _ptr(fq))
    return dict(q=q, sbytes=sb, g=np.float32(g.value), fq=fq)


def fp8_encode_n(y, fmt: int):
    y = _f32(y).ravel()
    out = np.empty(y.size, np.uint8)
    lib().orc_fp8_encode_n(_ptr(y), y.size, fmt, _ptr(out))
    return out


def fp8_decode_n(b, fmt: int):
    b = np.ascontiguousarray(b, dtype=np.uint8).ravel()
    out = np.empty(b.size, np.float32)
    lib().orc_fp8_decode_n(_ptr(b), b.size, fmt, _ptr(out))
    return out


def amax_finite(x) -> np.float32:
    x = _f32(x).ravel()
    return np.float32(lib().orc_amax_finite(_ptr(x), x.size))


def fp8_scale(amax: float, fmt: int):
    s = _F()
    flags = lib().orc_fp8_scale(amax, fmt, ctypes.byref(s))
    return np.float32(s.value), flags


def fp8_quantize(x, fmt: int, scale: float, want_q: bool = True, want_fq: bool = True, q=None, fq=None):
    x = _f32(x).ravel()
    q = _out(q, x.size, np.uint8) if want_q else None
    fq = _out(fq, x.size, np.float32) if want_fq else None
    lib().orc_fp8_quantize(_ptr(x), x.size, fmt, scale, _ptr(q), _ptr(fq))
    return q, fq


def fp8_dequantize(q, fmt: int, scale: float, out=None):
    q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
    out = _out(out, q.size, np.float32)
    lib().orc_fp8_dequantize(_ptr(q), q.size, fmt, scale, _ptr(out))
    return out


def q4dq_sizes(n: int):
    nb = (n + 63) // 64
    return (n + 1) // 2, nb, (nb + 255) // 256


def q4dq_quantize(x, want_block_scale: bool = True, want_recon: bool = True, packed=None, qscale=None, sup=None,
                  recon=None):
    x = _f32(x).ravel()
    n = x.size
    npk, nb, ns = q4dq_sizes(n)
    packed = _out(packed, npk, np.uint8)
    qscale = _out(qscale, nb, np.uint8)
    sup = _out(sup, ns, np.float32)
    bs = np.empty(nb, np.float32) if want_block_scale else None
    recon = _out(recon, n, np.float32) if want_recon else None
    flags = lib().orc_q4dq_quantize(_ptr(x), n, _ptr(packed), _ptr(qscale), _ptr(sup), _ptr(bs),
                                    _ptr(recon))
    return dict(packed=packed, qscale=qscale, super=sup, block_scale=bs, recon=recon, flags=flags)


def q4dq_dequantize(packed, qscale, sup, n: int, out=None):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    qscale = np.ascontiguousarray(qscale, dtype=np.uint8)
    sup = _f32(sup)
    out = _out(out, n, np.float32)
    lib().orc_q4dq_dequantize(_ptr(packed), _ptr(qscale), _ptr(sup), n, _ptr(out))
    return out


def mxfp8_rows(x, dtype: int = BF16, want_fq: bool = True, q=None, e8m0=None, fq=None):
    if dtype == BF16:
        x = np.ascontiguousarray(x, dtype=np.uint16)
    else:
        x = _f32(x)
    rows, cols = x.shape
    nbr = (cols + 31) // 32
    q = _out(q, (rows, cols), np.uint8)
    e8 = _out(e8m0, (rows, nbr), np.uint8)
    fq = _out(fq, (rows, cols), np.float32) if want_fq else None
    lib().orc_mxfp8_rows(_ptr(x), dtype, rows, cols, _ptr(q), _ptr(e8), _ptr(fq))
    return dict(q=q, e8m0=e8, fq=fq)


# ---------------------------------------------------------------------------
# Stochastic rounding ([QAT] RoundingMode::Stochastic) and its Philox4x32-10 stream
# ---------------------------------------------------------------------------

def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_uniform(seed: int, index: int) -> np.float32:
    return np.float32(lib().orc_sr_uniform(seed, index))


def sr_uniform_n(seed: int, offset: int, n: int):
    out = np.empty(n, np.float32)
    lib().orc_sr_uniform_n(seed, offset, n, _ptr(out))
    return out


def quantize_sr(x: float, scale: float, zp: int, qmin: int, qmax: int, u: float) -> int:
    return lib().orc_quantize_sr(x, scale, zp, qmin, qmax, u)


def fake_quant_int_sr(x, bits: int, scheme: int, scale: float, zp: int, seed: int, offset: int = 0):
    x = _f32(x).ravel()
    codes = np.empty(x.size, np.int8)
    fq = np.empty(x.size, np.float32)
    lib().orc_fake_quant_int_sr(_ptr(x), x.size, bits, scheme, scale, zp, seed, offset, _ptr(codes),
                                _ptr(fq))
    return codes, fq


def fp8_encode_sr(y: float, fmt: int, u: float) -> int:
    return lib().orc_fp8_encode_sr(y, fmt, u)


def fp8_quantize_sr(x, fmt: int, scale: float, seed: int, offset: int = 0, want_q: bool = True,
                    want_fq: bool = True):
    x = _f32(x).ravel()
    q = np.empty(x.size, np.uint8) if want_q else None
    fq = np.empty(x.size, np.float32) if want_fq else None
    lib().orc_fp8_quantize_sr(_ptr(x), x.size, fmt, scale, seed, offset, _ptr(q), _ptr(fq))
    return q, fq


# ---------------------------------------------------------------------------
# QAT step ([QAT] QatOptimizer::step): AdamW master update, then requantize
# ---------------------------------------------------------------------------
ADAM_DEFAULTS = dict(beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def adamw_bias_corrections(beta1: float, beta2: float, t: int):
    b1, b2 = _F(), _F()
    lib().orc_adamw_bias_corrections(beta1, beta2, t, ctypes.byref(b1), ctypes.byref(b2))
    return np.float32(b1.value), np.float32(b2.value)


def _state(w, g, m, v):
    w = _f32(w).ravel().copy()
    g = _f32(g).ravel()
    m = _f32(m).ravel().copy()
    v = _f32(v).ravel().copy()
    assert w.size == g.size == m.size == v.size
    return w, g, m, v


def adamw_update(w, g, m, v, lr, t, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """One master update; returns the new (w, m, v) (inputs are not modified)."""
    w, g, m, v = _state(w, g, m, v)
    bc1, bc2 = adamw_bias_corrections(beta1, beta2, t)
    lib().orc_adamw_update(_ptr(w), _ptr(g), _ptr(m), _ptr(v), w.size, lr, beta1, beta2, eps, weight_decay,
                           float(bc1), float(bc2))
    return w, m, v


def qat_step_int(w, g, m, v, lr, t, bits=8, scheme=0, rounding=0, seed=0, offset=0, beta1=0.9,
                 beta2=0.999, eps=1e-8, weight_decay=0.0):
    w, g, m, v = _state(w, g, m, v)
    codes = np.empty(w.size, np.int8)
    view = np.empty(w.size, np.float32)
    s, z, lo, hi = _F(), _I32(), _F(), _F()
    flags = lib().orc_qat_step_int(_ptr(w), _ptr(g), _ptr(m), _ptr(v), w.size, lr, beta1, beta2, eps,
                                   weight_decay, t, bits, scheme, rounding, seed, offset, ctypes.byref(s),
                                   ctypes.byref(z), ctypes.byref(lo), ctypes.byref(hi), _ptr(codes), _ptr(view))
    return dict(w=w, m=m, v=v, scale=np.float32(s.value), zp=z.value, lo=np.float32(lo.value),
                hi=np.float32(hi.value), codes=codes, view=view, flags=flags)


def qat_step_fp8(w, g, m, v, lr, t, fmt=0, rounding=0, seed=0, offset=0, beta1=0.9, beta2=0.999,
                 eps=1e-8, weight_decay=0.0):
    w, g, m, v = _state(w, g, m, v)
    q = np.empty(w.size, np.uint8)
    view = np.empty(w.size, np.float32)
    lib().orc_qat_step_fp8(_ptr(w), _ptr(g), _ptr(m), _ptr(v), w.size, lr, beta1, beta2, eps, weight_decay, t,
                           fmt, rounding, seed, offset, _ptr(q), _ptr(view))
    return dict(w=w, m=m, v=v, q=q, view=view)
