"""Python binding of libfq.so (include/fq.h): argument marshalling only.

Every function named ``fq_*`` here calls the C entry point of the same name with
device pointers taken from torch tensors and the current HIP stream; all the
arithmetic runs in the library's gfx950 kernels.  A non-zero status raises
``FqError``.  The convenience helpers at the end (``params_int`` ...) only
allocate output tensors with torch and call the ``fq_*`` functions.

There is no fallback: importing this module raises if libfq.so is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfq.so")

OK, E_INVALID, E_UNSUPPORTED, E_DIM, E_HIP = 0, -1, -2, -3, -4
FLAG_NONFINITE, FLAG_DEGENERATE = 1, 2
SYM, AFFINE = 0, 1
E4M3, E5M2, E2M1, E2M3, E3M2 = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
ROUND_NEAREST, ROUND_STOCHASTIC = 0, 1


class AdamWConfig(ctypes.Structure):
    """fq_adamw_config (include/fq.h): QatConfig's Adam / AdamW hyper-parameters."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class FqError(RuntimeError):
    def __init__(self, name: str, status: int, msg: str):
        super().__init__(f"{name}: {msg} (status {status})")
        self.status = status


class FqFlagError(FqError):
    """A data-dependent condition that a call with check=True found in its device
    flag word (status = the flag bits): the pages' InvalidState for a calibration
    group holding a non-finite value (FLAG_NONFINITE) or no usable range
    (FLAG_DEGENERATE).  The results are written all the same."""


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m fake_quant_amd.build` "
                      "(there is no non-HIP fallback)")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t
_U64 = ctypes.c_uint64

_SIGS = {
    "fq_version": (_INT, []),
    "fq_status_string": (ctypes.c_char_p, [_INT]),
    "fq_workspace_bytes": (_SZ, [_I64]),
    "fq_q4dq_sizes": (_INT, [_I64, _P, _P, _P]),
    "fq_tensor_params_int": (_INT, [_P, _I64, _INT, _INT, _P, _SZ, _P, _P, _P]),
    "fq_fake_quant_int_tensor": (_INT, [_P, _I64, _INT, _INT, _P, _P, _P, _P]),
    "fq_calibrate_fake_quant_int_tensor": (_INT, [_P, _I64, _INT, _INT, _P, _SZ, _P, _P, _P, _P, _P]),
    "fq_calibrate_fake_quant_int_tensor_noalloc": (_INT, [_P, _I64, _INT, _INT, _P, _P, _P, _P, _P]),
    "fq_dequantize_int_tensor": (_INT, [_P, _I64, _INT, _P, _P, _P]),
    "fq_ste_backward": (_INT, [_P, _I64, _P, _I64, _P, _P, _P]),
    "fq_quant_rows": (_INT, [_P, _INT, _I64, _I64, _INT, _INT, _P, _P, _P, _P, _P, _P]),
    "fq_dequantize_rows": (_INT, [_P, _I64, _I64, _INT, _P, _P, _P, _P]),
    "fq_fp8_tensor_scale": (_INT, [_P, _I64, _P, _SZ, _P, _P, _P, _P]),
    "fq_fp8_quantize": (_INT, [_P, _I64, _INT, _P, _P, _P, _P]),
    "fq_fp8_dequantize": (_INT, [_P, _I64, _INT, _P, _P, _P]),
    "fq_q4dq_quantize": (_INT, [_P, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "fq_q4dq_dequantize": (_INT, [_P, _P, _P, _I64, _P, _P]),
    "fq_mxfp8_rows": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P, _P]),
    "fq_fake_quant_int_tensor_sr": (_INT, [_P, _I64, _INT, _INT, _P, _U64, _U64, _P, _P, _P]),
    "fq_fp8_quantize_sr": (_INT, [_P, _I64, _INT, _P, _U64, _U64, _P, _P, _P]),
    "fq_cols_workspace_bytes": (_SZ, [_I64, _I64]),
    "fq_quant_cols": (_INT, [_P, _INT, _I64, _I64, _INT, _INT, _P, _SZ, _P, _P, _P, _P, _P, _P]),
    "fq_quant_groups": (_INT, [_P, _INT, _I64, _I64, _I64, _INT, _INT, _P, _P, _P, _P, _P, _P]),
    "fq_percentile_workspace_bytes": (_SZ, [_I64]),
    "fq_mx_rows": (_INT, [_P, _INT, _I64, _I64, _INT, _P, _P, _P, _P]),
    "fq_nvfp4": (_INT, [_P, _I64, _P, _SZ, _P, _P, _P, _P, _P]),
    "fq_tensor_params_percentile": (_INT, [_P, _I64, _INT, _INT, ctypes.c_double, _P, _SZ, _P, _P, _P]),
    "fq_qat_step_int": (_INT, [_P, _P, _P, _P, _I64, _P, _I64, _INT, _INT, _INT, _U64, _U64, _P, _SZ, _P, _P, _P,
                               _P, _P]),
    "fq_qat_step_fp8": (_INT, [_P, _P, _P, _P, _I64, _P, _I64, _INT, _INT, _U64, _U64, _P, _P, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTS = tuple(_SIGS)

# Measurement helpers of the benchmark (include/fq_bench.h), not steps of the method.
_BENCH_SIGS = {
    "fqb_flush": (_INT, [_P, _SZ, _P, _P]),
    "fqb_copy_f32": (_INT, [_P, _P, _I64, _P]),
}
for _name, (_res, _args) in _BENCH_SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

BENCH_EXPORTS = tuple(_BENCH_SIGS)


def lib():
    return _lib


def _ptr(t):
    """Device (or host, for tests of argument checks) address of a tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(name: str, st: int):
    if st != OK:
        raise FqError(name, st, _lib.fq_status_string(st).decode())


def _need(name: str, what: str, t, nbytes: int):
    """Host-side guard before any launch: a tensor argument must be a contiguous
    GPU tensor holding at least the bytes the call touches (the C ABI trusts the
    sizes it is given).  Plain integers are raw addresses and are passed as is."""
    if t is None or isinstance(t, int):
        return
    if not t.is_cuda:
        raise FqError(name, E_INVALID, f"{what} is not a GPU tensor")
    if not t.is_contiguous():
        raise FqError(name, E_INVALID, f"{what} is not contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise FqError(name, E_INVALID, f"{what} holds {have} bytes, the call touches {nbytes}")


def _codes_bytes(n: int, bits: int) -> int:
    return n if bits == 8 else (n + 1) // 2


# ---------------------------------------------------------------------------
# C entry points (same names, same argument order; tensors in, status checked)
# ---------------------------------------------------------------------------

def fq_version() -> int:
    return _lib.fq_version()


def fq_workspace_bytes(n: int) -> int:
    return _lib.fq_workspace_bytes(n)


def fq_q4dq_sizes(n: int):
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("fq_q4dq_sizes", _lib.fq_q4dq_sizes(n, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def fq_tensor_params_int(x, n, bits, scheme, workspace, workspace_bytes, params, flags=None, stream=None):
    nm = "fq_tensor_params_int"
    _need(nm, "x", x, 4 * n)
    _need(nm, "workspace", workspace, workspace_bytes)
    _need(nm, "params", params, 16)
    _need(nm, "flags", flags, 4)
    _check("fq_tensor_params_int",
           _lib.fq_tensor_params_int(_ptr(x), n, bits, scheme, _ptr(workspace), workspace_bytes,
                                     _ptr(params), _ptr(flags), _stream(stream)))


def fq_fake_quant_int_tensor(x, n, bits, scheme, params, codes=None, fq=None, stream=None):
    nm = "fq_fake_quant_int_tensor"
    _need(nm, "x", x, 4 * n)
    _need(nm, "params", params, 16)
    _need(nm, "codes", codes, _codes_bytes(n, bits))
    _need(nm, "fq", fq, 4 * n)
    _check("fq_fake_quant_int_tensor",
           _lib.fq_fake_quant_int_tensor(_ptr(x), n, bits, scheme, _ptr(params), _ptr(codes), _ptr(fq),
                                         _stream(stream)))


def fq_calibrate_fake_quant_int_tensor(x, n, bits, scheme, workspace, workspace_bytes, params, codes=None,
                                       fq=None, flags=None, stream=None):
    nm = "fq_calibrate_fake_quant_int_tensor"
    _need(nm, "x", x, 4 * n)
    _need(nm, "workspace", workspace, workspace_bytes)
    _need(nm, "params", params, 16)
    _need(nm, "codes", codes, _codes_bytes(n, bits))
    _need(nm, "fq", fq, 4 * n)
    _need(nm, "flags", flags, 4)
    _check(nm, _lib.fq_calibrate_fake_quant_int_tensor(_ptr(x), n, bits, scheme, _ptr(workspace), workspace_bytes,
                                                       _ptr(params), _ptr(codes), _ptr(fq), _ptr(flags),
                                                       _stream(stream)))


def fq_calibrate_fake_quant_int_tensor_noalloc(x, n, bits, scheme, params, codes=None, fq=None, flags=None,
                                               stream=None):
    nm = "fq_calibrate_fake_quant_int_tensor_noalloc"
    _need(nm, "x", x, 4 * n)
    _need(nm, "params", params, 16)
    _need(nm, "codes", codes, _codes_bytes(n, bits))
    _need(nm, "fq", fq, 4 * n)
    _need(nm, "flags", flags, 4)
    _check(nm, _lib.fq_calibrate_fake_quant_int_tensor_noalloc(_ptr(x), n, bits, scheme, _ptr(params), _ptr(codes),
                                                               _ptr(fq), _ptr(flags), _stream(stream)))


def fq_cols_workspace_bytes(rows, cols) -> int:
    return int(_lib.fq_cols_workspace_bytes(rows, cols))


def fq_quant_cols(x, dtype, rows, cols, bits, scheme, workspace, workspace_bytes, codes, fq, scale, zero_point,
                  flags=None, stream=None):
    nm = "fq_quant_cols"
    esz = 4 if dtype == F32 else 2
    _need(nm, "x", x, esz * rows * cols)
    _need(nm, "workspace", workspace, workspace_bytes)
    _need(nm, "codes", codes, rows * (cols if bits == 8 else (cols + 1) // 2))
    _need(nm, "fq", fq, 4 * rows * cols)
    _need(nm, "scale", scale, 4 * cols)
    _need(nm, "zero_point", zero_point, 4 * cols)
    _need(nm, "flags", flags, 4)
    _check(nm, _lib.fq_quant_cols(_ptr(x), dtype, rows, cols, bits, scheme, _ptr(workspace), workspace_bytes,
                                  _ptr(codes), _ptr(fq), _ptr(scale), _ptr(zero_point), _ptr(flags),
                                  _stream(stream)))


def fq_fake_quant_int_tensor_sr(x, n, bits, scheme, params, seed, offset=0, codes=None, fq=None, stream=None):
    nm = "fq_fake_quant_int_tensor_sr"
    _need(nm, "x", x, 4 * n)
    _need(nm, "params", params, 16)
    _need(nm, "codes", codes, _codes_bytes(n, bits))
    _need(nm, "fq", fq, 4 * n)
    _check(nm, _lib.fq_fake_quant_int_tensor_sr(_ptr(x), n, bits, scheme, _ptr(params), seed, offset, _ptr(codes),
                                                _ptr(fq), _stream(stream)))


def fq_dequantize_int_tensor(codes, n, bits, params, out, stream=None):
    nm = "fq_dequantize_int_tensor"
    _need(nm, "codes", codes, _codes_bytes(n, bits))
    _need(nm, "params", params, 16)
    _need(nm, "out", out, 4 * n)
    _check("fq_dequantize_int_tensor",
           _lib.fq_dequantize_int_tensor(_ptr(codes), n, bits, _ptr(params), _ptr(out), _stream(stream)))


def fq_ste_backward(grad, n_grad, x, n_x, bounds, grad_in, stream=None):
    nm = "fq_ste_backward"
    _need(nm, "grad", grad, 4 * n_grad)
    _need(nm, "x", x, 4 * n_x)
    _need(nm, "bounds", bounds, 8)
    _need(nm, "grad_in", grad_in, 4 * n_x)
    _check("fq_ste_backward",
           _lib.fq_ste_backward(_ptr(grad), n_grad, _ptr(x), n_x, _ptr(bounds), _ptr(grad_in),
                                _stream(stream)))


def fq_quant_rows(x, dtype, rows, cols, bits, scheme, codes, fq, scale, zero_point, flags=None, stream=None):
    nm = "fq_quant_rows"
    _need(nm, "x", x, rows * cols * (2 if dtype == BF16 else 4))
    _need(nm, "codes", codes, rows * _codes_bytes(cols, bits))
    _need(nm, "fq", fq, 4 * rows * cols)
    _need(nm, "scale", scale, 4 * rows)
    _need(nm, "zero_point", zero_point, 4 * rows)
    _need(nm, "flags", flags, 4)
    _check("fq_quant_rows",
           _lib.fq_quant_rows(_ptr(x), dtype, rows, cols, bits, scheme, _ptr(codes), _ptr(fq), _ptr(scale),
                              _ptr(zero_point), _ptr(flags), _stream(stream)))


def fq_dequantize_rows(codes, rows, cols, bits, scale, zero_point, out, stream=None):
    nm = "fq_dequantize_rows"
    _need(nm, "codes", codes, rows * _codes_bytes(cols, bits))
    _need(nm, "scale", scale, 4 * rows)
    _need(nm, "zero_point", zero_point, 4 * rows)
    _need(nm, "out", out, 4 * rows * cols)
    _check("fq_dequantize_rows",
           _lib.fq_dequantize_rows(_ptr(codes), rows, cols, bits, _ptr(scale), _ptr(zero_point), _ptr(out),
                                   _stream(stream)))


def fq_fp8_tensor_scale(x, n, workspace, workspace_bytes, scale_e4m3=None, scale_e5m2=None, flags=None,
                        stream=None):
    nm = "fq_fp8_tensor_scale"
    _need(nm, "x", x, 4 * n)
    _need(nm, "workspace", workspace, workspace_bytes)
    _need(nm, "scale_e4m3", scale_e4m3, 4)
    _need(nm, "scale_e5m2", scale_e5m2, 4)
    _need(nm, "flags", flags, 4)
    _check("fq_fp8_tensor_scale",
           _lib.fq_fp8_tensor_scale(_ptr(x), n, _ptr(workspace), workspace_bytes, _ptr(scale_e4m3),
                                    _ptr(scale_e5m2), _ptr(flags), _stream(stream)))


def fq_fp8_quantize(x, n, fmt, scale, q=None, fq=None, stream=None):
    nm = "fq_fp8_quantize"
    _need(nm, "x", x, 4 * n)
    _need(nm, "scale", scale, 4)
    _need(nm, "q", q, n)
    _need(nm, "fq", fq, 4 * n)
    _check("fq_fp8_quantize",
           _lib.fq_fp8_quantize(_ptr(x), n, fmt, _ptr(scale), _ptr(q), _ptr(fq), _stream(stream)))


def fq_fp8_quantize_sr(x, n, fmt, scale, seed, offset=0, q=None, fq=None, stream=None):
    nm = "fq_fp8_quantize_sr"
    _need(nm, "x", x, 4 * n)
    _need(nm, "scale", scale, 4)
    _need(nm, "q", q, n)
    _need(nm, "fq", fq, 4 * n)
    _check(nm, _lib.fq_fp8_quantize_sr(_ptr(x), n, fmt, _ptr(scale), seed, offset, _ptr(q), _ptr(fq),
                                       _stream(stream)))


def fq_qat_step_int(master, grad, m, v, n, cfg, t, bits, scheme, rounding, seed, offset, workspace,
                    workspace_bytes, params, codes=None, view=None, flags=None, stream=None):
    nm = "fq_qat_step_int"
    for what, tt in (("master", master), ("grad", grad), ("m", m), ("v", v), ("view", view)):
        _need(nm, what, tt, 4 * n)
    _need(nm, "workspace", workspace, workspace_bytes)
    _need(nm, "params", params, 16)
    _need(nm, "codes", codes, _codes_bytes(n, bits))
    _need(nm, "flags", flags, 4)
    _check(nm, _lib.fq_qat_step_int(_ptr(master), _ptr(grad), _ptr(m), _ptr(v), n, ctypes.byref(cfg), t, bits,
                                    scheme, rounding, seed, offset, _ptr(workspace), workspace_bytes, _ptr(params),
                                    _ptr(codes), _ptr(view), _ptr(flags), _stream(stream)))


def fq_qat_step_fp8(master, grad, m, v, n, cfg, t, fmt, rounding, seed, offset, q=None, view=None, stream=None):
    nm = "fq_qat_step_fp8"
    for what, tt in (("master", master), ("grad", grad), ("m", m), ("v", v), ("view", view)):
        _need(nm, what, tt, 4 * n)
    _need(nm, "q", q, n)
    _check(nm, _lib.fq_qat_step_fp8(_ptr(master), _ptr(grad), _ptr(m), _ptr(v), n, ctypes.byref(cfg), t, fmt,
                                    rounding, seed, offset, _ptr(q), _ptr(view), _stream(stream)))


def fq_fp8_dequantize(q, n, fmt, scale, out, stream=None):
    nm = "fq_fp8_dequantize"
    _need(nm, "q", q, n)
    _need(nm, "scale", scale, 4)
    _need(nm, "out", out, 4 * n)
    _check("fq_fp8_dequantize",
           _lib.fq_fp8_dequantize(_ptr(q), n, fmt, _ptr(scale), _ptr(out), _stream(stream)))


def fq_q4dq_quantize(x, n, packed, qscale, super_scale, block_scale=None, recon=None, flags=None, stream=None):
    nm = "fq_q4dq_quantize"
    nb = (n + 63) // 64
    _need(nm, "x", x, 4 * n)
    _need(nm, "packed", packed, (n + 1) // 2)
    _need(nm, "qscale", qscale, nb)
    _need(nm, "super_scale", super_scale, 4 * ((nb + 255) // 256))
    _need(nm, "block_scale", block_scale, 4 * nb)
    _need(nm, "recon", recon, 4 * n)
    _need(nm, "flags", flags, 4)
    _check("fq_q4dq_quantize",
           _lib.fq_q4dq_quantize(_ptr(x), n, _ptr(packed), _ptr(qscale), _ptr(super_scale), _ptr(block_scale),
                                 _ptr(recon), _ptr(flags), _stream(stream)))


def fq_q4dq_dequantize(packed, qscale, super_scale, n, out, stream=None):
    nm = "fq_q4dq_dequantize"
    nb = (n + 63) // 64
    _need(nm, "packed", packed, (n + 1) // 2)
    _need(nm, "qscale", qscale, nb)
    _need(nm, "super_scale", super_scale, 4 * ((nb + 255) // 256))
    _need(nm, "out", out, 4 * n)
    _check("fq_q4dq_dequantize",
           _lib.fq_q4dq_dequantize(_ptr(packed), _ptr(qscale), _ptr(super_scale), n, _ptr(out),
                                   _stream(stream)))


def fq_mxfp8_rows(x, dtype, rows, cols, q, e8m0, fq=None, stream=None):
    nm = "fq_mxfp8_rows"
    _need(nm, "x", x, rows * cols * (2 if dtype == BF16 else 4))
    _need(nm, "q", q, rows * cols)
    _need(nm, "e8m0", e8m0, rows * ((cols + 31) // 32))
    _need(nm, "fq", fq, 4 * rows * cols)
    _check("fq_mxfp8_rows",
           _lib.fq_mxfp8_rows(_ptr(x), dtype, rows, cols, _ptr(q), _ptr(e8m0), _ptr(fq), _stream(stream)))


# ---------------------------------------------------------------------------
# Convenience: allocate outputs with torch on x's device, call the entry points
# ---------------------------------------------------------------------------

def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def fq_quant_groups(x, dtype, rows, cols, group, bits, scheme, codes, fq, scale, zero_point, flags=None,
                    stream=None):
    nm = "fq_quant_groups"
    esz = 4 if dtype == F32 else 2
    ng = (cols + group - 1) // group if group > 0 else 0
    _need(nm, "x", x, esz * rows * cols)
    _need(nm, "codes", codes, rows * (cols if bits == 8 else (cols + 1) // 2))
    _need(nm, "fq", fq, 4 * rows * cols)
    _need(nm, "scale", scale, 4 * rows * ng)
    _need(nm, "zero_point", zero_point, 4 * rows * ng)
    _need(nm, "flags", flags, 4)
    _check(nm, _lib.fq_quant_groups(_ptr(x), dtype, rows, cols, group, bits, scheme, _ptr(codes), _ptr(fq),
                                    _ptr(scale), _ptr(zero_point), _ptr(flags), _stream(stream)))


def fq_mx_rows(x, dtype, rows, cols, elem, q, e8m0, fq=None, stream=None):
    nm = "fq_mx_rows"
    _need(nm, "x", x, rows * cols * (2 if dtype == BF16 else 4))
    _need(nm, "q", q, rows * ((cols + 1) // 2 if elem == E2M1 else cols))
    _need(nm, "e8m0", e8m0, rows * ((cols + 31) // 32))
    _need(nm, "fq", fq, 4 * rows * cols)
    _check(nm, _lib.fq_mx_rows(_ptr(x), dtype, rows, cols, elem, _ptr(q), _ptr(e8m0), _ptr(fq), _stream(stream)))


def fq_nvfp4(x, n, workspace, workspace_bytes, q, scales, tensor_scale, fq=None, stream=None):
    nm = "fq_nvfp4"
    _need(nm, "x", x, 4 * n)
    _need(nm, "workspace", workspace, workspace_bytes)
    _need(nm, "q", q, (n + 1) // 2)
    _need(nm, "scales", scales, (n + 15) // 16)
    _need(nm, "tensor_scale", tensor_scale, 4)
    _need(nm, "fq", fq, 4 * n)
    _check(nm, _lib.fq_nvfp4(_ptr(x), n, _ptr(workspace), workspace_bytes, _ptr(q), _ptr(scales), _ptr(tensor_scale),
                             _ptr(fq), _stream(stream)))


def fq_percentile_workspace_bytes(n) -> int:
    return int(_lib.fq_percentile_workspace_bytes(n))


def fq_tensor_params_percentile(x, n, bits, scheme, clip_fraction, workspace, workspace_bytes, params, flags=None,
                                stream=None):
    nm = "fq_tensor_params_percentile"
    _need(nm, "x", x, 4 * n)
    _need(nm, "workspace", workspace, workspace_bytes)
    _need(nm, "params", params, 16)
    _need(nm, "flags", flags, 4)
    _check(nm, _lib.fq_tensor_params_percentile(_ptr(x), n, bits, scheme, float(clip_fraction), _ptr(workspace),
                                                workspace_bytes, _ptr(params), _ptr(flags), _stream(stream)))


def _zeros_flags(like):
    return torch.zeros(1, dtype=torch.int32, device=like.device)


def raise_on_flags(name: str, flags):
    """Synchronise on the flag word and raise FqFlagError if any bit is set."""
    f = int(flags.item())
    if f:
        what = [m for bit, m in ((FLAG_NONFINITE, "a calibration group held Inf or NaN"),
                                 (FLAG_DEGENERATE, "a calibration group had no usable range")) if f & bit]
        raise FqFlagError(name, f, "; ".join(what) or "unknown flag")


def params_int(x, bits=8, scheme=SYM, check=False):
    """Per-tensor calibration -> (params int32[4] view of fq_int_params, flags)."""
    n = x.numel()
    wsb = fq_workspace_bytes(n)
    ws = _empty(max(wsb // 4, 1), torch.float32, x)
    params = _empty(4, torch.int32, x)
    flags = _zeros_flags(x)
    fq_tensor_params_int(x, n, bits, scheme, ws, wsb, params, flags)
    if check:
        raise_on_flags("params_int", flags)
    return params, flags


def params_percentile(x, clip_fraction, bits=8, scheme=SYM, check=False):
    """Per-tensor calibration on the clipped tails -> (params int32[4], flags)."""
    n = x.numel()
    wsb = fq_percentile_workspace_bytes(n)
    ws = _empty(wsb // 4, torch.float32, x)
    params = _empty(4, torch.int32, x)
    flags = _zeros_flags(x)
    fq_tensor_params_percentile(x, n, bits, scheme, clip_fraction, ws, wsb, params, flags)
    if check:
        raise_on_flags("params_percentile", flags)
    return params, flags


def params_fields(params):
    """(scale, zero_point, real_min, real_max) from an int32[4] fq_int_params buffer."""
    p = params.cpu()
    f = p.view(torch.float32)
    return float(f[0]), int(p[1]), float(f[2]), float(f[3])


def fake_quant_int_tensor(x, params, bits=8, scheme=SYM, want_codes=True, want_fq=True):
    n = x.numel()
    codes = _empty(n if bits == 8 else (n + 1) // 2, torch.int8 if bits == 8 else torch.uint8, x) if want_codes else None
    fq = _empty(n, torch.float32, x) if want_fq else None
    fq_fake_quant_int_tensor(x, n, bits, scheme, params, codes, fq)
    return codes, fq


def calibrate_fake_quant_int_tensor(x, bits=8, scheme=SYM, want_codes=True, want_fq=True, check=False):
    """Per-tensor calibration and fake-quant in one call -> (params int32[4], codes, fq, flags)."""
    n = x.numel()
    wsb = fq_workspace_bytes(n)
    ws = _empty(max(wsb // 4, 1), torch.float32, x)
    params = _empty(4, torch.int32, x)
    flags = _zeros_flags(x)
    codes = _empty(n if bits == 8 else (n + 1) // 2, torch.int8 if bits == 8 else torch.uint8, x) if want_codes else None
    fq = _empty(n, torch.float32, x) if want_fq else None
    fq_calibrate_fake_quant_int_tensor(x, n, bits, scheme, ws, wsb, params, codes, fq, flags)
    if check:
        raise_on_flags("calibrate_fake_quant_int_tensor", flags)
    return params, codes, fq, flags


def fake_quant_int_tensor_sr(x, params, seed, offset=0, bits=8, scheme=SYM, want_codes=True, want_fq=True):
    n = x.numel()
    codes = _empty(n if bits == 8 else (n + 1) // 2, torch.int8 if bits == 8 else torch.uint8, x) if want_codes else None
    fq = _empty(n, torch.float32, x) if want_fq else None
    fq_fake_quant_int_tensor_sr(x, n, bits, scheme, params, seed, offset, codes, fq)
    return codes, fq


def dequantize_int_tensor(codes, n, params, bits=8):
    out = _empty(n, torch.float32, codes)
    fq_dequantize_int_tensor(codes, n, bits, params, out)
    return out


def ste_backward(grad, x, bounds):
    out = _empty(x.numel(), torch.float32, x)
    fq_ste_backward(grad, grad.numel(), x, x.numel(), bounds, out)
    return out


def quant_rows(x, bits=8, scheme=SYM, want_codes=True, want_fq=True, check=False):
    rows, cols = x.shape
    dtype = BF16 if x.dtype == torch.bfloat16 else F32
    if want_codes:
        codes = _empty((rows, cols), torch.int8, x) if bits == 8 else _empty((rows, (cols + 1) // 2), torch.uint8, x)
    else:
        codes = None
    fq = _empty((rows, cols), torch.float32, x) if want_fq else None
    scale = _empty(rows, torch.float32, x)
    zp = _empty(rows, torch.int32, x)
    flags = _zeros_flags(x)
    fq_quant_rows(x, dtype, rows, cols, bits, scheme, codes, fq, scale, zp, flags)
    if check:
        raise_on_flags("quant_rows", flags)
    return dict(codes=codes, fq=fq, scale=scale, zp=zp, flags=flags)


def dequantize_rows(codes, rows, cols, scale, zp, bits=8):
    out = _empty((rows, cols), torch.float32, codes)
    fq_dequantize_rows(codes, rows, cols, bits, scale, zp, out)
    return out


def fp8_tensor_scale(x, check=False):
    n = x.numel()
    wsb = fq_workspace_bytes(n)
    ws = _empty(max(wsb // 4, 1), torch.float32, x)
    s = _empty(2, torch.float32, x)
    flags = _zeros_flags(x)
    fq_fp8_tensor_scale(x, n, ws, wsb, s[0:1], s[1:2], flags)
    if check:
        raise_on_flags("fp8_tensor_scale", flags)
    return s, flags


def fp8_quantize(x, fmt, scale, want_q=True, want_fq=True):
    n = x.numel()
    q = _empty(n, torch.uint8, x) if want_q else None
    fq = _empty(n, torch.float32, x) if want_fq else None
    fq_fp8_quantize(x, n, fmt, scale, q, fq)
    return q, fq


def fp8_quantize_sr(x, fmt, scale, seed, offset=0, want_q=True, want_fq=True):
    n = x.numel()
    q = _empty(n, torch.uint8, x) if want_q else None
    fq = _empty(n, torch.float32, x) if want_fq else None
    fq_fp8_quantize_sr(x, n, fmt, scale, seed, offset, q, fq)
    return q, fq


def fp8_dequantize(q, fmt, scale):
    out = _empty(q.numel(), torch.float32, q)
    fq_fp8_dequantize(q, q.numel(), fmt, scale, out)
    return out


def q4dq_quantize(x, want_block_scale=True, want_recon=True, check=False):
    n = x.numel()
    npk, nb, ns = fq_q4dq_sizes(n)
    packed = _empty(npk, torch.uint8, x)
    qscale = _empty(nb, torch.uint8, x)
    sup = _empty(ns, torch.float32, x)
    bs = _empty(nb, torch.float32, x) if want_block_scale else None
    recon = _empty(n, torch.float32, x) if want_recon else None
    flags = _zeros_flags(x)
    fq_q4dq_quantize(x, n, packed, qscale, sup, bs, recon, flags)
    if check:
        raise_on_flags("q4dq_quantize", flags)
    return dict(packed=packed, qscale=qscale, super=sup, block_scale=bs, recon=recon, flags=flags)


def q4dq_dequantize(packed, qscale, sup, n):
    out = _empty(n, torch.float32, packed)
    fq_q4dq_dequantize(packed, qscale, sup, n, out)
    return out


def mxfp8_rows(x, want_fq=True):
    rows, cols = x.shape
    dtype = BF16 if x.dtype == torch.bfloat16 else F32
    q = _empty((rows, cols), torch.uint8, x)
    e8 = _empty((rows, (cols + 31) // 32), torch.uint8, x)
    fq = _empty((rows, cols), torch.float32, x) if want_fq else None
    fq_mxfp8_rows(x, dtype, rows, cols, q, e8, fq)
    return dict(q=q, e8m0=e8, fq=fq)


# ---------------------------------------------------------------------------
# Measurement helpers (include/fq_bench.h)
# ---------------------------------------------------------------------------

def fqb_flush(scratch, nbytes, sink, stream=None):
    _need("fqb_flush", "scratch", scratch, nbytes)
    _need("fqb_flush", "sink", sink, 4)
    _check("fqb_flush", _lib.fqb_flush(_ptr(scratch), nbytes, _ptr(sink), _stream(stream)))


def fqb_copy_f32(x, y, n, stream=None):
    _need("fqb_copy_f32", "x", x, 4 * n)
    _need("fqb_copy_f32", "y", y, 4 * n)
    _check("fqb_copy_f32", _lib.fqb_copy_f32(_ptr(x), _ptr(y), n, _stream(stream)))


def adamw_config(lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    return AdamWConfig(lr, beta1, beta2, eps, weight_decay)


def qat_step_int(master, grad, m, v, t, cfg, bits=8, scheme=SYM, rounding=ROUND_NEAREST, seed=0, offset=0,
                 want_codes=True, check=False):
    """One QAT step with an integer target; master / m / v are updated in place.
    Returns dict(params, codes, view, flags)."""
    n = master.numel()
    wsb = fq_workspace_bytes(n)
    ws = _empty(max(wsb // 4, 1), torch.float32, master)
    params = _empty(4, torch.int32, master)
    flags = _zeros_flags(master)
    codes = (_empty(n if bits == 8 else (n + 1) // 2, torch.int8 if bits == 8 else torch.uint8, master)
             if want_codes else None)
    view = _empty(n, torch.float32, master)
    fq_qat_step_int(master, grad, m, v, n, cfg, t, bits, scheme, rounding, seed, offset, ws, wsb, params, codes,
                    view, flags)
    if check:
        raise_on_flags("qat_step_int", flags)
    return dict(params=params, codes=codes, view=view, flags=flags)


def qat_step_fp8(master, grad, m, v, t, cfg, fmt=E4M3, rounding=ROUND_NEAREST, seed=0, offset=0):
    """One QAT step with an fp8 target; master / m / v are updated in place.
    Returns dict(q, view)."""
    n = master.numel()
    q = _empty(n, torch.uint8, master)
    view = _empty(n, torch.float32, master)
    fq_qat_step_fp8(master, grad, m, v, n, cfg, t, fmt, rounding, seed, offset, q, view)
    return dict(q=q, view=view)


def mx_rows(x, elem, want_fq=True):
    """MXFP4 / MXFP6 (or MXFP8 with E4M3) blocks of 32 along the rows of a 2-D tensor."""
    rows, cols = x.shape
    dtype = BF16 if x.dtype == torch.bfloat16 else F32
    q = _empty((rows, (cols + 1) // 2) if elem == E2M1 else (rows, cols), torch.uint8, x)
    e8 = _empty((rows, (cols + 31) // 32), torch.uint8, x)
    fq = _empty((rows, cols), torch.float32, x) if want_fq else None
    fq_mx_rows(x, dtype, rows, cols, elem, q, e8, fq)
    return dict(q=q, e8m0=e8, fq=fq)


def nvfp4(x, want_fq=True):
    """NVFP4 of a float32 tensor (flattened): E2M1 codes, E4M3 block scales, tensor scale."""
    n = x.numel()
    wsb = fq_workspace_bytes(n)
    ws = _empty(max(wsb // 4, 4), torch.float32, x)
    q = _empty((n + 1) // 2, torch.uint8, x)
    sb = _empty((n + 15) // 16, torch.uint8, x)
    g = _empty(1, torch.float32, x)
    fq = _empty(n, torch.float32, x) if want_fq else None
    fq_nvfp4(x, n, ws, ws.numel() * 4, q, sb, g, fq)
    return dict(q=q, scales=sb, g=g, fq=fq)


def quant_groups(x, group, bits=8, scheme=SYM, want_codes=True, want_fq=True, check=False):
    """Group-wise calibration + quantize of a 2-D fp32 / bf16 tensor along its rows."""
    rows, cols = x.shape
    dtype = BF16 if x.dtype == torch.bfloat16 else F32
    ng = (cols + group - 1) // group
    codes = None
    if want_codes:
        codes = (_empty((rows, cols), torch.int8, x) if bits == 8
                 else _empty((rows, (cols + 1) // 2), torch.uint8, x))
    fq = _empty((rows, cols), torch.float32, x) if want_fq else None
    scale = _empty((rows, ng), torch.float32, x)
    zp = _empty((rows, ng), torch.int32, x)
    flags = _zeros_flags(x)
    fq_quant_groups(x, dtype, rows, cols, group, bits, scheme, codes, fq, scale, zp, flags)
    if check:
        raise_on_flags("quant_groups", flags)
    return dict(codes=codes, fq=fq, scale=scale, zp=zp, flags=flags)


def quant_cols(x, bits=8, scheme=SYM, want_codes=True, want_fq=True, check=False):
    """Per-column calibration + quantize of a 2-D fp32 / bf16 tensor."""
    rows, cols = x.shape
    dtype = BF16 if x.dtype == torch.bfloat16 else F32
    wsb = fq_cols_workspace_bytes(rows, cols)
    ws = _empty(wsb // 4, torch.float32, x)
    codes = None
    if want_codes:
        codes = (_empty((rows, cols), torch.int8, x) if bits == 8
                 else _empty((rows, (cols + 1) // 2), torch.uint8, x))
    fq = _empty((rows, cols), torch.float32, x) if want_fq else None
    scale = _empty(cols, torch.float32, x)
    zp = _empty(cols, torch.int32, x)
    flags = _zeros_flags(x)
    fq_quant_cols(x, dtype, rows, cols, bits, scheme, ws, wsb, codes, fq, scale, zp, flags)
    if check:
        raise_on_flags("quant_cols", flags)
    return dict(codes=codes, fq=fq, scale=scale, zp=zp, flags=flags)
