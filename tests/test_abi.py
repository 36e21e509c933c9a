"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libfq.so loads and exports every function include/fq.h declares;
* pure host helpers (version, status strings, workspace and double-quant sizes);
* argument checks return their status before anything is enqueued (every call
  here is rejected by the checks, so no HIP call is made): unsupported widths /
  schemes / formats / dtypes (the pages' UnsupportedOperation), empty tensors and
  null buffers (InvalidState for arguments), length mismatch (DimensionMismatch);
* the oracle and the product share no code.
"""
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fq.h")
BENCH_HEADER = os.path.join(ROOT, "include", "fq_bench.h")


@pytest.fixture(scope="module")
def fq():
    lib = os.path.join(ROOT, "fake_quant_amd", "libfq.so")
    if not os.path.exists(lib):
        from fake_quant_amd import build
        build.build()
    from fake_quant_amd import fq as mod
    return mod


def declared_functions(header=HEADER, prefix="fq_"):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(rf"\b({prefix}[a-z0-9_]+)\s*\(", text)))


def header_define(name):
    m = re.search(rf"#define\s+{name}\s+\(?(-?\d+)u?\)?", open(HEADER).read())
    return int(m.group(1))


def test_exports_every_declared_symbol(fq):
    decl = declared_functions()
    assert len(decl) == 29
    for name in decl:
        assert hasattr(fq.lib(), name), name
    assert sorted(fq.EXPORTS) == decl


def test_exports_bench_helpers(fq):
    decl = declared_functions(BENCH_HEADER, "fqb_")
    assert decl == ["fqb_copy_f32", "fqb_flush"]
    for name in decl:
        assert hasattr(fq.lib(), name), name
    assert sorted(fq.BENCH_EXPORTS) == decl
    L = fq.lib()
    P = FAKE
    assert L.fqb_flush(None, 1 << 20, P, None) == fq.E_INVALID
    assert L.fqb_flush(P, 8, P, None) == fq.E_INVALID
    assert L.fqb_flush(P + 4, 1 << 20, P, None) == fq.E_INVALID
    assert L.fqb_copy_f32(P, P + 4096, 6, None) == fq.E_INVALID
    assert L.fqb_copy_f32(P + 4, P + 4096, 8, None) == fq.E_INVALID
    assert L.fqb_copy_f32(P, None, 8, None) == fq.E_INVALID


def test_constants_match_header(fq):
    assert fq.fq_version() == header_define("FQ_ABI_VERSION")
    for name, val in [("FQ_OK", fq.OK), ("FQ_E_INVALID", fq.E_INVALID), ("FQ_E_UNSUPPORTED", fq.E_UNSUPPORTED),
                      ("FQ_E_DIM", fq.E_DIM), ("FQ_E_HIP", fq.E_HIP),
                      ("FQ_FLAG_NONFINITE", fq.FLAG_NONFINITE), ("FQ_FLAG_DEGENERATE", fq.FLAG_DEGENERATE)]:
        assert header_define(name) == val, name
    text = open(HEADER).read()
    for name, val in [("FQ_E4M3", fq.E4M3), ("FQ_E5M2", fq.E5M2), ("FQ_E2M1", fq.E2M1), ("FQ_E2M3", fq.E2M3),
                      ("FQ_E3M2", fq.E3M2), ("FQ_F32", fq.F32), ("FQ_BF16", fq.BF16), ("FQ_SYM", fq.SYM),
                      ("FQ_AFFINE", fq.AFFINE)]:
        assert int(re.search(rf"\b{name} = (\d+)", text).group(1)) == val, name
    for st in (0, -1, -2, -3, -4):
        assert fq.lib().fq_status_string(st) != b"unknown status"
    assert fq.lib().fq_status_string(7) == b"unknown status"


def test_host_sizes(fq):
    assert fq.fq_workspace_bytes(0) == 0
    assert fq.fq_workspace_bytes(1) == 16
    assert fq.fq_workspace_bytes(1 << 20) == 128 * 16  # one partial per 8192 elements
    assert fq.fq_workspace_bytes(1 << 40) == 16384 * 16
    assert fq.fq_q4dq_sizes(1) == (1, 1, 1)
    assert fq.fq_q4dq_sizes(200) == (100, 4, 1)
    assert fq.fq_q4dq_sizes(1 << 30) == (1 << 29, 1 << 24, 1 << 16)
    assert fq.fq_q4dq_sizes(16385) == (8193, 257, 2)
    with pytest.raises(fq.FqError):
        fq.fq_q4dq_sizes(0)


FAKE = 0x10000  # a non-null, well-aligned address that is never dereferenced


def status(fn, *args):
    return getattr(__import__("fake_quant_amd.fq", fromlist=["x"]).lib(), fn)(*args)


def test_argument_checks(fq):
    L = fq.lib()
    P = FAKE
    # unsupported widths / schemes / formats / dtypes
    for bits in (0, 3, 16):
        assert L.fq_quant_rows(P, 0, 4, 4, bits, 0, P, P, P, P, None, None) == fq.E_UNSUPPORTED
        assert L.fq_tensor_params_int(P, 8, bits, 0, P, 1 << 20, P, None, None) == fq.E_UNSUPPORTED
        assert L.fq_fake_quant_int_tensor(P, 8, bits, 0, P, P, P, None) == fq.E_UNSUPPORTED
        assert L.fq_dequantize_int_tensor(P, 8, bits, P, P, None) == fq.E_UNSUPPORTED
        assert L.fq_dequantize_rows(P, 2, 2, bits, P, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_quant_rows(P, 0, 4, 4, 8, 2, P, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_quant_rows(P, 2, 4, 4, 8, 0, P, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_fp8_quantize(P, 8, 2, P, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_fp8_dequantize(P, 8, -1, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_mxfp8_rows(P, 5, 1, 32, P, P, P, None) == fq.E_UNSUPPORTED
    # empty tensors and missing buffers
    assert L.fq_tensor_params_int(P, 0, 8, 0, P, 16, P, None, None) == fq.E_INVALID
    assert L.fq_tensor_params_int(None, 8, 8, 0, P, 16, P, None, None) == fq.E_INVALID
    assert L.fq_tensor_params_int(P, 8, 8, 0, P, 0, P, None, None) == fq.E_INVALID  # workspace too small
    assert L.fq_tensor_params_int(P + 4, 8, 8, 0, P + 4, 16, P, None, None) == fq.E_INVALID  # ws misaligned
    assert L.fq_fake_quant_int_tensor(P, 8, 8, 0, P, None, None, None) == fq.E_INVALID  # no output
    assert L.fq_fake_quant_int_tensor(P, 0, 8, 0, P, P, P, None) == fq.E_INVALID
    assert L.fq_quant_rows(P, 0, 0, 4, 8, 0, P, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_quant_rows(P, 0, 4, 0, 8, 0, P, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_quant_rows(P, 0, 4, 4, 8, 0, P, P, None, P, None, None) == fq.E_INVALID
    assert L.fq_quant_rows(P + 1, 0, 4, 4, 8, 0, P, P, P, P, None, None) == fq.E_INVALID  # misaligned f32
    assert L.fq_fp8_tensor_scale(P, 8, P, 1 << 20, None, None, None, None) == fq.E_INVALID
    # the workspace-free calibration + fake-quant: every argument error before any HIP call
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(P, 8, 3, 0, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(P, 8, 8, 2, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(P, 0, 8, 0, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(None, 8, 8, 0, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(P, 8, 8, 0, None, P, P, None, None) == fq.E_INVALID
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(P, 8, 8, 0, P, None, None, None, None) == fq.E_INVALID
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(P, 8, 8, 0, P + 2, P, P, None, None) == fq.E_INVALID
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(P + 1, 8, 8, 0, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(P, 8, 8, 0, P, P, P + 2, None, None) == fq.E_INVALID
    assert L.fq_calibrate_fake_quant_int_tensor_noalloc(P, 8, 8, 0, P, P, P, P + 1, None) == fq.E_INVALID
    assert L.fq_fp8_quantize(P, 8, 0, P, None, None, None) == fq.E_INVALID
    assert L.fq_fp8_quantize(P, 8, 0, None, P, P, None) == fq.E_INVALID
    assert L.fq_fp8_dequantize(P, 0, 0, P, P, None) == fq.E_INVALID
    assert L.fq_q4dq_quantize(P, 0, P, P, P, None, None, None, None) == fq.E_INVALID
    assert L.fq_q4dq_quantize(P, 8, None, P, P, None, None, None, None) == fq.E_INVALID
    assert L.fq_q4dq_dequantize(P, P, None, 8, P, None) == fq.E_INVALID
    assert L.fq_mxfp8_rows(P, 1, 1, 32, None, P, None, None) == fq.E_INVALID
    assert L.fq_mxfp8_rows(P, 1, 0, 32, P, P, None, None) == fq.E_INVALID
    # the one-call calibration + fake-quant checks the union of its two calls' arguments
    C = L.fq_calibrate_fake_quant_int_tensor
    assert C(P, 8, 3, 0, P, 1 << 20, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert C(P, 8, 8, 2, P, 1 << 20, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert C(P, 0, 8, 0, P, 1 << 20, P, P, P, None, None) == fq.E_INVALID  # empty
    assert C(None, 8, 8, 0, P, 1 << 20, P, P, P, None, None) == fq.E_INVALID
    assert C(P, 8, 8, 0, None, 1 << 20, P, P, P, None, None) == fq.E_INVALID  # no workspace
    assert C(P, 8, 8, 0, P, 0, P, P, P, None, None) == fq.E_INVALID  # workspace too small
    assert C(P, 8, 8, 0, P + 4, 1 << 20, P, P, P, None, None) == fq.E_INVALID  # workspace misaligned
    assert C(P, 8, 8, 0, P, 1 << 20, None, P, P, None, None) == fq.E_INVALID  # no params
    assert C(P, 8, 8, 0, P, 1 << 20, P, None, None, None, None) == fq.E_INVALID  # no output
    assert C(P + 1, 8, 8, 0, P, 1 << 20, P, P, P, None, None) == fq.E_INVALID  # misaligned f32
    assert C(P, 8, 8, 0, P, 1 << 20, P, P, P + 2, None, None) == fq.E_INVALID  # misaligned fq
    # stochastic rounding entry points share the checks of their nearest-rounding twins
    assert L.fq_fake_quant_int_tensor_sr(P, 8, 3, 0, P, 1, 0, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_fake_quant_int_tensor_sr(P, 8, 8, 2, P, 1, 0, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_fake_quant_int_tensor_sr(P, 0, 8, 0, P, 1, 0, P, P, None) == fq.E_INVALID
    assert L.fq_fake_quant_int_tensor_sr(P, 8, 8, 0, None, 1, 0, P, P, None) == fq.E_INVALID
    assert L.fq_fake_quant_int_tensor_sr(P, 8, 8, 0, P, 1, 0, None, None, None) == fq.E_INVALID
    assert L.fq_fp8_quantize_sr(P, 8, 2, P, 1, 0, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_fp8_quantize_sr(P, 8, 0, None, 1, 0, P, P, None) == fq.E_INVALID
    assert L.fq_fp8_quantize_sr(P, 8, 0, P, 1, 0, None, None, None) == fq.E_INVALID
    assert L.fq_fp8_quantize_sr(P + 2, 8, 0, P, 1, 0, P, P, None) == fq.E_INVALID
    # per-column calibration
    assert fq.fq_cols_workspace_bytes(0, 5) == 0
    assert fq.fq_cols_workspace_bytes(3, 5) == 4 * 5 * 16
    assert fq.fq_cols_workspace_bytes(4096, 4096) == 65 * 4096 * 16
    assert L.fq_quant_cols(P, 2, 4, 4, 8, 0, P, 1 << 20, P, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_quant_cols(P, 0, 4, 4, 5, 0, P, 1 << 20, P, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_quant_cols(P, 0, 0, 4, 8, 0, P, 1 << 20, P, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_quant_cols(P, 0, 4, 4, 8, 0, P, 16, P, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_quant_cols(P, 0, 4, 4, 8, 0, P, 1 << 20, P, P, None, P, None, None) == fq.E_INVALID
    # FP4 / FP6 block formats
    assert L.fq_mx_rows(P, 2, 4, 64, fq.E2M1, P, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_mx_rows(P, 0, 4, 64, 5, P, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_mx_rows(P, 0, 4, 64, fq.E5M2, P, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_mx_rows(P, 0, 0, 64, fq.E2M1, P, P, P, None) == fq.E_INVALID
    assert L.fq_mx_rows(P, 0, 4, 64, fq.E3M2, None, P, P, None) == fq.E_INVALID
    assert L.fq_mx_rows(P + 2, 0, 4, 64, fq.E2M3, P, P, P, None) == fq.E_INVALID
    ws16 = fq.fq_workspace_bytes(16)
    assert L.fq_nvfp4(P, 0, P, 1 << 20, P, P, P, P, None) == fq.E_INVALID
    assert L.fq_nvfp4(P, 16, P, 0, P, P, P, P, None) == fq.E_INVALID
    assert L.fq_nvfp4(P, 16, None, ws16, P, P, P, P, None) == fq.E_INVALID
    assert L.fq_nvfp4(P, 16, P, ws16, P, P, None, P, None) == fq.E_INVALID
    assert L.fq_nvfp4(P + 2, 16, P, ws16, P, P, P, P, None) == fq.E_INVALID
    # group-wise calibration
    assert L.fq_quant_groups(P, 2, 4, 64, 32, 8, 0, P, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_quant_groups(P, 0, 4, 64, 32, 5, 0, P, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_quant_groups(P, 0, 4, 64, 32, 8, 3, P, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_quant_groups(P, 0, 4, 64, 0, 8, 0, P, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_quant_groups(P, 0, 0, 64, 32, 8, 0, P, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_quant_groups(P, 0, 4, 64, 32, 8, 0, P, P, None, P, None, None) == fq.E_INVALID
    assert L.fq_quant_groups(P + 2, 0, 4, 64, 32, 8, 0, P, P, P, P, None, None) == fq.E_INVALID
    # percentile calibration: clip fraction in [0, 0.5), fixed workspace
    assert fq.fq_percentile_workspace_bytes(0) == 0
    wsp = fq.fq_percentile_workspace_bytes(8)
    assert wsp >= 3 * 2 * 2048 * 8 and wsp % 4 == 0
    assert fq.fq_percentile_workspace_bytes(1 << 24) >= wsp + 4 * (1 << 24) // 16
    assert L.fq_tensor_params_percentile(P, 8, 5, 0, 0.01, P, wsp, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_tensor_params_percentile(P, 8, 8, 2, 0.01, P, wsp, P, None, None) == fq.E_UNSUPPORTED
    for cf in (-0.01, 0.5, 0.7, float("nan"), float("inf")):
        assert L.fq_tensor_params_percentile(P, 8, 8, 0, cf, P, wsp, P, None, None) == fq.E_INVALID
    assert L.fq_tensor_params_percentile(P, 0, 8, 0, 0.01, P, wsp, P, None, None) == fq.E_INVALID
    assert L.fq_tensor_params_percentile(P, 8, 8, 0, 0.01, P, wsp - 1, P, None, None) == fq.E_INVALID
    assert L.fq_tensor_params_percentile(P, 8, 8, 0, 0.01, None, wsp, P, None, None) == fq.E_INVALID
    assert L.fq_tensor_params_percentile(P, 8, 8, 0, 0.01, P, wsp, None, None, None) == fq.E_INVALID
    assert L.fq_tensor_params_percentile(P + 2, 8, 8, 0, 0.01, P, wsp, P, None, None) == fq.E_INVALID
    # QAT step: configuration and step number checked on the host
    import ctypes
    cfg = fq.AdamWConfig(0.1, 0.9, 0.999, 1e-8, 0.0)
    bad = fq.AdamWConfig(0.1, 1.0, 0.999, 1e-8, 0.0)
    ws = 1 << 20
    assert L.fq_qat_step_int(P, P, P, P, 8, ctypes.byref(cfg), 1, 8, 0, 2, 0, 0, P, ws, P, P, P, None, None) == fq.E_UNSUPPORTED
    assert L.fq_qat_step_int(P, P, P, P, 8, ctypes.byref(cfg), 0, 8, 0, 0, 0, 0, P, ws, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_qat_step_int(P, P, P, P, 8, ctypes.byref(bad), 1, 8, 0, 0, 0, 0, P, ws, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_qat_step_int(P, P, P, P, 8, None, 1, 8, 0, 0, 0, 0, P, ws, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_qat_step_int(P, P, P, P, 8, ctypes.byref(cfg), 1, 8, 0, 0, 0, 0, P, ws, P, None, None, None, None) == fq.E_INVALID
    assert L.fq_qat_step_int(P, P, P, P, 8, ctypes.byref(cfg), 1, 8, 0, 0, 0, 0, P, 0, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_qat_step_fp8(P, P, P, P, 8, ctypes.byref(cfg), 1, 3, 0, 0, 0, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_qat_step_fp8(P, P, P, P, 8, ctypes.byref(cfg), 1, 0, 0, 0, 0, None, None, None) == fq.E_INVALID
    assert L.fq_qat_step_fp8(P, None, P, P, 8, ctypes.byref(cfg), 1, 0, 0, 0, 0, P, P, None) == fq.E_INVALID
    # empty inputs and missing buffers of the remaining entry points (no launch)
    assert L.fq_dequantize_int_tensor(P, 0, 8, P, P, None) == fq.E_INVALID
    assert L.fq_dequantize_int_tensor(P, 8, 6, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_dequantize_int_tensor(P, 8, 8, None, P, None) == fq.E_INVALID
    assert L.fq_dequantize_rows(P, 0, 4, 8, P, P, P, None) == fq.E_INVALID
    assert L.fq_dequantize_rows(P, 4, 0, 8, P, P, P, None) == fq.E_INVALID
    assert L.fq_dequantize_rows(P, 4, 4, 2, P, P, P, None) == fq.E_UNSUPPORTED
    assert L.fq_dequantize_rows(P, 4, 4, 8, P, None, P, None) == fq.E_INVALID
    assert L.fq_fp8_tensor_scale(P, 0, P, 1 << 20, P, P, None, None) == fq.E_INVALID
    assert L.fq_fp8_tensor_scale(P, 8, P, 1 << 20, None, None, None, None) == fq.E_INVALID
    assert L.fq_fp8_tensor_scale(P, 8, P, 0, P, P, None, None) == fq.E_INVALID
    assert L.fq_qat_step_int(P, P, P, P, 0, ctypes.byref(cfg), 1, 8, 0, 0, 0, 0, P, ws, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_qat_step_fp8(P, P, P, P, 0, ctypes.byref(cfg), 1, 0, 0, 0, 0, P, P, None) == fq.E_INVALID
    assert L.fq_quant_cols(P, 0, 4, 0, 8, 0, P, 1 << 20, P, P, P, P, None, None) == fq.E_INVALID
    assert L.fq_mx_rows(P, 0, 4, 0, fq.E2M1, P, P, P, None) == fq.E_INVALID
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    assert L.fq_q4dq_sizes(0, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == fq.E_INVALID
    # STE: length mismatch, empty
    assert L.fq_ste_backward(P, 3, P, 2, P, P, None) == fq.E_DIM
    assert L.fq_ste_backward(P, 0, P, 0, P, P, None) == fq.E_INVALID
    assert L.fq_ste_backward(None, 2, P, 2, P, P, None) == fq.E_INVALID


def test_binding_raises_on_error(fq):
    with pytest.raises(fq.FqError) as ei:
        fq.fq_ste_backward(FAKE, 3, FAKE, 2, FAKE, FAKE, stream=None)
    assert ei.value.status == fq.E_DIM


def test_oracle_and_product_share_no_code():
    """Neither side imports, includes or links the other."""
    prod = []
    for d, _, files in os.walk(os.path.join(ROOT, "fake_quant_amd")):
        prod += [os.path.join(d, f) for f in files if f.endswith((".py", ".hip", ".h"))]
    for p in prod:
        text = open(p).read()
        assert "oracle" not in re.findall(r"^\s*(?:from|import|#include)\s+\S*", text, flags=re.M).__str__(), p
        assert "liboracle" not in text and "orc_" not in text, p
    for p in ("oracle.c", "oracle.py"):
        text = open(os.path.join(ROOT, "oracle", p)).read()
        assert "fake_quant_amd" not in text and "libfq" not in text and "fq.h" not in text, p
        assert "fqk::" not in text and "fq_device" not in text, p


def test_library_imports_no_allocator(fq):
    """libfq.so never allocates, frees or clears device memory itself (callers own
    every buffer; the workspace-free entry point uses a static device array): no
    HIP allocator or memset routine is among its undefined dynamic symbols."""
    lib = os.path.join(ROOT, "fake_quant_amd", "libfq.so")
    res = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True)
    syms = [ln.split()[-1].split("@")[0] for ln in res.stdout.splitlines() if ln.strip()]
    assert "hipLaunchKernel" in syms
    bad = [s for s in syms if re.match(r"hip(Ext)?(Malloc|Free|HostAlloc|HostMalloc|MemAlloc|Memset|MallocAsync)", s)]
    assert bad == []
