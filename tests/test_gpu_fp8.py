"""GPU parity of the per-tensor fp8 path against the oracle: finite-amax scale,
saturating E4M3 / E5M2 quantize + fake-quant, dequantize.

Workload: 2^26 float32 sign * 2^U(-20, 20) with 0.1 % each of +-Inf, NaN and
zeros (full size, every element compared), plus ragged / unaligned / special
inputs and a sweep of every fp32 exponent and rounding boundary.
"""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu


def check_fp8(fq, orc, x_t, what="", full=True):
    n = x_t.numel()
    log(f"fp8 case {what} n={n}")
    x = to_np(x_t)
    s_t, flags = fq.fp8_tensor_scale(x_t)
    torch.cuda.synchronize()
    amax = orc.amax_finite(x)
    for fmt in (0, 1):
        s_ref, f_ref = orc.fp8_scale(float(amax), fmt)
        s_gpu = s_t[fmt:fmt + 1]
        assert_bits(to_np(s_gpu), np.float32([s_ref]), f"{what} scale fmt{fmt}")
        if s_ref == 0:
            assert int(flags.item()) & 2
        q, fqv = fq.fp8_quantize(x_t, fmt, s_gpu)
        deq = fq.fp8_dequantize(q, fmt, s_gpu)
        torch.cuda.synchronize()
        rq, rf = orc.fp8_quantize(x, fmt, float(s_ref))
        assert_bits(to_np(q), rq, f"{what} bytes fmt{fmt}")
        assert_f32(to_np(fqv), rf, f"{what} fq fmt{fmt}")
        assert_f32(to_np(deq), orc.fp8_dequantize(rq, fmt, float(s_ref)), f"{what} dequant fmt{fmt}")


def test_full_size_workload(fqlib, orc):
    x = synthetic.fp8_inputs(device="cuda")
    check_fp8(fqlib, orc, x, what="log-uniform 2^26")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 1023, 1025, 65537, 100003])
def test_ragged_sizes(fqlib, orc, n):
    x = synthetic.fp8_inputs(n=n, device="cuda", seed=n, special_frac=0.01)
    check_fp8(fqlib, orc, x, what=f"ragged {n}")


def test_unaligned(fqlib, orc):
    buf = synthetic.fp8_inputs(n=70003, device="cuda", seed=8, special_frac=0.01)
    for off in (1, 2, 3):
        check_fp8(fqlib, orc, buf[off:off + 65536], what=f"offset {off}")


def test_zero_scale(fqlib, orc):
    x = torch.tensor([0.0, -0.0, float("nan"), float("inf"), -float("inf"), 0.0], device="cuda")
    check_fp8(fqlib, orc, x, what="no finite magnitude")


def boundary_sweep():
    """Every binary32 exponent with rounding-boundary mantissas of both formats."""
    lows = []
    for mb in (2, 3):
        half, full = 1 << (22 - mb), 1 << (23 - mb)
        lows += [0, 1, half - 1, half, half + 1, full - 1]
    lows = np.array(sorted(set(lows)), np.uint32)
    tops = np.arange(16, dtype=np.uint32) << 19
    exps = np.arange(0, 256, dtype=np.uint32)
    e, t, l = np.meshgrid(exps, tops, lows, indexing="ij")
    bits = ((e << 23) | t | l).ravel()
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 1e-3, 1e-30, 2e20, 7.1e-41, 448.0])
def test_boundary_sweep_given_scale(fqlib, orc, scale):
    y = boundary_sweep()
    yt = torch.from_numpy(y).cuda()
    s = np.float32(scale)
    st = torch.tensor([s], device="cuda")
    for fmt in (0, 1):
        log(f"fp8 boundary sweep scale={scale} fmt={fmt}")
        q, fqv = fqlib.fp8_quantize(yt, fmt, st)
        torch.cuda.synchronize()
        rq, rf = orc.fp8_quantize(y, fmt, float(s))
        assert_bits(to_np(q), rq, f"sweep bytes scale {scale} fmt {fmt}")
        assert_f32(to_np(fqv), rf, f"sweep fq scale {scale} fmt {fmt}")


def test_dequantize_all_codes(fqlib, orc):
    codes = np.tile(np.arange(256, dtype=np.uint8), 5)
    ct = torch.from_numpy(codes).cuda()
    for scale in (1.0, 0.0, 3.5, 1e30, 2.0 ** -140):
        st = torch.tensor([np.float32(scale)], device="cuda")
        for fmt in (0, 1):
            out = fqlib.fp8_dequantize(ct, fmt, st)
            torch.cuda.synchronize()
            assert_f32(to_np(out), orc.fp8_dequantize(codes, fmt, float(np.float32(scale))),
                       f"dequant codes scale {scale} fmt {fmt}")


def test_deterministic(fqlib):
    x = synthetic.fp8_inputs(n=1 << 22, device="cuda")
    s, _ = fqlib.fp8_tensor_scale(x)
    a = fqlib.fp8_quantize(x, 0, s[0:1])
    b = fqlib.fp8_quantize(x, 0, s[0:1])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
