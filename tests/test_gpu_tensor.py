"""GPU parity of the per-tensor path against the oracle: tensor-scope calibration,
integer quantize / fake-quant / dequantize, STE backward.

Workload: 2^20 float32 ~ N(0, 1) with an N(0, 1) upstream gradient, symmetric
int8 (the configured case) plus affine and int4, and ragged / unaligned / special
inputs.  Bars: codes bit-exact, params bit-exact, float outputs <= 1 ulp.
"""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu


def unpack_nibbles(packed, n):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(2 * p.size, np.int8)
    hi = (p >> 4).astype(np.int16)
    lo = (p & 0xF).astype(np.int16)
    out[0::2] = np.where(hi >= 8, hi - 16, hi)
    out[1::2] = np.where(lo >= 8, lo - 16, lo)
    return out[:n]


def check_tensor(fq, orc, x_t, bits, scheme, g_t=None, what=""):
    log(f"tensor case {what} n={x_t.numel()} bits={bits} scheme={scheme}")
    n = x_t.numel()
    x = to_np(x_t)
    params, flags = fq.params_int(x_t, bits, scheme)
    codes, fqv = fq.fake_quant_int_tensor(x_t, params, bits, scheme)
    deq = fq.dequantize_int_tensor(codes, n, params, bits)
    torch.cuda.synchronize()
    s, zp, lo, hi = fq.params_fields(params)
    ref = orc.tensor_params_int(x, bits, scheme)
    assert_bits(np.float32([s, lo, hi]), np.float32([ref["scale"], ref["lo"], ref["hi"]]), what + " params")
    assert zp == ref["zp"], what
    assert int(flags.item()) == ref["flags"], what
    rc, rf = orc.fake_quant_int(x, bits, scheme, float(ref["scale"]), ref["zp"])
    got_codes = to_np(codes) if bits == 8 else unpack_nibbles(to_np(codes), n)
    assert_bits(got_codes.astype(np.int8), rc, what + " codes")
    if bits == 4 and n % 2:
        assert to_np(codes)[-1] & 0xF == 0, what + " pad nibble"
    assert_f32(to_np(fqv), rf, what + " fq")
    assert_f32(to_np(deq), orc.dequantize_int(rc, float(ref["scale"]), ref["zp"]), what + " dequant")
    check_calibrate_fake_quant(fq, x_t, bits, scheme, ref, rc, rf, what)
    if g_t is not None:
        bounds = params.view(torch.float32)[2:4]
        gi = fq.ste_backward(g_t, x_t, bounds)
        rev = torch.flip(bounds, [0]).contiguous()
        gi2 = fq.ste_backward(g_t, x_t, rev)
        torch.cuda.synchronize()
        want = orc.ste_backward(to_np(g_t), x, float(ref["lo"]), float(ref["hi"]))
        assert_bits(to_np(gi), want, what + " ste")
        assert_bits(to_np(gi2), want, what + " ste reversed bounds")


def check_calibrate_fake_quant(fq, x_t, bits, scheme, ref, rc, rf, what):
    """The one-call calibration + fake-quant against the oracle's two steps."""
    n = x_t.numel()
    params, codes, fqv, flags = fq.calibrate_fake_quant_int_tensor(x_t, bits, scheme)
    torch.cuda.synchronize()
    s, zp, lo, hi = fq.params_fields(params)
    assert_bits(np.float32([s, lo, hi]), np.float32([ref["scale"], ref["lo"], ref["hi"]]), what + " one-call params")
    assert zp == ref["zp"], what + " one-call zp"
    assert int(flags.item()) == ref["flags"], what + " one-call flags"
    got_codes = to_np(codes) if bits == 8 else unpack_nibbles(to_np(codes), n)
    assert_bits(got_codes.astype(np.int8), rc, what + " one-call codes")
    if bits == 4 and n % 2:
        assert to_np(codes)[-1] & 0xF == 0, what + " one-call pad nibble"
    assert_f32(to_np(fqv), rf, what + " one-call fq")


@pytest.mark.parametrize("n", [(1 << 22) - 5, 1 << 22, (1 << 22) + 4, (1 << 22) + 8197])
def test_one_call_fold_boundary(fqlib, orc, n):
    """Around the largest tensor whose fake-quant blocks fold the reduction
    partials themselves (512 partials of 8192 elements): that path at and below
    it, the two-call sequence above."""
    x, _ = synthetic.tensor_inputs(n=n, device="cuda", seed=n % 1000)
    xn = to_np(x)
    for bits, scheme in [(8, 0), (4, 1)]:
        log(f"one-call boundary n={n} bits={bits} scheme={scheme}")
        ref = orc.tensor_params_int(xn, bits, scheme)
        rc, rf = orc.fake_quant_int(xn, bits, scheme, float(ref["scale"]), ref["zp"])
        check_calibrate_fake_quant(fqlib, x, bits, scheme, ref, rc, rf, f"boundary {n}")


@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 0), (4, 1)])
def test_full_size_workload(fqlib, orc, bits, scheme):
    x, g = synthetic.tensor_inputs(device="cuda")
    check_tensor(fqlib, orc, x, bits, scheme, g, what="N(0,1) 2^20")


@pytest.mark.parametrize("n", [1, 2, 3, 5, 7, 1023, 1025, 4097, 65537, 262147])
def test_ragged_sizes(fqlib, orc, n):
    x, g = synthetic.tensor_inputs(n=n, device="cuda", seed=n)
    for bits, scheme in [(8, 0), (4, 1)]:
        check_tensor(fqlib, orc, x, bits, scheme, g, what=f"ragged {n}")


def test_unaligned_views(fqlib, orc):
    buf, gbuf = synthetic.tensor_inputs(n=70001, device="cuda", seed=3)
    for off in (1, 2, 3):
        x = buf[off:off + 65536 + off]
        g = gbuf[off:off + 65536 + off]
        for bits, scheme in [(8, 1), (4, 0)]:
            check_tensor(fqlib, orc, x, bits, scheme, g, what=f"offset {off}")


def special_inputs():
    rng = np.random.default_rng(9)
    cases = {
        "zeros": np.zeros(1000, np.float32),
        "neg_zero": np.full(33, -0.0, np.float32),
        "nonfinite": np.concatenate([rng.standard_normal(500), [np.inf, -np.inf, np.nan] * 3]).astype(np.float32),
        "all_nan": np.full(17, np.nan, np.float32),
        "tiny": (rng.standard_normal(4099) * 1e-30).astype(np.float32),
        "denormal": (rng.standard_normal(999) * 1e-41).astype(np.float32),
        "huge": (rng.standard_normal(4096) * 1e37).astype(np.float32),
        "positive": np.abs(rng.standard_normal(5000)).astype(np.float32) + 3.0,
        "negative": -np.abs(rng.standard_normal(5000)).astype(np.float32) - 0.5,
        "single": np.array([-2.5], np.float32),
        "ties": (np.arange(-300, 300) + 0.5).astype(np.float32) / np.float32(127),
    }
    return cases


@pytest.mark.parametrize("name", list(special_inputs()))
def test_special_values(fqlib, orc, name):
    x = torch.from_numpy(special_inputs()[name]).cuda()
    g = torch.ones_like(x)
    for bits in (8, 4):
        for scheme in (0, 1):
            check_tensor(fqlib, orc, x, bits, scheme, g, what=name)


def test_given_params_extremes(fqlib, orc):
    """Quantize with caller-given parameters: tiny and huge scales (the exact
    division's fallback path), zero scale, and a zero-point at the range end."""
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-40, 39, 4000),
                        [np.inf, -np.inf, np.nan, 0.0, -0.0, 3e38, -3e38, 1e-45]]).astype(np.float32)
    xt = torch.from_numpy(x).cuda()
    for scale, zp in [(1e-30, 0), (3e-19, 5), (7e18, -3), (0.0, 0), (1.0, -128), (2.5e-39, 0), (1e25, 7),
                      (1.8e-18, 0), (5e17, 2), (0.1, 3)]:
        for bits, scheme in [(8, 0), (8, 1), (4, 1)]:
            qmin, qmax = orc.q_range(bits, scheme)
            zz = min(max(zp, qmin), qmax) if scheme == 1 else 0
            p = torch.tensor([0, zz, 0, 0], dtype=torch.int32)
            p.view(torch.float32)[0] = scale
            p = p.cuda()
            codes, fqv = fqlib.fake_quant_int_tensor(xt, p, bits, scheme)
            torch.cuda.synchronize()
            rc, rf = orc.fake_quant_int(x, bits, scheme, float(np.float32(scale)), zz)
            got = to_np(codes) if bits == 8 else unpack_nibbles(to_np(codes), x.size)
            assert_bits(got.astype(np.int8), rc, f"given scale {scale} zp {zz} bits {bits}")
            assert_f32(to_np(fqv), rf, f"given scale {scale} fq")


def test_deterministic(fqlib):
    x, g = synthetic.tensor_inputs(device="cuda")
    outs = []
    for _ in range(2):
        params, _ = fqlib.params_int(x, 8, 1)
        codes, fqv = fqlib.fake_quant_int_tensor(x, params, 8, 1)
        outs.append((params.clone(), codes.clone(), fqv.clone()))
    for _ in range(2):
        params, codes, fqv, _ = fqlib.calibrate_fake_quant_int_tensor(x, 8, 1)
        outs.append((params.clone(), codes.clone(), fqv.clone()))
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
