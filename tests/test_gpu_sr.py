"""GPU parity of stochastic rounding ([QAT] RoundingMode::Stochastic) against the
oracle: per-tensor integer fake-quant and per-tensor fp8 quantize, bit-exact codes
and bytes, fake-quant values within the float bar, for ragged sizes, offsets into
the Philox stream (multiples of four and not), unaligned views, special values and
both quotient paths (exact fast quotient and true division).  A tensor quantized
in two calls with matching offsets equals one call.
"""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu

SEED = 0x5EED_0F_C0FFEE
OFFSETS = [0, 1, 2, 3, 4, (1 << 33) + 6]


def params_tensor(scale, zp):
    p = torch.tensor([0, zp, 0, 0], dtype=torch.int32)
    p.view(torch.float32)[0] = float(np.float32(scale))
    return p.cuda()


def check_int(fq, orc, x_t, bits, scheme, scale, zp, seed, offset, what):
    log(f"sr int case {what} n={x_t.numel()} bits={bits} scheme={scheme} offset={offset}")
    codes, fqv = fq.fake_quant_int_tensor_sr(x_t, params_tensor(scale, zp), seed, offset, bits, scheme)
    torch.cuda.synchronize()
    x = to_np(x_t)
    rc, rf = orc.fake_quant_int_sr(x, bits, scheme, float(scale), zp, seed, offset)
    if bits == 4:
        n = x.size
        pk = np.zeros((n + 1) // 2, np.uint8)
        nib = (rc.astype(np.int16) & 0xF).astype(np.uint8)
        pk[:] = nib[0::2] << 4
        pk[: n // 2] |= nib[1::2]
        rc = pk
    assert_bits(to_np(codes).view(np.uint8), rc.view(np.uint8), what + " codes")
    assert_f32(to_np(fqv), rf, what + " fq")


def check_fp8(fq, orc, x_t, fmt, scale, seed, offset, what):
    log(f"sr fp8 case {what} n={x_t.numel()} fmt={fmt} offset={offset}")
    st = torch.tensor([float(np.float32(scale))], dtype=torch.float32, device="cuda")
    q, fqv = fq.fp8_quantize_sr(x_t, fmt, st, seed, offset)
    torch.cuda.synchronize()
    rq, rf = orc.fp8_quantize_sr(to_np(x_t), fmt, float(scale), seed, offset)
    assert_bits(to_np(q), rq, what + " bytes")
    assert_f32(to_np(fqv), rf, what + " fq")


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1000, 4099, (1 << 20) + 3])
@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 0), (4, 1)])
def test_int_sizes(fqlib, orc, n, bits, scheme):
    x_t, _ = synthetic.tensor_inputs(n, device="cuda", seed=n)
    ref = orc.tensor_params_int(to_np(x_t), bits, scheme)
    check_int(fqlib, orc, x_t, bits, scheme, ref["scale"], ref["zp"], SEED, 0, f"n={n}")


@pytest.mark.parametrize("offset", OFFSETS)
def test_int_offsets_and_split(fqlib, orc, offset):
    n = 10_007
    x_t, _ = synthetic.tensor_inputs(n, device="cuda", seed=5)
    ref = orc.tensor_params_int(to_np(x_t), 8, 1)
    check_int(fqlib, orc, x_t, 8, 1, ref["scale"], ref["zp"], SEED, offset, f"offset {offset}")
    # the same tensor in two calls (split at a non-multiple of four) equals one call
    p = params_tensor(ref["scale"], ref["zp"])
    whole_c, whole_f = fqlib.fake_quant_int_tensor_sr(x_t, p, SEED, offset, 8, 1)
    k = 4_999
    a_c, a_f = fqlib.fake_quant_int_tensor_sr(x_t[:k].contiguous(), p, SEED, offset, 8, 1)
    b_c, b_f = fqlib.fake_quant_int_tensor_sr(x_t[k:].contiguous(), p, SEED, offset + k, 8, 1)
    torch.cuda.synchronize()
    assert torch.equal(whole_c, torch.cat([a_c, b_c]))
    assert torch.equal(whole_f.view(torch.int32), torch.cat([a_f, b_f]).view(torch.int32))


def test_int_specials_and_division_paths(fqlib, orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(4097).astype(np.float32)
    x[:8] = [np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-45, -1e30, 1e30]
    xt = torch.from_numpy(x).cuda()
    for bits, scheme in ((8, 0), (8, 1), (4, 1)):
        for scale, zp in ((0.013, 0), (0.02, -7 if bits == 4 else -100), (0.0, 0), (1e-30, 0), (3e22, 1)):
            if bits == 4 and zp < -8:
                zp = -3
            check_int(fqlib, orc, xt, bits, scheme, scale, zp, 77, 3, f"specials scale={scale} zp={zp}")
    # unaligned view
    buf = torch.from_numpy(rng.standard_normal(3000).astype(np.float32)).cuda()
    check_int(fqlib, orc, buf[1:2001], 8, 0, 0.01, 0, 11, 0, "unaligned")


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_workload(fqlib, orc, fmt):
    n = 1 << 22
    x_t = synthetic.fp8_inputs(n, device="cuda")
    s, _ = orc.fp8_scale(float(orc.amax_finite(to_np(x_t))), fmt)
    check_fp8(fqlib, orc, x_t, fmt, s, SEED, 0, "fp8 workload")


@pytest.mark.parametrize("offset", OFFSETS)
@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_ragged_offsets(fqlib, orc, fmt, offset):
    for n in (1, 2, 7, 1025):
        x_t = synthetic.fp8_inputs(n, device="cuda", seed=n)
        check_fp8(fqlib, orc, x_t, fmt, 1.0 if n < 8 else 0.37, SEED + n, offset, f"n={n}")


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_specials(fqlib, orc, fmt):
    maxv = 448.0 if fmt == 0 else 57344.0
    base = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-40, -1e-40, maxv, -maxv, maxv * 1.04, 1e30,
                     1.0625, -1.0625, 2.0 ** -9, 2.0 ** -10, 3.0 * 2.0 ** -17, 0.3, -0.7], np.float32)
    x = np.tile(base, 300)
    xt = torch.from_numpy(x).cuda()
    for scale in (1.0, 0.0, 1e-30, 2.5e-39, 7e18):
        check_fp8(fqlib, orc, xt, fmt, scale, 123, 1, f"specials scale={scale}")
    buf = torch.from_numpy(np.tile(base, 40)).cuda()
    check_fp8(fqlib, orc, buf[3:603], fmt, 1.0, 5, 0, "unaligned")


def test_deterministic(fqlib):
    x_t = synthetic.fp8_inputs(1 << 20, device="cuda")
    st = torch.tensor([0.5], device="cuda")
    a, af = fqlib.fp8_quantize_sr(x_t, 0, st, 9, 0)
    b, bf = fqlib.fp8_quantize_sr(x_t, 0, st, 9, 0)
    c, _ = fqlib.fp8_quantize_sr(x_t, 0, st, 10, 0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(af.view(torch.int32), bf.view(torch.int32))
    assert not torch.equal(a, c), "a different seed draws different numbers"
