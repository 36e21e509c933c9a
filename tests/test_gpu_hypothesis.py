"""Property-style GPU parity with drawn sizes, after the proptests of the [DQ]
page (100 cases each, drawn lengths and magnitudes): random lengths, magnitudes,
row shapes, offsets and formats, each compared bit for bit with the oracle.
Derandomized so every run draws the same cases."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from conftest import log
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])


def draw_array(n, log_mag, seed, specials):
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(4, n) * 10.0 ** log_mag).astype(np.float32)
    if specials and n > 8:
        idx = rng.choice(n, size=min(4, n // 4), replace=False)
        x[idx] = np.array([np.nan, np.inf, -np.inf, -0.0], np.float32)[: idx.size]
    return x


@SETTINGS
@given(n=st.integers(1, 3 * 16384 + 77), log_mag=st.floats(-30, 30), seed=st.integers(0, 2**31),
       specials=st.booleans())
def test_q4dq_drawn(fqlib, orc, n, log_mag, seed, specials):
    log(f"hypothesis q4dq n={n} log_mag={log_mag:.2f} seed={seed} specials={specials}")
    x = draw_array(n, log_mag, seed, specials)
    r = fqlib.q4dq_quantize(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    ref = orc.q4dq_quantize(x)
    assert_bits(to_np(r["packed"]), ref["packed"], "packed")
    assert_bits(to_np(r["qscale"]), ref["qscale"], "qscale")
    assert_bits(to_np(r["super"]), ref["super"], "super")
    assert_f32(to_np(r["recon"]), ref["recon"], "recon")


@SETTINGS
@given(rows=st.integers(1, 9), cols=st.integers(1, 9000), bits=st.sampled_from([4, 8]),
       scheme=st.sampled_from([0, 1]), bf16=st.booleans(), log_mag=st.floats(-20, 20),
       seed=st.integers(0, 2**31), specials=st.booleans())
def test_rows_drawn(fqlib, orc, rows, cols, bits, scheme, bf16, log_mag, seed, specials):
    log(f"hypothesis rows {rows}x{cols} bits={bits} scheme={scheme} bf16={bf16} seed={seed}")
    x = draw_array(rows * cols, log_mag, seed, specials).reshape(rows, cols)
    xt = torch.from_numpy(x).cuda()
    if bf16:
        xt = xt.to(torch.bfloat16)
    r = fqlib.quant_rows(xt, bits, scheme)
    torch.cuda.synchronize()
    xs = to_np(xt)
    ref = orc.quant_rows(xs.view(np.uint16) if bf16 else xs, bits, scheme, dtype=1 if bf16 else 0)
    assert_bits(to_np(r["codes"]), ref["codes"], "codes")
    assert_bits(to_np(r["scale"]), ref["scale"], "scale")
    assert_bits(to_np(r["zp"]), ref["zp"], "zp")
    assert_f32(to_np(r["fq"]), ref["fq"], "fq")


@SETTINGS
@given(n=st.integers(1, 70000), fmt=st.sampled_from([0, 1]), log_scale=st.floats(-30, 30),
       seed=st.integers(0, 2**31), offset=st.integers(0, 2**40), sr=st.booleans())
def test_fp8_drawn(fqlib, orc, n, fmt, log_scale, seed, offset, sr):
    log(f"hypothesis fp8 n={n} fmt={fmt} log_scale={log_scale:.2f} seed={seed} sr={sr} offset={offset}")
    x = draw_array(n, log_scale, seed, True)
    scale = np.float32(10.0 ** log_scale / 7.0)
    xt = torch.from_numpy(x).cuda()
    stt = torch.tensor([scale], device="cuda")
    if sr:
        q, fqv = fqlib.fp8_quantize_sr(xt, fmt, stt, seed, offset)
        rq, rf = orc.fp8_quantize_sr(x, fmt, float(scale), seed, offset)
    else:
        q, fqv = fqlib.fp8_quantize(xt, fmt, stt)
        rq, rf = orc.fp8_quantize(x, fmt, float(scale))
    torch.cuda.synchronize()
    assert_bits(to_np(q), rq, "bytes")
    assert_f32(to_np(fqv), rf, "fq")


@SETTINGS
@given(rows=st.integers(1, 6), cols=st.integers(1, 3000), bf16=st.booleans(), log_mag=st.floats(-30, 30),
       seed=st.integers(0, 2**31))
def test_mx_drawn(fqlib, orc, rows, cols, bf16, log_mag, seed):
    log(f"hypothesis mx {rows}x{cols} bf16={bf16} seed={seed}")
    x = draw_array(rows * cols, log_mag, seed, True).reshape(rows, cols)
    xt = torch.from_numpy(x).cuda()
    if bf16:
        xt = xt.to(torch.bfloat16)
    r = fqlib.mxfp8_rows(xt)
    q, e8, fqv = r["q"], r["e8m0"], r["fq"]
    torch.cuda.synchronize()
    xs = to_np(xt)
    ref = orc.mxfp8_rows(xs.view(np.uint16) if bf16 else xs, dtype=1 if bf16 else 0)
    assert_bits(to_np(q), ref["q"], "q")
    assert_bits(to_np(e8), ref["e8m0"], "e8m0")
    assert_f32(to_np(fqv), ref["fq"], "fq")


@SETTINGS
@given(n=st.integers(1, 200000), bits=st.sampled_from([4, 8]), scheme=st.sampled_from([0, 1]),
       log_mag=st.floats(-30, 30), seed=st.integers(0, 2**31), specials=st.booleans(),
       offset=st.integers(0, 3))
def test_tensor_one_call_drawn(fqlib, orc, n, bits, scheme, log_mag, seed, specials, offset):
    """Per-tensor calibration + fake-quant in one call (the two-launch fold path for
    aligned buffers, the two calls for offset views) against the oracle."""
    log(f"hypothesis tensor one-call n={n} bits={bits} scheme={scheme} seed={seed} offset={offset}")
    x = draw_array(n, log_mag, seed, specials)
    buf = torch.zeros(n + 4, dtype=torch.float32, device="cuda")
    buf[offset:offset + n] = torch.from_numpy(x).cuda()
    xt = buf[offset:offset + n]
    params, codes, fqv, flags = fqlib.calibrate_fake_quant_int_tensor(xt, bits, scheme)
    torch.cuda.synchronize()
    ref = orc.tensor_params_int(x, bits, scheme)
    rc, rf = orc.fake_quant_int(x, bits, scheme, float(ref["scale"]), ref["zp"])
    s, zp, lo, hi = fqlib.params_fields(params)
    assert_bits(np.float32([s, lo, hi]), np.float32([ref["scale"], ref["lo"], ref["hi"]]), "params")
    assert zp == ref["zp"]
    assert int(flags.item()) == ref["flags"]
    c = to_np(codes)
    if bits == 4:
        p = c.astype(np.uint8)
        hi_n, lo_n = (p >> 4).astype(np.int16), (p & 0xF).astype(np.int16)
        u = np.empty(2 * p.size, np.int16)
        u[0::2], u[1::2] = hi_n, lo_n
        c = np.where(u >= 8, u - 16, u)[:n]
    assert_bits(c.astype(np.int8), rc, "codes")
    assert_f32(to_np(fqv), rf, "fq")
