"""Property-style GPU parity for the rows beyond the step, with drawn shapes,
magnitudes and options (as the drawn cases of the step's operations): per-column
and group-wise calibration, percentile calibration, MX FP4 / FP6 blocks and
NVFP4, each compared bit for bit with the oracle.  Derandomized so every run
draws the same cases."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from conftest import log
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=30, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])


def draw_array(n, log_mag, seed, specials):
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(4, n) * 10.0 ** log_mag).astype(np.float32)
    if specials and n > 8:
        idx = rng.choice(n, size=min(4, n // 4), replace=False)
        x[idx] = np.array([np.nan, np.inf, -np.inf, -0.0], np.float32)[: idx.size]
    return x


def to_dev(x, bf16):
    t = torch.from_numpy(x).cuda()
    return t.to(torch.bfloat16) if bf16 else t


def host(t):
    a = to_np(t)
    return (a.view(np.uint16), 1) if t.dtype == torch.bfloat16 else (a, 0)


@SETTINGS
@given(rows=st.integers(1, 70), cols=st.integers(1, 700), bits=st.sampled_from([4, 8]),
       scheme=st.sampled_from([0, 1]), bf16=st.booleans(), log_mag=st.floats(-20, 20),
       seed=st.integers(0, 2**31), specials=st.booleans())
def test_cols_drawn(fqlib, orc, rows, cols, bits, scheme, bf16, log_mag, seed, specials):
    log(f"hypothesis cols {rows}x{cols} bits={bits} scheme={scheme} bf16={bf16} seed={seed}")
    xt = to_dev(draw_array(rows * cols, log_mag, seed, specials).reshape(rows, cols), bf16)
    r = fqlib.quant_cols(xt, bits, scheme)
    torch.cuda.synchronize()
    xs, dt = host(xt)
    ref = orc.quant_cols(xs, bits, scheme, dtype=dt)
    assert_bits(to_np(r["codes"]), ref["codes"], "codes")
    assert_bits(to_np(r["scale"]), ref["scale"], "scale")
    assert_bits(to_np(r["zp"]), ref["zp"], "zp")
    assert_f32(to_np(r["fq"]), ref["fq"], "fq")
    assert int(r["flags"].item()) == ref["flags"]


@SETTINGS
@given(rows=st.integers(1, 20), ngroups=st.integers(1, 12), group=st.sampled_from([1, 3, 4, 8, 16, 24, 32, 64, 128, 256]),
       extra=st.sampled_from([0, 0, 0, 1, 5]), bits=st.sampled_from([4, 8]), scheme=st.sampled_from([0, 1]),
       bf16=st.booleans(), log_mag=st.floats(-20, 20), seed=st.integers(0, 2**31), specials=st.booleans())
def test_groups_drawn(fqlib, orc, rows, ngroups, group, extra, bits, scheme, bf16, log_mag, seed, specials):
    cols = ngroups * group + extra
    log(f"hypothesis groups {rows}x{cols} group={group} bits={bits} scheme={scheme} bf16={bf16} seed={seed}")
    xt = to_dev(draw_array(rows * cols, log_mag, seed, specials).reshape(rows, cols), bf16)
    r = fqlib.quant_groups(xt, group, bits, scheme)
    torch.cuda.synchronize()
    xs, dt = host(xt)
    ref = orc.quant_groups(xs, group, bits, scheme, dtype=dt)
    assert_bits(to_np(r["codes"]), ref["codes"], "codes")
    assert_bits(to_np(r["scale"]), ref["scale"], "scale")
    assert_bits(to_np(r["zp"]), ref["zp"], "zp")
    assert_f32(to_np(r["fq"]), ref["fq"], "fq")
    assert int(r["flags"].item()) == ref["flags"]


@SETTINGS
@given(n=st.integers(1, 200000), cf=st.sampled_from([0.0, 1e-4, 0.001, 0.01, 0.1, 0.3, 0.49]),
       bits=st.sampled_from([4, 8]), scheme=st.sampled_from([0, 1]), log_mag=st.floats(-20, 20),
       seed=st.integers(0, 2**31), specials=st.booleans(), levels=st.sampled_from([0, 0, 3, 50]))
def test_percentile_drawn(fqlib, orc, n, cf, bits, scheme, log_mag, seed, specials, levels):
    log(f"hypothesis percentile n={n} cf={cf} bits={bits} scheme={scheme} seed={seed} levels={levels}")
    x = draw_array(n, log_mag, seed, specials)
    if levels:  # heavy ties
        x = np.round(x / np.float32(10.0 ** log_mag) * levels).astype(np.float32) * np.float32(10.0 ** log_mag)
    params, flags = fqlib.params_percentile(torch.from_numpy(x).cuda(), cf, bits, scheme)
    torch.cuda.synchronize()
    ref = orc.percentile_params(x, bits, scheme, cf)
    s, zp, lo, hi = fqlib.params_fields(params)
    assert_bits(np.float32([s, lo, hi]), np.float32([ref["scale"], ref["lo"], ref["hi"]]), "params")
    assert zp == ref["zp"] and int(flags.item()) == ref["flags"]


@SETTINGS
@given(rows=st.integers(1, 30), cols=st.integers(1, 600), elem=st.sampled_from([2, 3, 4]), bf16=st.booleans(),
       log_mag=st.floats(-30, 30), seed=st.integers(0, 2**31), specials=st.booleans())
def test_mx_drawn(fqlib, orc, rows, cols, elem, bf16, log_mag, seed, specials):
    log(f"hypothesis mx {rows}x{cols} elem={elem} bf16={bf16} seed={seed}")
    xt = to_dev(draw_array(rows * cols, log_mag, seed, specials).reshape(rows, cols), bf16)
    r = fqlib.mx_rows(xt, elem)
    torch.cuda.synchronize()
    xs, dt = host(xt)
    ref = orc.mx_rows(xs, elem, dtype=dt)
    assert_bits(to_np(r["q"]), ref["q"], "codes")
    assert_bits(to_np(r["e8m0"]), ref["e8m0"], "e8m0")
    assert_f32(to_np(r["fq"]), ref["fq"], "fq")


@SETTINGS
@given(n=st.integers(1, 100000), log_mag=st.floats(-35, 35), seed=st.integers(0, 2**31), specials=st.booleans())
def test_nvfp4_drawn(fqlib, orc, n, log_mag, seed, specials):
    log(f"hypothesis nvfp4 n={n} log_mag={log_mag:.2f} seed={seed} specials={specials}")
    x = draw_array(n, log_mag, seed, specials)
    r = fqlib.nvfp4(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    ref = orc.nvfp4(x)
    assert_bits(to_np(r["g"]), np.float32([ref["g"]]), "tensor scale")
    assert_bits(to_np(r["scales"]), ref["sbytes"], "block scales")
    assert_bits(to_np(r["q"]), ref["q"], "codes")
    assert_f32(to_np(r["fq"]), ref["fq"], "fq")


@SETTINGS
@given(n=st.integers(1, 300000), bits=st.sampled_from([4, 8]), scheme=st.sampled_from([0, 1]),
       rounding=st.sampled_from([0, 0, 1]), wd=st.sampled_from([0.0, 0.01]), off=st.sampled_from([0, 0, 1, 3]),
       log_mag=st.floats(-6, 3), seed=st.integers(0, 2**31))
def test_qat_int_drawn(fqlib, orc, n, bits, scheme, rounding, wd, off, log_mag, seed):
    # the integer QAT step over two steps: nearest rounding on aligned buffers
    # takes the two-launch form (the requantize folds the update's partials),
    # stochastic rounding or a misaligned view (off > 0) the three-launch one
    log(f"qat drawn n={n} bits={bits} scheme={scheme} rounding={rounding} wd={wd} off={off}")
    rng = np.random.default_rng(seed)
    w0 = (rng.standard_normal(n) * 10.0 ** log_mag).astype(np.float32)
    grads = [rng.standard_normal(n).astype(np.float32) for _ in range(2)]
    lr = 1e-2
    cfg = fqlib.adamw_config(lr, weight_decay=wd)
    wb = torch.zeros(n + off, device="cuda")
    mb = torch.zeros(n + off, device="cuda")
    vb = torch.zeros(n + off, device="cuda")
    w, m, v = wb[off:], mb[off:], vb[off:]
    w.copy_(torch.from_numpy(w0))
    ow, om, ov = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t, g in enumerate(grads, start=1):
        r = fqlib.qat_step_int(w, torch.from_numpy(g).cuda(), m, v, t, cfg, bits, scheme, rounding, seed, 5)
        torch.cuda.synchronize()
        ref = orc.qat_step_int(ow, g, om, ov, lr, t, bits=bits, scheme=scheme, rounding=rounding, seed=seed,
                               offset=5, weight_decay=wd)
        ow, om, ov = ref["w"], ref["m"], ref["v"]
        assert_f32(to_np(w), ow, f"master step {t}")
        assert_f32(to_np(m), om, f"m step {t}")
        assert_f32(to_np(v), ov, f"v step {t}")
        s, zp, lo, hi = fqlib.params_fields(r["params"])
        assert_bits(np.float32([s, lo, hi]), np.float32([ref["scale"], ref["lo"], ref["hi"]]), f"params step {t}")
        assert zp == ref["zp"]
        codes = to_np(r["codes"])
        if bits == 4:
            p = codes.astype(np.uint8)
            hi4 = (p >> 4).astype(np.int16)
            lo4 = (p & 0xF).astype(np.int16)
            un = np.empty(2 * p.size, np.int16)
            un[0::2] = np.where(hi4 >= 8, hi4 - 16, hi4)
            un[1::2] = np.where(lo4 >= 8, lo4 - 16, lo4)
            codes = un[:n].astype(np.int8)
        else:
            codes = codes.view(np.int8)
        assert_bits(codes, ref["codes"], f"codes step {t}")
        assert_f32(to_np(r["view"]), ref["view"], f"view step {t}")
        assert int(r["flags"].item()) == ref["flags"]
