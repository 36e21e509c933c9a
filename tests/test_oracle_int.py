"""Pins of the oracle's integer grid, per-row calibration and STE backward.

Page: optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs ("Quantization-Aware
Training (QAT) primitives"): module docs "Integer quantization (int8 / int4)",
IntDtype::q_range, QuantParams::{from_minmax, from_absmax}, fake_quant_int,
per_channel_params, fake_quant_backward and the unit tests whose values sit in
tests/golden/qat_int_examples.txt.

Independent checks used (none re-types the oracle's own expression):
* the page's worked values and round trips;
* brute force over every code: the chosen code minimises |fl(x/s) - (q - zp)| with
  ties to even, then clamps (numpy does the binary32 division);
* the page's invariants: error <= scale/2, the zero-point cancels in the round
  trip, restricted symmetric codes never reach -128 / -8, the nudged affine
  window contains 0 exactly and covers [min, max];
* a numpy vectorised second implementation of the page's "integer pipeline" for the
  SQNR-per-bit property (about 6 dB per bit).
"""
import math

import numpy as np
import pytest

from conftest import read_golden_kv

G = read_golden_kv("qat_int_examples.txt")
SYM, AFFINE = 0, 1


def floats(s):
    return [float(v) for v in s.split(",")]


def f32(v):
    return float(np.float32(v))


def test_q_range_table(orc):
    assert orc.q_range(8, SYM) == (-127, 127)
    assert orc.q_range(8, AFFINE) == (-128, 127)
    assert orc.q_range(4, SYM) == (-7, 7)
    assert orc.q_range(4, AFFINE) == (-8, 7)
    for bad in [int(b) for b in G["widths"]["bad"].split(",")]:
        with pytest.raises(ValueError):
            orc.q_range(bad, SYM)


@pytest.mark.parametrize("case", ["absmax_int8", "absmax_int4"])
def test_from_absmax_grid_round_trip(orc, case):
    c = G[case]
    bits = int(c["bits"])
    absmax = f32(float(c["absmax"]))
    s, zp, flags = orc.params_from_minmax(-absmax, absmax, bits, SYM)
    assert flags == 0 and zp == int(c["zp"])
    # binary32 reading of "scale = absmax / qmax": the nearest float to the page's value
    assert s == f32(float(c["scale"]))
    qmin, qmax = orc.q_range(bits, SYM)
    for k in range(int(c["kmin"]), int(c["kmax"]) + 1):
        on_grid = orc.dequantize(k, s, zp)
        q = orc.quantize(on_grid, s, zp, qmin, qmax)
        assert q == k
        assert orc.dequantize(q, s, zp) == on_grid


def test_error_bounded_by_half_scale(orc):
    c = G["error_bound"]
    absmax = f32(float(c["absmax"]))
    s, zp, _ = orc.params_from_minmax(-absmax, absmax, 8, SYM)
    qmin, qmax = orc.q_range(8, SYM)
    x = float(c["start"])
    n = 0
    while x <= float(c["stop"]):
        xf = f32(x)
        fq = orc.dequantize(orc.quantize(xf, s, zp, qmin, qmax), s, zp)
        # scale/2 plus the binary32 rounding of x/scale and of the product
        assert abs(fq - xf) <= s / 2 * (1 + 2 ** -20) + abs(xf) * 2 ** -22
        x += float(c["step"])
        n += 1
    assert n == 293


def test_per_channel_scales(orc):
    c = G["per_channel"]
    x = np.array([floats(c["row0"]), floats(c["row1"])], np.float32)
    r = orc.quant_rows(x, 8, SYM)
    assert r["flags"] == 0
    tol = float(c["tol"])
    assert abs(r["scale"][0] - float(c["scale0"])) < tol
    assert abs(r["scale"][1] - float(c["scale1"])) < tol
    assert r["scale"][1] > 10 * r["scale"][0]
    for i in range(2):
        assert np.all(np.abs(r["fq"][i] - x[i]) <= r["scale"][i] / 2 * (1 + 2 ** -20))


def test_ste_example_and_order(orc):
    c = G["ste"]
    x = np.array(floats(c["x"]), np.float32)
    g = np.ones_like(x)
    want = np.array(floats(c["expect"]), np.float32)
    lo, hi = float(c["lo"]), float(c["hi"])
    np.testing.assert_array_equal(orc.ste_backward(g, x, lo, hi), want)
    np.testing.assert_array_equal(orc.ste_backward(g, x, hi, lo), want)  # either order
    # inclusive ends, NaN -> +0, the gradient bits pass unchanged
    x2 = np.array([-1.0, 1.0, np.nan, 0.25], np.float32)
    g2 = np.array([-0.0, 3.5, 7.0, -2.0], np.float32)
    out = orc.ste_backward(g2, x2, -1.0, 1.0)
    assert out.view(np.uint32).tolist() == [g2.view(np.uint32)[0], g2.view(np.uint32)[1], 0,
                                            g2.view(np.uint32)[3]]


def test_affine_example_round_trip_and_nudge(orc):
    c = G["affine_grid"]
    data = np.array(floats(c["data"]), np.float32)
    p = orc.tensor_params_int(data, 8, AFFINE)
    s, zp = float(p["scale"]), p["zp"]
    assert p["flags"] == 0
    qmin, qmax = orc.q_range(8, AFFINE)
    assert qmin <= zp <= qmax
    # real 0 maps onto an exact code
    assert orc.dequantize(zp, s, zp) == 0.0
    # the clamp window covers [min, max] up to half a step
    lo, hi = float(p["lo"]), float(p["hi"])
    assert lo <= data.min() + s / 2 and hi >= data.max() - s / 2
    assert lo == orc.dequantize(qmin, s, zp) and hi == orc.dequantize(qmax, s, zp)
    # scale spans the nudged range over qmax - qmin steps (one binary32 rounding)
    rng_ = np.float32(np.float32(max(data.max(), 0)) - np.float32(min(data.min(), 0)))
    assert s == float(np.float32(rng_ / np.float32(qmax - qmin)))
    for q in range(qmin, qmax + 1):
        v = orc.dequantize(q, s, zp)
        assert orc.quantize(v, s, zp, qmin, qmax) == q


def test_degenerate_and_nonfinite_flags(orc):
    zeros = np.array(floats(G["degenerate"]["data"]), np.float32)
    for scheme in (SYM, AFFINE):
        p = orc.tensor_params_int(zeros, 8, scheme)
        assert p["flags"] & 2 and p["scale"] == 0 and p["zp"] == 0
        codes, fq = orc.fake_quant_int(zeros, 8, scheme, float(p["scale"]), p["zp"])
        assert not codes.any() and not fq.any() and not np.signbit(fq).any()
    x = np.array([1.0, np.inf, -2.0, np.nan], np.float32)
    p = orc.tensor_params_int(x, 8, SYM)
    assert p["flags"] == 1  # NONFINITE, calibrated on the finite elements
    assert p["scale"] == np.float32(np.float32(2.0) / np.float32(127))
    codes, fq = orc.fake_quant_int(x, 8, SYM, float(p["scale"]), p["zp"])
    assert codes.tolist() == [64, 127, -127, 0]  # +Inf clamps, NaN -> code 0
    allnan = np.array([np.nan, np.nan], np.float32)
    p = orc.tensor_params_int(allnan, 4, AFFINE)
    assert p["flags"] == 3


def brute_force_code(x, s, zp, qmin, qmax):
    """Code whose offset q - zp is nearest fl(x/s) (ties to an even offset), clamped."""
    t = np.float32(np.float32(x) / np.float32(s))
    if np.isnan(t):
        return 0
    if np.isinf(t):
        return qmax if t > 0 else qmin
    best, best_d = None, None
    for k in range(int(math.floor(t)) - 1, int(math.floor(t)) + 3):
        d = abs(float(t) - k)
        if best is None or d < best_d or (d == best_d and k % 2 == 0):
            best, best_d = k, d
    return min(max(best + zp, qmin), qmax)


@pytest.mark.parametrize("bits,scheme", [(8, SYM), (8, AFFINE), (4, SYM), (4, AFFINE)])
def test_quantize_brute_force(orc, bits, scheme):
    rng = np.random.default_rng(bits * 10 + scheme)
    qmin, qmax = orc.q_range(bits, scheme)
    for _ in range(4000):
        s = float(np.float32(np.exp(rng.uniform(-8, 4))))
        zp = int(rng.integers(qmin, qmax + 1)) if scheme == AFFINE else 0
        kind = rng.integers(0, 3)
        if kind == 0:  # exact ties t = k + 1/2
            x = float(np.float32((rng.integers(-300, 300) + 0.5) * s))
        elif kind == 1:
            x = float(np.float32(rng.uniform(-1.2, 1.2) * s * (qmax - qmin)))
        else:
            x = float(np.float32(rng.standard_normal() * s * 4))
        assert orc.quantize(x, s, zp, qmin, qmax) == brute_force_code(x, s, zp, qmin, qmax)


def test_doc_formula_order(orc):
    """The doc formula rounds before adding the zero-point: x/scale = 0.49999997 with
    zero-point -37 gives code -37 (adding -37 first would round -36.5 to -36)."""
    s = 1.0
    x = float(np.float32(0.49999997))
    assert orc.quantize(x, s, -37, -128, 127) == -37
    assert orc.quantize(-x, s, 37, -128, 127) == 37


@pytest.mark.parametrize("bits", [8, 4])
def test_rows_invariants(orc, bits):
    """Per-row calibration on lognormal-scaled rows: zero-point cancels, error <=
    scale/2 inside the window, symmetric codes stay in the restricted range, and the
    packed int4 layout is the page's nibble order."""
    rng = np.random.default_rng(7)
    rows, cols = 33, 250
    sig = np.exp(rng.normal(-3, 0.5, rows)).astype(np.float32)
    x = (rng.standard_normal((rows, cols)).astype(np.float32) * sig[:, None]).astype(np.float32)
    x[3, :] = 0.0  # degenerate row
    x[5, 7] = np.inf
    for scheme in (SYM, AFFINE):
        qmin, qmax = orc.q_range(bits, scheme)
        r = orc.quant_rows(x, bits, scheme)
        assert r["flags"] == 3
        if bits == 8:
            codes = r["codes"].astype(np.int32)
        else:
            pk = r["codes"]
            hi = (pk >> 4).astype(np.int32)
            lo = (pk & 0xF).astype(np.int32)
            codes = np.empty((rows, cols), np.int32)
            codes[:, 0::2] = hi[:, : (cols + 1) // 2]
            codes[:, 1::2] = lo[:, : cols // 2]
            codes = np.where(codes >= 8, codes - 16, codes)
        assert codes.min() >= qmin and codes.max() <= qmax
        if scheme == SYM:
            assert (codes != qmin - 1).all()
        s = r["scale"]
        zp = r["zp"]
        # dequant of the stored codes is the fake-quant output
        deq = ((codes - zp[:, None]).astype(np.float32) * s[:, None]).astype(np.float32)
        np.testing.assert_array_equal(deq, r["fq"])
        # zero-point cancellation: fq = clamp(RNE(fl(x/s)), qmin - zp, qmax - zp) * s
        ok = s > 0
        t = (x[ok] / s[ok, None]).astype(np.float32)
        rr = np.clip(np.rint(t), (qmin - zp[ok])[:, None], (qmax - zp[ok])[:, None])
        np.testing.assert_array_equal((rr.astype(np.float32) * s[ok, None]).astype(np.float32),
                                      r["fq"][ok])
        # error bound inside the representable window
        inside = ok[:, None] & np.isfinite(x) & (x >= (qmin - zp)[:, None] * s[:, None]) & (
            x <= (qmax - zp)[:, None] * s[:, None])
        err = np.abs(r["fq"] - x)
        assert np.all(err[inside] <= (s[:, None] / 2 * (1 + 2 ** -20) + np.abs(x) * 2 ** -22)[inside])
        assert s[3] == 0 and zp[3] == 0 and not r["fq"][3].any()


def test_rows_match_scalar_path_and_bf16(orc):
    """quant_rows equals per-row finite_min_max + from_minmax + quantize; bf16 rows
    are the exact widening of their bits."""
    rng = np.random.default_rng(3)
    x = np.maximum(rng.standard_normal((9, 64)), 0).astype(np.float32)
    bits16 = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation gives valid bf16
    wide = (bits16.astype(np.uint32) << 16).view(np.float32)
    r16 = orc.quant_rows(bits16, 8, AFFINE, dtype=1)
    r32 = orc.quant_rows(wide, 8, AFFINE)
    for k in ("codes", "fq", "scale", "zp"):
        np.testing.assert_array_equal(r16[k], r32[k])
    qmin, qmax = orc.q_range(8, AFFINE)
    for i in range(9):
        mn, mx, _ = orc.finite_min_max(wide[i])
        s, zp, _ = orc.params_from_minmax(mn, mx, 8, AFFINE)
        assert r32["scale"][i] == np.float32(s) and r32["zp"][i] == zp
        assert zp == -128  # ReLU rows: min 0 maps to the lowest code
        for j in range(64):
            assert r32["codes"][i, j] == orc.quantize(float(wide[i, j]), s, zp, qmin, qmax)


def test_sqnr_about_six_db_per_bit(orc):
    """CS349E demo 5: per-row integer quantisation of Gaussian data gains about 6 dB
    of SQNR per extra bit (20 log10 2 = 6.02).  int8 vs int4 here: about 4 x 6 dB."""
    rng = np.random.default_rng(0)
    z = rng.standard_normal((64, 4096)).astype(np.float32)

    def sqnr(fq):
        return 10 * np.log10(np.sum(z.astype(np.float64) ** 2) / np.sum((fq - z).astype(np.float64) ** 2))

    s8 = sqnr(orc.quant_rows(z, 8, SYM)["fq"])
    s4 = sqnr(orc.quant_rows(z, 4, SYM)["fq"])
    assert 20.0 < s8 - s4 < 28.0
