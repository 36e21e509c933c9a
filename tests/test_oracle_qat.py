"""Pins of the oracle's QAT step ([QAT] QatOptimizer::step: AdamW update of the
fp32 master, then requantize -- per-tensor min / max recalibration and
fake_quant_int for integer targets, fake_quant_fp8 of the master for fp8 targets).

* The page's two optimizer tests (int8 symmetric and fp8 E4M3 targets): the
  master moves, stays off the grid, and the view is the fake-quant of the
  updated master under the recalibrated parameters.
* Closed forms of Adam with bias correction: the first step moves every weight
  by lr g / (|g| + eps); a constant gradient moves it by that amount every step;
  decoupled weight decay alone scales the master by (1 - lr wd)^T; a zero
  gradient without decay leaves the master bit-identical.
* Sign symmetry, and the stochastic view's bracketing levels.
"""
import numpy as np
import pytest

LR = 0.1


def f32(v):
    return np.float32(v)


def test_page_int8_symmetric_target(orc):
    w0 = np.float32([0.12, -0.37, 0.88, -0.05, 0.51])
    g = np.float32([0.1, -0.2, 0.05, 0.3, -0.15])
    z = np.zeros(5, np.float32)
    r = orc.qat_step_int(w0, g, z, z, 0.1, 1, bits=8, scheme=0)
    assert np.any(np.abs(r["w"] - w0) > 1e-6), "the master moved"
    p = orc.tensor_params_int(r["w"], 8, 0)
    assert (f32(r["scale"]), r["zp"]) == (p["scale"], p["zp"]), "recalibrated on the updated master"
    codes, view = orc.fake_quant_int(r["w"], 8, 0, float(p["scale"]), p["zp"])
    assert np.array_equal(r["codes"], codes) and np.array_equal(r["view"], view)
    k = r["view"].astype(np.float64) / float(r["scale"])
    # on the grid up to the one rounding of fl(code * scale) (binary32 reading)
    assert np.all(np.abs(k - np.round(k)) <= 2.0 ** -22 * np.maximum(1.0, np.abs(k))), "view on the grid"
    km = r["w"].astype(np.float64) / float(r["scale"])
    assert np.any(np.abs(km - np.round(km)) > 1e-6), "master keeps full precision"


def test_page_fp8_target(orc):
    w0 = np.float32([0.3, -1.2, 4.0, -0.01, 2.5])
    g = np.float32([0.2, 0.1, -0.3, 0.4, -0.05])
    z = np.zeros(5, np.float32)
    r = orc.qat_step_fp8(w0, g, z, z, 0.05, 1, fmt=0)
    assert np.array_equal(r["q"], orc.fp8_encode_n(r["w"], 0))
    assert np.array_equal(r["view"], orc.fp8_decode_n(r["q"], 0))
    assert np.any(r["w"] != w0)


def test_first_step_closed_form(orc):
    rng = np.random.default_rng(1)
    w0 = rng.standard_normal(10_000).astype(np.float32)
    g = (rng.standard_normal(10_000) * np.exp(rng.uniform(-8, 3, 10_000))).astype(np.float32)
    z = np.zeros_like(w0)
    w1, m1, v1 = orc.adamw_update(w0, g, z, z, LR, 1)
    expect = w0.astype(np.float64) - LR * g.astype(np.float64) / (np.abs(g.astype(np.float64)) + 1e-8)
    tol = 4 * np.spacing(np.maximum(np.abs(w0), f32(LR))).astype(np.float64)
    assert np.all(np.abs(w1 - expect) <= tol)
    c1, c2 = f32(1.0) - f32(0.9), f32(1.0) - f32(0.999)  # (1 - beta) in binary32
    assert np.array_equal(m1, c1 * g) and np.array_equal(v1, c2 * g * g)


def test_constant_gradient_closed_form(orc):
    """m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2 exactly in real arithmetic, so
    with bias correction every step moves the weight by lr g / (|g| + eps)."""
    rng = np.random.default_rng(2)
    w = rng.standard_normal(2000).astype(np.float32)
    g = (rng.standard_normal(2000) + 0.1).astype(np.float32)
    m = np.zeros_like(w)
    v = np.zeros_like(w)
    w0 = w.copy()
    T = 60
    for t in range(1, T + 1):
        w, m, v = orc.adamw_update(w, g, m, v, 0.01, t)
    expect = w0.astype(np.float64) - T * 0.01 * g / (np.abs(g.astype(np.float64)) + 1e-8)
    assert np.max(np.abs(w - expect)) < 2e-5


def test_weight_decay_alone(orc):
    w0 = np.float32([1.0, -2.5, 3e-3, 40.0])
    z = np.zeros(4, np.float32)
    w, m, v = w0.copy(), z.copy(), z.copy()
    for t in range(1, 101):
        w, m, v = orc.adamw_update(w, z, m, v, LR, t, weight_decay=0.01)
    expect = w0.astype(np.float64) * (1.0 - LR * 0.01) ** 100
    assert np.allclose(w, expect, rtol=2e-5, atol=0)
    assert np.all(m == 0) and np.all(v == 0)


def test_zero_gradient_is_identity(orc):
    rng = np.random.default_rng(3)
    w0 = rng.standard_normal(1000).astype(np.float32)
    z = np.zeros_like(w0)
    w, m, v = w0, z, z
    for t in range(1, 6):
        w, m, v = orc.adamw_update(w, z, m, v, LR, t)
    assert np.array_equal(w.view(np.uint32), w0.view(np.uint32))


def test_bias_corrections(orc):
    assert orc.adamw_bias_corrections(0.9, 0.999, 1) == (f32(1.0 - f32(0.9)), f32(1.0 - f32(0.999)))
    b1, b2 = orc.adamw_bias_corrections(0.9, 0.999, 100_000)
    assert b1 == f32(1.0) and b2 == f32(1.0)


def test_sign_symmetry(orc):
    rng = np.random.default_rng(4)
    w = rng.standard_normal(500).astype(np.float32)
    g = rng.standard_normal(500).astype(np.float32)
    m = (rng.standard_normal(500) * 0.01).astype(np.float32)
    v = (rng.random(500) * 0.01).astype(np.float32)
    a = orc.adamw_update(w, g, m, v, LR, 7, weight_decay=0.02)
    b = orc.adamw_update(-w, -g, -m, v, LR, 7, weight_decay=0.02)
    assert np.array_equal(a[0], -b[0]) and np.array_equal(a[1], -b[1]) and np.array_equal(a[2], b[2])


@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 1)])
def test_stochastic_view_brackets(orc, bits, scheme):
    rng = np.random.default_rng(5)
    w = rng.standard_normal(4096).astype(np.float32)
    g = rng.standard_normal(4096).astype(np.float32)
    z = np.zeros_like(w)
    r = orc.qat_step_int(w, g, z, z, 0.01, 1, bits=bits, scheme=scheme, rounding=1, seed=11)
    qmin, qmax = orc.q_range(bits, scheme)
    t = r["w"] / r["scale"]
    lo = np.clip(np.floor(t) + r["zp"], qmin, qmax)
    hi = np.clip(np.floor(t) + 1 + r["zp"], qmin, qmax)
    assert np.all((r["codes"] == lo) | (r["codes"] == hi))
    rf = orc.qat_step_fp8(w, g, z, z, 0.01, 1, fmt=1, rounding=1, seed=11)
    near = orc.fp8_encode_n(rf["w"], 1)
    assert np.all(np.abs(rf["q"].astype(int) - near.astype(int)) <= 1)


def test_page_association_of_the_update(orc):
    """[QAT] QatOptimizer::step writes v = beta2 v + (1 - beta2) g g,
    w -= lr weight_decay w and w -= lr m_hat / (sqrt(v_hat) + eps); Rust takes
    a * b * c and a * b / c left to right.  On inputs where the other grouping
    rounds differently in binary32, the oracle must give the page's grouping:
    ((1 - beta2) g) g, (lr wd) w and (lr m_hat) / (sqrt(v_hat) + eps)."""
    rng = np.random.default_rng(9)
    n = 200_000
    g = (rng.standard_normal(n) * np.exp(rng.uniform(-4, 4, n))).astype(np.float32)
    lr = f32(0.0173)  # not a power of two, so lr * x rounds
    z = np.zeros(n, np.float32)
    # from w = 0, m = v = 0 at t = 1 the step itself is the new master (0 - s = -s exactly)
    w1, m1, v1 = orc.adamw_update(z, g, z, z, float(lr), 1)
    c2 = f32(1.0) - f32(0.999)
    page_v, other_v = (c2 * g) * g, c2 * (g * g)
    assert np.count_nonzero(page_v != other_v) > 1000
    assert np.array_equal(v1.view(np.uint32), page_v.view(np.uint32))
    bc1, bc2 = orc.adamw_bias_corrections(0.9, 0.999, 1)
    m_hat, v_hat = m1 / bc1, v1 / bc2
    d = np.sqrt(v_hat) + f32(1e-8)
    page_w, other_w = -((lr * m_hat) / d), -(lr * (m_hat / d))
    assert np.count_nonzero(page_w != other_w) > 1000
    assert np.array_equal(w1.view(np.uint32), page_w.view(np.uint32))
    # decoupled decay alone (zero gradient: m_hat = 0 and the Adam step is 0)
    w0 = (rng.standard_normal(n) * 3).astype(np.float32)
    wd = f32(0.0371)
    wdec, _, _ = orc.adamw_update(w0, z, z, z, float(lr), 1, weight_decay=float(wd))
    page_d, other_d = w0 - (lr * wd) * w0, w0 - lr * (wd * w0)
    assert np.count_nonzero(page_d != other_d) > 10  # the subtraction from w absorbs most differences
    assert np.array_equal(wdec.view(np.uint32), page_d.view(np.uint32))
