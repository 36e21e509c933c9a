"""Pins of the oracle's percentile calibration ([QAT]
QuantParams::per_tensor_percentile: nearest-rank quantiles floor(cf * last) and
ceil((1 - cf) * last) of the sorted values, then from_minmax).

* The page's test: 0.00 .. 0.99 plus an outlier 1000, cf = 0.02, int8 symmetric
  -> a smaller scale than plain absmax calibration.
* cf = 0 selects the minimum and maximum: the result equals per-tensor min / max
  calibration (flags included) on data with zeros, signed zeros, duplicates and
  non-finite values.
* The selected values are the order statistics of numpy's sort of the finite
  values at the page's indices, and the parameters are from_minmax of them.
"""
import numpy as np
import pytest


def test_page_clips_outlier(orc):
    v = np.concatenate([np.arange(100) / 100.0, [1000.0]]).astype(np.float32)
    clipped = orc.percentile_params(v, 8, 0, 0.02)
    plain = orc.tensor_params_int(v, 8, 0)
    assert clipped["scale"] < plain["scale"]
    # last = 100: lo = floor(2.0) = 2 -> 0.02, hi = ceil(98.0) = 98 -> 0.98
    assert clipped["sel_min"] == np.float32(0.02) and clipped["sel_max"] == np.float32(0.98)


@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 0), (4, 1)])
def test_zero_fraction_is_minmax(orc, bits, scheme):
    rng = np.random.default_rng(bits + scheme)
    x = rng.standard_normal(5000).astype(np.float32)
    x[:30] = 0.0
    x[30:40] = -0.0
    x[40:60] = x[60]
    x[100] = np.nan
    x[200] = np.inf
    p = orc.percentile_params(x, bits, scheme, 0.0)
    q = orc.tensor_params_int(x, bits, scheme)
    assert (p["scale"], p["zp"], p["lo"], p["hi"], p["flags"]) == (q["scale"], q["zp"], q["lo"], q["hi"], q["flags"])


@pytest.mark.parametrize("n", [1, 2, 3, 10, 1001, 65537])
@pytest.mark.parametrize("cf", [0.0, 0.001, 0.02, 0.25, 0.49999])
def test_order_statistics(orc, n, cf):
    rng = np.random.default_rng(n)
    x = (rng.standard_t(3, n) * 0.1).astype(np.float32)
    if n > 10:
        x[::7] = np.round(x[::7], 1)  # duplicates
        x[3] = np.nan
        x[5] = -np.inf
    fin = np.sort(x[np.isfinite(x)], kind="stable")
    last = fin.size - 1
    lo = min(int(np.floor(cf * last)), last)
    hi = min(int(np.ceil((1.0 - cf) * last)), last)
    p = orc.percentile_params(x, 8, 1, cf)
    assert p["sel_min"] == fin[lo] and p["sel_max"] == fin[hi]
    s, z, f = orc.params_from_minmax(float(fin[lo]), float(fin[hi]), 8, 1)
    assert (p["scale"], p["zp"]) == (np.float32(s), z)


def test_no_finite_values(orc):
    p = orc.percentile_params(np.float32([np.nan, np.inf]), 8, 0, 0.1)
    assert p["scale"] == 0 and p["flags"] == 3  # NONFINITE | DEGENERATE
