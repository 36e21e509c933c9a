"""Pins of the oracle's per-column calibration ([QAT] per_channel_params and
fake_quant_int_per_channel with axis = 1: each column is a channel).

* The page's per-channel example laid out along columns: channel scales 1/127
  and 100/127 (binary32), error within half a scale.
* Axis 1 of X is axis 0 of X^T: every output (codes, fake-quant, scales,
  zero-points, flags) equals the per-row result of the transpose, for int8 and
  int4, symmetric and affine, fp32 and bf16, with zero / NaN / Inf columns.
"""
import numpy as np
import pytest


def unpack_rows(packed, cols):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], 2 * p.shape[1]), np.int8)
    hi = (p >> 4).astype(np.int16)
    lo = (p & 0xF).astype(np.int16)
    out[:, 0::2] = np.where(hi >= 8, hi - 16, hi)
    out[:, 1::2] = np.where(lo >= 8, lo - 16, lo)
    return out[:, :cols]


def test_page_example_along_columns(orc):
    x = np.float32([[0.0, 0.5, 1.0], [0.0, 50.0, 100.0]]).T.copy()  # 3 rows, 2 channel columns
    r = orc.quant_cols(x, 8, 0)
    assert r["scale"][0] == np.float32(np.float32(1.0) / np.float32(127.0))
    assert r["scale"][1] == np.float32(np.float32(100.0) / np.float32(127.0))
    assert r["scale"][1] > 10 * r["scale"][0]
    err = np.abs(r["fq"].astype(np.float64) - x)
    assert np.all(err <= r["scale"][None, :] / 2 + 1e-7)


@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 0), (4, 1)])
@pytest.mark.parametrize("bf16", [False, True])
def test_columns_are_rows_of_the_transpose(orc, bits, scheme, bf16):
    rng = np.random.default_rng(bits * 10 + scheme + bf16)
    rows, cols = 37, 23
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.normal(-2, 1, (1, cols)))).astype(np.float32)
    x[:, 3] = 0.0
    x[5, 7] = np.nan
    x[9, 8] = np.inf
    x[:, 11] = -np.abs(x[:, 11])
    if bf16:
        xb = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation is enough for a pin
        xt = np.ascontiguousarray(xb.T)
        r = orc.quant_cols(xb, bits, scheme, dtype=1)
        t = orc.quant_rows(xt, bits, scheme, dtype=1)
    else:
        r = orc.quant_cols(x, bits, scheme)
        t = orc.quant_rows(np.ascontiguousarray(x.T), bits, scheme)
    assert np.array_equal(r["scale"], t["scale"]) and np.array_equal(r["zp"], t["zp"])
    assert r["flags"] == t["flags"]
    codes_r = r["codes"] if bits == 8 else unpack_rows(r["codes"], cols)
    codes_t = t["codes"] if bits == 8 else unpack_rows(t["codes"], rows)
    assert np.array_equal(codes_r, codes_t.T)
    assert np.array_equal(r["fq"].view(np.uint32), t["fq"].T.view(np.uint32))
