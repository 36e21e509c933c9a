"""Pins of the oracle's group-wise quantization ([CS] demo 3 "granularity":
groups of `group` consecutive elements along each row, one scale per group;
each group calibrated as a [QAT] channel).

* A worked example with exact scales (127 -> 1.0, 254 -> 2.0, an affine group
  0..255 -> scale 1, zero-point -128): codes, ties to even and per-group scales
  by hand.
* One group per row (group = cols, or larger) is per-row quantization.
* Groups that divide the row are per-row quantization of the [rows * cols /
  group, group] reshape (every output, int8 and int4, f32 and bf16, specials).
* A ragged last group is the per-row result of that tail on its own.
* Group 1: every non-zero finite element gets code +-qmax (symmetric).
* The demo's finding: on a weight matrix with per-row scales, error falls from
  per-tensor to per-row to 128-groups to 32-groups, for INT8 and INT4.
"""
import numpy as np
import pytest


def test_worked_example(orc):
    x = np.float32([[127.0, -63.5, 2.5, 254.0, 1.0, -3.0]])
    r = orc.quant_groups(x, 3, 8, 0)
    assert r["scale"].tolist() == [[1.0, 2.0]]
    assert r["zp"].tolist() == [[0, 0]]
    # 127/1, -63.5 -> -64 (tie to even), 2.5 -> 2; 254/2 = 127, 0.5 -> 0, -1.5 -> -2
    assert r["codes"].tolist() == [[127, -64, 2, 127, 0, -2]]
    assert r["fq"].tolist() == [[127.0, -64.0, 2.0, 254.0, 0.0, -4.0]]
    a = orc.quant_groups(np.float32([[0.0, 255.0, 128.0, 3.0]]), 2, 8, 1)
    # affine int8 on [0, 255]: scale 255 / 255 = 1, zero-point RNE(-128 - 0) = -128
    assert a["scale"][0, 0] == 1.0 and a["zp"][0, 0] == -128
    assert a["codes"][0, :2].tolist() == [-128, 127]


@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 0), (4, 1)])
@pytest.mark.parametrize("dtype", [0, 1])
def test_one_group_per_row_is_per_row(orc, bits, scheme, dtype):
    rng = np.random.default_rng(bits * 10 + scheme + dtype)
    x = rng.standard_normal((7, 45)).astype(np.float32)
    x[2] = 0.0
    x[3, 5] = np.nan
    x[4, 9] = -np.inf
    if dtype == 1:
        x = (x.view(np.uint32) >> 16).astype(np.uint16)
    ref = orc.quant_rows(x, bits, scheme, dtype=dtype)
    for g in (45, 46, 1000):
        r = orc.quant_groups(x, g, bits, scheme, dtype=dtype)
        for k in ("codes", "fq"):
            assert np.array_equal(r[k].view(np.uint8), ref[k].view(np.uint8)), (g, k)
        assert np.array_equal(r["scale"][:, 0], ref["scale"]) and np.array_equal(r["zp"][:, 0], ref["zp"])
        assert r["flags"] == ref["flags"]


@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 0), (4, 1)])
@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("group", [2, 8, 32, 128])
def test_dividing_groups_are_rows_of_the_reshape(orc, bits, scheme, dtype, group):
    rng = np.random.default_rng(group + bits + scheme)
    rows, cols = 5, 256
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.standard_normal((rows, 1)))).astype(np.float32)
    x[1, :group] = 0.0           # a degenerate group
    x[2, 3] = np.nan
    x[3, 17] = np.inf
    x[4, 100] = -0.0
    if dtype == 1:
        x = (x.view(np.uint32) >> 16).astype(np.uint16)
    r = orc.quant_groups(x, group, bits, scheme, dtype=dtype)
    ref = orc.quant_rows(x.reshape(-1, group), bits, scheme, dtype=dtype)
    # even groups pack into whole bytes, so the nibble layouts coincide too
    assert np.array_equal(r["codes"].reshape(-1).view(np.uint8), ref["codes"].reshape(-1).view(np.uint8))
    assert np.array_equal(r["fq"].reshape(-1).view(np.uint32), ref["fq"].reshape(-1).view(np.uint32))
    assert np.array_equal(r["scale"].reshape(-1), ref["scale"]) and np.array_equal(r["zp"].reshape(-1), ref["zp"])
    assert r["flags"] == ref["flags"]


@pytest.mark.parametrize("bits,scheme", [(8, 1), (4, 0)])
def test_ragged_last_group(orc, bits, scheme):
    rng = np.random.default_rng(3)
    rows, cols, group = 4, 100, 32  # groups of 32, 32, 32 and a tail of 4
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[:, 96:] *= 50.0
    r = orc.quant_groups(x, group, bits, scheme)
    assert r["scale"].shape == (rows, 4)
    body = orc.quant_rows(np.ascontiguousarray(x[:, :96]).reshape(-1, group), bits, scheme)
    tail = orc.quant_rows(np.ascontiguousarray(x[:, 96:]), bits, scheme)
    assert np.array_equal(r["scale"][:, :3].reshape(-1), body["scale"])
    assert np.array_equal(r["scale"][:, 3], tail["scale"])
    assert np.array_equal(r["fq"][:, :96].reshape(-1), body["fq"].reshape(-1))
    assert np.array_equal(r["fq"][:, 96:], tail["fq"])


def test_group_of_one(orc):
    x = np.float32([[0.3, -2.0, 0.0, 1e-30, -7.5e20, 5.0]])
    r = orc.quant_groups(x, 1, 8, 0)
    assert r["codes"].tolist() == [[127, -127, 0, 127, -127, 127]]
    assert r["flags"] == 2  # the zero group is degenerate


def test_finer_groups_lower_error(orc):
    # the demo's weight matrix: per-row scales (lognormal, sigma 0.5)
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 4096)) * 0.02 * np.exp(rng.normal(0, 0.5, size=(64, 1)))).astype(np.float32)

    def rel(fq):
        return np.linalg.norm(fq.astype(np.float64) - w) / np.linalg.norm(w.astype(np.float64))

    for bits in (8, 4):
        tensor = rel(orc.quant_rows(w.reshape(1, -1), bits, 0)["fq"].reshape(w.shape))
        row = rel(orc.quant_rows(w, bits, 0)["fq"])
        g128 = rel(orc.quant_groups(w, 128, bits, 0)["fq"])
        g32 = rel(orc.quant_groups(w, 32, bits, 0)["fq"])
        assert tensor > row > g128 > g32, (bits, tensor, row, g128, g32)
