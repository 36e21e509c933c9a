"""Pins of the oracle's fp8 cast against what the pages and IEEE arithmetic fix.

Page: optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, module docs "fp8
quantization (E4M3 / E5M2)" (format table, saturation, unified ULP rule) and
its fp8 unit tests (fixtures in tests/golden/qat_fp8_*.txt).

Independent second definitions used here (none calls the oracle's code path):
* a closed-form table of every finite fp8 value built from the format table;
* "nearest representable value, ties to the even code" evaluated with numpy
  searchsorted over that table (equal to the page's unified ULP rule followed by
  saturation for every finite input);
* torch's float8_e4m3fn / float8_e5m2 conversions (library routine) for
  finite inputs no larger than max-normal.
"""
import math

import numpy as np
import pytest
import torch

from conftest import parse_num, read_golden

FMT = {"E4M3": 0, "E5M2": 1}


def format_table():
    out = {}
    for row in read_golden("qat_fp8_format_table.txt"):
        name, mb, bias, mx, mnn, mns, maxbits, nanbits, infbits = row
        out[name] = dict(mbits=int(mb), bias=int(bias), max=parse_num(mx), min_normal=parse_num(mnn),
                         min_sub=parse_num(mns), max_bits=int(parse_num(maxbits)),
                         nan_bits=int(parse_num(nanbits)),
                         inf_bits=None if infbits == "-" else int(parse_num(infbits)))
    return out


TABLE = format_table()


def closed_form_positive_values(name):
    """All non-negative finite values of the format, indexed by their 7-bit code."""
    f = TABLE[name]
    mb, bias = f["mbits"], f["bias"]
    ebits = 7 - mb
    vals = []
    for code in range(128):
        e, m = code >> mb, code & ((1 << mb) - 1)
        if name == "E4M3" and e == (1 << ebits) - 1 and m == (1 << mb) - 1:
            break  # S.1111.111 is NaN
        if name == "E5M2" and e == (1 << ebits) - 1:
            break  # exponent field 11111: Inf / NaN
        if e == 0:
            v = m * 2.0 ** (1 - bias - mb)
        else:
            v = (1 + m / 2 ** mb) * 2.0 ** (e - bias)
        vals.append(v)
    return np.array(vals, dtype=np.float64)


def nearest_even_encode(y: np.ndarray, name: str) -> np.ndarray:
    """Second definition: nearest finite fp8 value, ties to the even code; NaN -> 0x7F."""
    V = closed_form_positive_values(name)
    y = y.astype(np.float32)
    a = np.abs(np.where(np.isnan(y), 0, y).astype(np.float64))
    a_fin = np.minimum(a, V[-1])  # above max-normal (and Inf): the largest value
    idx = np.searchsorted(V, a_fin, side="left")
    idx = np.clip(idx, 0, len(V) - 1)
    lo = np.clip(idx - 1, 0, len(V) - 1)
    d_hi = np.abs(V[idx] - a_fin)
    d_lo = np.abs(a_fin - V[lo])
    pick = np.where(d_lo < d_hi, lo, idx)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, idx), pick)
    sign = np.signbit(y).astype(np.uint8) << 7
    out = (sign | pick.astype(np.uint8)).astype(np.uint8)
    out[np.isnan(y)] = 0x7F
    return out


@pytest.mark.parametrize("name", ["E4M3", "E5M2"])
def test_format_constants(orc, name):
    """Decoded limits equal the format table (max, min-normal, min-subnormal)."""
    f = TABLE[name]
    fmt = FMT[name]
    assert orc.fp8_decode(f["max_bits"], fmt) == f["max"]
    assert orc.fp8_decode(0x80 | f["max_bits"], fmt) == -f["max"]
    assert orc.fp8_decode(1 << f["mbits"], fmt) == f["min_normal"]
    assert orc.fp8_decode(0x01, fmt) == f["min_sub"]
    assert math.isnan(orc.fp8_decode(f["nan_bits"], fmt))
    if f["inf_bits"] is not None:
        assert orc.fp8_decode(f["inf_bits"], fmt) == math.inf
    # the page's closed forms 1.75 * 2^8 and 1.75 * 2^15, 2^(1-bias), 2^(1-bias-mbits)
    emax = {"E4M3": 8, "E5M2": 15}[name]
    assert f["max"] == 1.75 * 2.0 ** emax
    assert f["min_normal"] == 2.0 ** (1 - f["bias"])
    assert f["min_sub"] == 2.0 ** (1 - f["bias"] - f["mbits"])


@pytest.mark.parametrize("name", ["E4M3", "E5M2"])
def test_decode_all_codes_matches_closed_form(orc, name):
    fmt = FMT[name]
    V = closed_form_positive_values(name)
    dec = orc.fp8_decode_n(np.arange(256, dtype=np.uint8), fmt).astype(np.float64)
    for code in range(256):
        mag = code & 0x7F
        sign = -1.0 if code & 0x80 else 1.0
        if mag < len(V):
            assert dec[code] == sign * V[mag], (name, code)
            if mag == 0:
                assert math.copysign(1.0, dec[code]) == sign
        elif name == "E5M2" and mag == 0x7C:
            assert dec[code] == sign * math.inf
        else:
            assert math.isnan(dec[code]), (name, code)


def test_page_worked_values(orc):
    """The page's fp8 unit tests, value by value (tests/golden/qat_fp8_examples.txt)."""
    rows = read_golden("qat_fp8_examples.txt")
    assert len(rows) == 32
    for test, name, xin, want in rows:
        fmt = FMT[name]
        x = np.float32(parse_num(xin))
        b = orc.fp8_encode(float(x), fmt)
        got = orc.fp8_decode(b, fmt)
        w = parse_num(want)
        if math.isnan(w):
            assert math.isnan(got), test
            assert b == TABLE[name]["nan_bits"]
        else:
            assert got == w, (test, xin, got, w)
            assert math.copysign(1.0, got) == math.copysign(1.0, w)
    # saturated outputs are the page's largest-finite bit patterns
    assert orc.fp8_encode(1000.0, 0) == TABLE["E4M3"]["max_bits"]
    assert orc.fp8_encode(-1000.0, 0) == 0x80 | TABLE["E4M3"]["max_bits"]
    assert orc.fp8_encode(math.inf, 1) == TABLE["E5M2"]["max_bits"]
    assert orc.fp8_encode(-math.inf, 1) == 0x80 | TABLE["E5M2"]["max_bits"]
    # 1.1 lands within half an ULP (0.125 / 2) of itself
    assert abs(orc.fp8_decode(orc.fp8_encode(1.1, 0), 0) - 1.1) <= 0.0625


@pytest.mark.parametrize("name", ["E4M3", "E5M2"])
def test_codes_round_trip_and_midpoints_tie_to_even(orc, name):
    """Brute force over all 256 codes: decode then encode is the identity (NaN
    codes -> 0x7F, E5M2 infinities saturate); every midpoint between neighbouring
    finite values goes to the neighbour with the even code."""
    fmt = FMT[name]
    f = TABLE[name]
    for code in range(256):
        v = orc.fp8_decode(code, fmt)
        b = orc.fp8_encode(v, fmt)
        mag = code & 0x7F
        if math.isnan(v):
            assert b == 0x7F
        elif math.isinf(v):
            assert b == (code & 0x80) | f["max_bits"]
        else:
            assert b == code, (name, hex(code), hex(b))
    V = closed_form_positive_values(name)
    for i in range(len(V) - 1):
        mid = np.float32((V[i] + V[i + 1]) / 2)
        assert float(mid) == (V[i] + V[i + 1]) / 2  # midpoints are exact in binary32
        even = i if i % 2 == 0 else i + 1
        assert orc.fp8_encode(float(mid), fmt) == even
        assert orc.fp8_encode(-float(mid), fmt) == 0x80 | even
        up = np.nextafter(mid, np.float32(np.inf))
        dn = np.nextafter(mid, np.float32(0))
        assert orc.fp8_encode(float(up), fmt) == i + 1
        assert orc.fp8_encode(float(dn), fmt) == i
    # just above max-normal: rounds down to max (below the midpoint) or saturates
    assert orc.fp8_encode(float(np.nextafter(np.float32(V[-1]), np.float32(np.inf))), fmt) == len(V) - 1


def structured_sample(seed=1):
    """fp32 inputs covering every rounding boundary of both formats plus noise."""
    rng = np.random.default_rng(seed)
    parts = [rng.integers(0, 2 ** 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)]
    lows = []
    for mb in (2, 3):
        half = 1 << (22 - mb)
        full = 1 << (23 - mb)
        lows += [0, 1, 2, half - 2, half - 1, half, half + 1, half + 2, full - 2, full - 1]
    lows = np.array(sorted(set(lows)), dtype=np.uint32)
    tops = np.arange(16, dtype=np.uint32) << 19  # top 4 mantissa bits
    exps = np.arange(127 - 40, 127 + 21, dtype=np.uint32)  # binades 2^-40 .. 2^20
    e, t, l = np.meshgrid(exps, tops, lows, indexing="ij")
    bits = (e << 23) | t | l
    bits = bits.ravel()
    parts += [bits, bits | np.uint32(0x80000000)]
    # binary32 subnormals and the extremes
    parts.append(np.array([0, 1, 2, 0x7FFFFF, 0x800000, 0x7F7FFFFF, 0x7F800000, 0x7FC00000,
                           0xFF800000, 0x80000000, 0x80000001], dtype=np.uint32))
    return np.concatenate(parts).view(np.float32)


@pytest.mark.parametrize("name", ["E4M3", "E5M2"])
def test_unified_ulp_rule_equals_nearest_even(orc, name):
    """Oracle cast == nearest representable value with ties to even, then saturate,
    over a sample that hits every rounding boundary of both formats."""
    fmt = FMT[name]
    y = structured_sample()
    got = orc.fp8_encode_n(y, fmt)
    want = nearest_even_encode(y, name)
    inf = np.isinf(y)
    want[inf] = (np.signbit(y[inf]).astype(np.uint8) << 7) | TABLE[name]["max_bits"]
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("name,tdt", [("E4M3", torch.float8_e4m3fn), ("E5M2", torch.float8_e5m2)])
def test_matches_torch_cast_in_range(orc, name, tdt):
    """torch's float8 conversion agrees wherever it is defined without overflow."""
    fmt = FMT[name]
    y = structured_sample(seed=2)
    keep = np.isfinite(y) & (np.abs(y) <= TABLE[name]["max"])
    y = y[keep]
    got = orc.fp8_encode_n(y, fmt)
    ref = torch.from_numpy(y).to(tdt).view(torch.uint8).numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_sign_and_specials(orc):
    for fmt in (0, 1):
        assert orc.fp8_encode(0.0, fmt) == 0x00
        assert orc.fp8_encode(-0.0, fmt) == 0x80
        assert orc.fp8_encode(math.nan, fmt) == 0x7F
        assert orc.fp8_encode(-math.nan, fmt) == 0x7F
        # binary32 subnormals round to signed zero in both formats
        tiny = float(np.array([1], np.uint32).view(np.float32)[0])
        assert orc.fp8_encode(tiny, fmt) == 0x00
        assert orc.fp8_encode(-tiny, fmt) == 0x80


def test_per_tensor_scale_and_zero_scale(orc):
    """Per-tensor fp8 calibration: scale = finite amax / max-normal; a zero scale gives
    byte 0 and fake-quant +0 (marlin_repack.rs `quantized_fp8_bits`)."""
    x = np.array([1.0, -896.0, np.inf, np.nan, 3.0], np.float32)
    amax = orc.amax_finite(x)
    assert amax == np.float32(896.0)
    s, flags = orc.fp8_scale(float(amax), 0)
    assert s == np.float32(2.0) and flags == 0
    q, fq = orc.fp8_quantize(x, 0, float(s))
    assert list(q) == [orc.fp8_encode(0.5, 0), 0x80 | TABLE["E4M3"]["max_bits"],
                       TABLE["E4M3"]["max_bits"], 0x7F, orc.fp8_encode(1.5, 0)]
    assert fq[1] == -896.0 and fq[2] == 896.0 and np.isnan(fq[3]) and fq[4] == 3.0
    z = np.array([0.0, -0.0, np.nan, np.inf], np.float32)
    s0, flags0 = orc.fp8_scale(float(orc.amax_finite(z)), 1)
    assert s0 == 0.0 and flags0 == 2
    q0, fq0 = orc.fp8_quantize(z, 1, float(s0))
    assert list(q0) == [0, 0, 0, 0]
    assert all(v == 0.0 and not np.signbit(v) for v in fq0)
    # dequantize is decode * scale
    codes = np.arange(256, dtype=np.uint8)
    out = orc.fp8_dequantize(codes, 1, 0.5)
    dec = orc.fp8_decode_n(codes, 1)
    np.testing.assert_array_equal(out, (dec * np.float32(0.5)).astype(np.float32))
