"""Pins of the oracle's stochastic rounding ([QAT] module docs "Rounding modes",
RoundingMode::Stochastic: round up with probability equal to the fractional part,
unbiased in expectation) and of its Philox4x32-10 stream.

* The generator against the published known-answer vectors of Philox4x32-10
  (the Random123 release of Salmon, Moraes, Dror and Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC'11).
* The stream layout reading (element i -> word i mod 4 of block floor(i/4), 24-bit
  draws) and its statistics.
* The rounding rule in closed form, over exact 24-bit draws.
* The page's own tests: unbiasedness by Monte-Carlo averaging (scale 0.1, a value
  70 % of the way between two grid points, 400 000 draws, 8 sigma, only the two
  bracketing levels) and stability of a value exactly on the grid.
* Special values, and the fp8 grid: on-grid values never move, between two
  neighbours only those two come out, saturation, NaN, signed zero, ties.
"""
import numpy as np
import pytest

from conftest import read_golden  # noqa: F401  (shared fixtures module)

E4M3, E5M2 = 0, 1
TWO24 = 1 << 24


def f32(v):
    return np.float32(v)


# ---------------------------------------------------------------------------
# Philox4x32-10
# ---------------------------------------------------------------------------

# Known-answer vectors of philox4x32_10 published with the generator (counter, key, output).
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(orc, ctr, key, out):
    assert [int(v) for v in orc.philox4x32_10(ctr, key)] == list(out)


def test_stream_layout(orc):
    """Element i takes word i mod 4 of the block at counter floor(i/4) (low, high
    32 bits) under key (seed low, seed high), scaled by 2^-24 after >> 8."""
    for seed in (0, 1, 0x1234_5678_9ABC_DEF0):
        key = (seed & 0xFFFFFFFF, seed >> 32)
        for i in (0, 1, 2, 3, 4, 7, 1001, (1 << 34) + 5, (1 << 40) + 2):
            b = i >> 2
            w = orc.philox4x32_10((b & 0xFFFFFFFF, b >> 32, 0, 0), key)
            expect = f32(int(w[i & 3]) >> 8) * f32(2.0 ** -24)
            assert orc.sr_uniform(seed, i) == expect, (seed, i)
    # offsets address the same stream
    a = orc.sr_uniform_n(99, 0, 64)
    b = orc.sr_uniform_n(99, 13, 40)
    assert np.array_equal(a[13:53], b)


def test_stream_statistics(orc):
    n = 1 << 20
    u = orc.sr_uniform_n(2024, 0, n).astype(np.float64)
    assert u.min() >= 0.0 and u.max() < 1.0
    k = u * TWO24
    assert np.array_equal(k, np.floor(k)), "draws carry 24 random bits"
    sig = np.sqrt(1.0 / 12.0 / n)
    assert abs(u.mean() - 0.5) < 6 * sig
    assert abs(u.var() - 1.0 / 12.0) < 6 * np.sqrt(1.0 / 180.0 / n)
    counts = np.bincount((u * 256).astype(np.int64), minlength=256)
    chi2 = ((counts - n / 256) ** 2 / (n / 256)).sum()
    assert chi2 < 255 + 6 * np.sqrt(2 * 255), chi2  # chi-square, 255 degrees of freedom
    lag = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(lag) < 6 / np.sqrt(n)
    # words of one block are not correlated either (stride 4 apart and within)
    assert abs(np.corrcoef(u[0::4], u[1::4])[0, 1]) < 6 / np.sqrt(n / 4)


# ---------------------------------------------------------------------------
# integer grid
# ---------------------------------------------------------------------------

def test_rule_closed_form(orc):
    """Up iff the 24-bit draw is below the fractional part; integers never move."""
    for t, lower, frac in ((3.25, 3, 0.25), (-2.75, -3, 0.25), (10.5, 10, 0.5), (-0.125, -1, 0.875)):
        edge = int(np.ceil(frac * TWO24))
        for j, up in ((0, True), (edge - 1, True), (edge, False), (TWO24 - 1, False)):
            u = f32(j) * f32(2.0 ** -24)
            q = orc.quantize_sr(f32(t), f32(1.0), 0, -128, 127, u)
            assert q == lower + (1 if up else 0), (t, j)
    for t in (0.0, -0.0, 5.0, -7.0, 127.0):
        for j in (0, 1, TWO24 - 1):
            assert orc.quantize_sr(f32(t), f32(1.0), 0, -128, 127, f32(j) * f32(2.0 ** -24)) == int(t)


def test_unbiased_monte_carlo(orc):
    """[QAT] stochastic_rounding_is_unbiased, in binary32: scale from absmax 12.7
    (int8 symmetric, 0.1), value 70 % of the way between two grid levels."""
    scale = f32(orc.params_from_minmax(-12.7, 12.7, 8, 0)[0])
    assert scale == f32(f32(12.7) / f32(127.0))
    value = f32(f32(3.0) + f32(f32(0.7) * scale))
    n = 400_000
    codes, fq = orc.fake_quant_int_sr(np.full(n, value, np.float32), 8, 0, float(scale), 0, seed=12345)
    t = f32(value / scale)
    lo_code = int(np.floor(t))
    levels = {lo_code, lo_code + 1}
    assert set(np.unique(codes).tolist()) == levels, "only the two bracketing levels, both seen"
    assert np.all((fq == f32(f32(lo_code) * scale)) | (fq == f32(f32(lo_code + 1) * scale)))
    mean = fq.astype(np.float64).mean()
    assert abs(mean - float(value)) < 8 * float(scale) / np.sqrt(n)


def test_exact_grid_value_is_stable(orc):
    """[QAT] stochastic_rounding_exact_grid_value_is_stable: a value whose quotient
    is an exact integer never moves, whatever the draw."""
    scale = f32(orc.params_from_minmax(-12.7, 12.7, 8, 0)[0])
    assert scale == f32(f32(12.7) / f32(127.0))
    ks = [k for k in range(-127, 128) if f32(f32(f32(k) * scale) / scale) == f32(k)]
    assert len(ks) > 100
    for k in ks[::10]:
        x = f32(f32(k) * scale)
        codes, fq = orc.fake_quant_int_sr(np.full(1000, x, np.float32), 8, 0, float(scale), 0, seed=99)
        assert np.all(codes == k) and np.all(fq == x)


def test_int_specials(orc):
    u = f32(0.999)
    assert orc.quantize_sr(f32(np.nan), f32(0.1), 3, -128, 127, u) == 0
    assert orc.quantize_sr(f32(np.inf), f32(0.1), 3, -128, 127, u) == 127
    assert orc.quantize_sr(f32(-np.inf), f32(0.1), 3, -128, 127, u) == -128
    assert orc.quantize_sr(f32(1.0), f32(0.0), 0, -128, 127, u) == 0
    assert orc.quantize_sr(f32(1e30), f32(0.1), 0, -8, 7, f32(0.0)) == 7
    # zero point added after rounding (doc-formula reading): with t = 1e-5 and zp = 100
    # the code order would round fl(t + 100) = 100 + 7.6e-6 and move down for u = 9e-6
    assert orc.quantize_sr(f32(1e-5), f32(1.0), 100, -128, 127, f32(9e-6)) == 101
    # t = 2.5, zp = 4
    assert orc.quantize_sr(f32(0.25), f32(0.1), 4, -128, 127, f32(0.0)) == 2 + 1 + 4
    assert orc.quantize_sr(f32(0.25), f32(0.1), 4, -128, 127, f32(0.75)) == 2 + 4


# ---------------------------------------------------------------------------
# fp8 grid
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp8_on_grid_never_moves(orc, fmt):
    vals = orc.fp8_decode_n(np.arange(256, dtype=np.uint8), fmt)
    fin = np.isfinite(vals)
    for b in np.arange(256)[fin]:
        y = vals[b]
        for u in (0.0, 0.3, 0.999999):
            assert orc.fp8_encode_sr(float(y), fmt, u) == orc.fp8_encode(float(y), fmt), (fmt, b, u)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp8_between_neighbours(orc, fmt):
    """Between two adjacent positive codes only those two come out, up iff the
    draw is below the fractional position; negative values mirror."""
    vals = orc.fp8_decode_n(np.arange(256, dtype=np.uint8), fmt)
    maxv = 448.0 if fmt == E4M3 else 57344.0
    for b in range(0, 0x7F):
        lo, hi = float(vals[b]), float(vals[b + 1])
        if not (np.isfinite(hi) and hi <= maxv):
            continue
        for frac in (0.125, 0.5, 0.875):
            y = f32(lo + (hi - lo) * frac)
            if not (lo < y < hi):
                continue
            fr = (float(y) - lo) / (hi - lo)
            edge = int(np.ceil(fr * TWO24))
            for j, up in ((0, True), (edge - 1, True), (edge, False), (TWO24 - 1, False)):
                u = float(f32(j) * f32(2.0 ** -24))
                assert orc.fp8_encode_sr(float(y), fmt, u) == (b + 1 if up else b), (fmt, b, frac, j)
                assert orc.fp8_encode_sr(float(-y), fmt, u) == 0x80 | (b + 1 if up else b)


def test_fp8_unbiased(orc):
    n = 200_000
    for fmt, y in ((E4M3, 1.3), (E4M3, 0.003), (E5M2, 1000.7), (E5M2, 3e-6)):
        q, fq = orc.fp8_quantize_sr(np.full(n, y, np.float32), fmt, 1.0, seed=7 + fmt)
        vals = np.unique(fq)
        assert len(vals) == 2
        step = float(vals[1] - vals[0])
        assert abs(fq.astype(np.float64).mean() - float(f32(y))) < 8 * step / np.sqrt(n)


def test_fp8_specials(orc):
    for fmt, top, maxv in ((E4M3, 0x7E, 448.0), (E5M2, 0x7B, 57344.0)):
        for u in (0.0, 0.5, 0.999):
            assert orc.fp8_encode_sr(np.inf, fmt, u) == top
            assert orc.fp8_encode_sr(-np.inf, fmt, u) == 0x80 | top
            assert orc.fp8_encode_sr(np.nan, fmt, u) == 0x7F
            assert orc.fp8_encode_sr(0.0, fmt, u) == 0x00
            assert orc.fp8_encode_sr(-0.0, fmt, u) == 0x80
            assert orc.fp8_encode_sr(1e30, fmt, u) == top
            # above max-normal but below the next step: saturates either way
            assert orc.fp8_encode_sr(maxv * 1.05, fmt, u) == top
        # a binary32 subnormal rounds to 0 or the smallest fp8 subnormal
        tiny = float(np.float32(1e-40))
        assert orc.fp8_encode_sr(tiny, fmt, 0.999) == 0x00
    # half way between two E4M3 codes: up with probability exactly 1/2
    assert orc.fp8_encode_sr(1.0625, E4M3, float(f32((1 << 23) - 1) * f32(2.0 ** -24))) == 0x39
    assert orc.fp8_encode_sr(1.0625, E4M3, 0.5) == 0x38
    q0, _ = orc.fp8_quantize_sr(np.ones(8, np.float32), E4M3, 0.0, seed=1)
    assert np.all(q0 == 0)
