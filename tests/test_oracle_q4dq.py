"""Pins of the oracle's 4-bit blocks with double-quantised scales, and of the
32-element E4M3 blocks with power-of-two (E8M0) scales.

Pages:
* aprender-train 0.32.0 entrenar/quant/double_quant.rs ("Double quantization for
  QLoRA"): module docs (memory per 64 values), quantize_4bit_double,
  dequantize_4bit_double, reconstruct_scales and its tests
  (tests/golden/dq_examples.txt);
* CS349E 05_quantization_basics.py demo 4, `block_scaled` kind "e8m0"
  (tests/golden/cs_mx_examples.txt).

The first-level quantizer's body is not on the page (it is imported); its
reading (64-element blocks, scale absmax/7, ties to even) is pinned here by the
page's own tests and by brute force, and its tie rule is a reading.
"""
import math

import numpy as np
import pytest

from conftest import read_golden_kv

DQ = read_golden_kv("dq_examples.txt")
MX = read_golden_kv("cs_mx_examples.txt")


def unpack_page_decoder(packed, n):
    """dequantize_4bit_double's nibble rule, written independently: the element with
    index i reads byte i//2, the high nibble when i is even, sign-extended."""
    codes = np.empty(n, np.int32)
    for i in range(n):
        byte = int(packed[i // 2])
        nib = (byte >> 4) & 0xF if i % 2 == 0 else byte & 0xF
        codes[i] = nib - 16 if nib & 0x8 else nib
    return codes


def single_dequant(codes, bscale):
    """4-bit dequantisation with the unquantised fp32 block scales."""
    n = codes.size
    s = np.repeat(bscale, 64)[:n]
    return (codes.astype(np.float32) * s).astype(np.float32)


def sizes(n):
    nb = (n + 63) // 64
    return (n + 1) // 2, nb, (nb + 255) // 256


def test_memory_per_64_values():
    c = DQ["memory_per_64"]
    data, s1, s2, share = (float(c[k]) for k in ("data", "single_scale", "double_scale", "super_share"))
    assert (data + s1) * 8 / 64 == 4.5
    assert round((data + s2 + share) * 8 / 64, 2) == 4.13
    assert share == 4 / 256


def test_small_input(orc):
    c = DQ["small_input"]
    x = np.array([float(v) for v in c["values"].split(",")], np.float32)
    r = orc.q4dq_quantize(x)
    assert r["qscale"].size == int(c["num_blocks"]) and r["super"].size == int(c["super_scales"])
    out = orc.q4dq_dequantize(r["packed"], r["qscale"], r["super"], x.size)
    assert out.size == int(c["len"])
    # only block: its scale is the super-block maximum, so the u8 code is 255 and the
    # reconstructed scale equals the fp32 scale exactly
    assert r["qscale"][0] == 255 and r["super"][0] == r["block_scale"][0]
    np.testing.assert_array_equal(out, r["recon"])


def test_zeros_and_length(orc):
    z = DQ["zeros"]
    r = orc.q4dq_quantize(np.zeros(int(z["n"]), np.float32))
    assert np.all(np.abs(r["recon"]) < float(z["tol"]))
    assert not r["packed"].any() and not r["qscale"].any()
    assert r["super"][0] == np.float32(1e-8)  # the page's floor on the super-scale
    L = DQ["length"]
    n = int(L["n"])
    x = (np.arange(n) * float(L["step"])).astype(np.float32)
    r = orc.q4dq_quantize(x)
    assert r["recon"].size == n and r["packed"].size == 100 and r["qscale"].size == 4


def test_within_one_percent_of_single(orc):
    c = DQ["within_1pct"]
    n = int(c["n"])
    x = (np.sin(np.arange(n, dtype=np.float32) * np.float32(float(c["freq"]))) * np.float32(float(c["amp"]))).astype(np.float32)
    r = orc.q4dq_quantize(x)
    codes = unpack_page_decoder(r["packed"], n)
    single = single_dequant(codes, r["block_scale"])
    double = orc.q4dq_dequantize(r["packed"], r["qscale"], r["super"], n)
    np.testing.assert_array_equal(double, r["recon"])
    assert np.all(np.abs(single - double) <= np.abs(single) * float(c["rel"]) + float(c["abs"]))


def test_memory_savings_and_ratio(orc):
    c = DQ["savings"]
    n = int(c["n"])
    x = np.sin(np.arange(n, dtype=np.float32) * np.float32(float(c["freq"]))).astype(np.float32)
    r = orc.q4dq_quantize(x)
    npk, nb, ns = sizes(n)
    assert (r["packed"].size, r["qscale"].size, r["super"].size) == (npk, nb, ns)
    single_bytes = npk + 4 * nb
    double_bytes = npk + nb + 4 * ns
    assert double_bytes < single_bytes
    savings = 4 * nb - (nb + 4 * ns)
    assert savings * 8 / n > float(c["min_bits"])
    assert (4 * n) / double_bytes > (4 * n) / single_bytes


def test_scale_reconstruction_accuracy(orc):
    c = DQ["scale_recon"]
    n = int(c["n"])
    x = (np.sin(np.arange(n, dtype=np.float32) * np.float32(float(c["freq"]))) * np.float32(float(c["amp"]))).astype(np.float32)
    r = orc.q4dq_quantize(x)
    bs = r["block_scale"]
    recon_s = (r["qscale"].astype(np.float32) / np.float32(255) * r["super"][np.arange(bs.size) // 256]).astype(np.float32)
    assert np.all(np.abs(bs - recon_s) <= np.abs(bs) * float(c["rel"]) + float(c["abs"]))


@pytest.mark.parametrize("mag", [0.1, 1.7, 9.9])
@pytest.mark.parametrize("n", [64, 320, 960])
def test_property_within_one_percent(orc, n, mag):
    x = (np.sin(np.arange(n, dtype=np.float32) * np.float32(0.1)) * np.float32(mag)).astype(np.float32)
    r = orc.q4dq_quantize(x)
    single = single_dequant(unpack_page_decoder(r["packed"], n), r["block_scale"])
    assert np.all(np.abs(single - r["recon"]) <= np.abs(single) * 0.01 + 1e-5)


def test_first_level_brute_force_and_double_quant_closed_forms(orc):
    """Student-t blocks, ragged length: each code is the nearest integer in [-7, 7] to
    fl(x / s_b) with ties to even; s_b = fl(absmax_b / 7); the super-scale is the
    group maximum (floored at 1e-8); the u8 scale is the half-away rounding of
    fl(fl(s_b / S) * 255); the largest block of a group gets 255 and its scale back
    exactly; every reconstructed scale is within S/510 (+ rounding) of s_b."""
    rng = np.random.default_rng(11)
    n = 64 * 256 * 2 + 64 * 37 + 13  # two full super-blocks, a partial one, a ragged block
    x = (rng.standard_t(4, n) * 0.02).astype(np.float32)
    x[64 * 5: 64 * 6] = 0.0  # an all-zero block
    r = orc.q4dq_quantize(x)
    codes = unpack_page_decoder(r["packed"], n)
    npk, nb, ns = sizes(n)
    assert r["block_scale"].size == nb and r["super"].size == ns
    for b in range(nb):
        blk = x[b * 64:(b + 1) * 64]
        sb = np.float32(np.abs(blk).max() / np.float32(7))
        assert r["block_scale"][b] == sb
        if sb == 0:
            assert not codes[b * 64:(b + 1) * 64].any()
            continue
        t = (blk / sb).astype(np.float32).astype(np.float64)
        fl = np.floor(t)
        frac = t - fl
        want = np.where(frac > 0.5, fl + 1, np.where(frac < 0.5, fl, np.where(fl % 2 == 0, fl, fl + 1)))
        want = np.clip(want, -7, 7)
        np.testing.assert_array_equal(codes[b * 64:b * 64 + blk.size], want.astype(np.int32))
    for k in range(ns):
        grp = r["block_scale"][k * 256:(k + 1) * 256]
        S = max(np.float32(grp.max()), np.float32(1e-8))
        assert r["super"][k] == S
        norm = (grp / S).astype(np.float32) * np.float32(255)
        half_away = np.sign(norm) * np.floor(np.abs(norm.astype(np.float64)) + 0.5)
        np.testing.assert_array_equal(r["qscale"][k * 256:(k + 1) * 256], np.clip(half_away, 0, 255).astype(np.uint8))
        top = int(np.argmax(grp))
        assert r["qscale"][k * 256 + top] == 255
        rec = (r["qscale"][k * 256:(k + 1) * 256].astype(np.float32) / np.float32(255) * S).astype(np.float32)
        assert rec[top] == grp[top]
        assert np.all(np.abs(rec - grp) <= S / 510 * (1 + 2 ** -20) + S * 2 ** -22)
    # nibbles outside the tensor stay zero (odd length: low nibble of the last byte)
    assert r["packed"][-1] & 0xF == 0


def test_mx_page_examples(orc):
    """E8M0 scale rule: amax = 300 -> frexp exponent 9 -> X = 2^(9 - 1 - 8) = 1, byte 127;
    amax = 0 -> treated as 1 -> X = 2^-8; block max / X in [256, 512); above 448 clips."""
    emax = int(MX["emax_e4m3"]["value"])
    lo, hi, clip = (float(MX["block_max_range"][k]) for k in ("lo", "hi", "clip"))
    blk = int(MX["block_size"]["value"])
    x = np.zeros((1, 2 * blk), np.float32)
    x[0, 0] = 300.0
    x[0, 1] = -1.0
    r = orc.mxfp8_rows(x, dtype=0)
    m, k = math.frexp(300.0)
    assert k == 9 and r["e8m0"][0, 0] == k - 1 - emax + 127
    assert r["fq"][0, 0] == 288.0  # 300 on the E4M3 grid (step 32 in [256, 512))
    assert r["e8m0"][0, 1] == -emax + 127  # all-zero block
    rng = np.random.default_rng(5)
    y = (rng.standard_t(5, (64, 256)) * 0.02).astype(np.float32)
    r = orc.mxfp8_rows(y, dtype=0)
    X = np.ldexp(np.float32(1), r["e8m0"].astype(np.int32) - 127).astype(np.float64)
    bm = np.abs(y.reshape(64, 8, 32)).max(axis=2)
    ratio = bm / X
    assert np.all((ratio >= lo) & (ratio < hi))
    deq = np.abs(r["fq"]).reshape(64, 8, 32).max(axis=2) / X
    assert np.all(deq <= clip)
    over = ratio > clip + 16  # strictly beyond the round-to-448 midpoint 464
    assert np.all(deq[over] == clip)


def test_tie_rules(orc):
    """Ties: a 4-bit code at an exact .5 quotient goes to the even integer (the
    page's nearest mode is ties-to-even); a u8 scale code at an exact .5 goes away
    from zero (the page rounds it with f32::round)."""
    x = np.zeros(128, np.float32)
    x[0] = 7.0   # block 0: s = 1, the super-block maximum
    x[1] = 2.5   # quotient 2.5 -> code 2
    x[2] = -3.5  # quotient -3.5 -> code -4
    # block 1: absmax a with fl(a / 7) = s1 and fl(fl(s1 / 1) * 255) = 2.5 exactly
    s1 = np.float32(2.5) / np.float32(255)
    while True:
        a = np.float32(s1 * np.float32(7))
        if np.float32(a / np.float32(7)) == s1 and np.float32(s1 * np.float32(255)) == np.float32(2.5):
            break
        s1 = np.nextafter(s1, np.float32(1))
    x[64] = a
    r = orc.q4dq_quantize(x)
    codes = unpack_page_decoder(r["packed"], 128)
    assert codes[:3].tolist() == [7, 2, -4]
    assert r["block_scale"][1] == s1 and r["super"][0] == 1.0
    assert r["qscale"].tolist() == [255, 3]
