"""GPU parity past 2^31 elements: every entry point on one input of
2^31 + 2^20 + 4099 float32 values (8.6 GB), so that element, byte and block
indices cross 2^31 and every block size (4, 16, 32, 64, 16384) leaves a ragged
tail.

The input is the 4-bit workload's Student-t(4) x 0.02 draw, clamped to +-100,
with planted values: the finite maximum 1000 just past 2^31, the finite minimum
-700 two elements before the end, and a NaN and a -Inf past 2^31.  The per-tensor
reductions are then checked through a property that holds at any size: their
result depends only on the finite extremes, so the oracle run on the planted
values alone gives the expected parameters and scales (for the QAT step, on a
sample that holds them: one update cannot move another element past them).  Element-wise outputs are
compared with the oracle on sampled indices (both ends, around 2^31, the planted
elements, random ones); block outputs on sampled whole blocks (whole super-blocks
for the double quantization, whole rows for the row and group paths, whole
columns for the column path).  Percentile calibration runs on a multiset whose
order statistics have a closed form (every integer in [-2^23, 2^23) repeated), once
with few candidates and once with a candidate overflow.
"""
import math

import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu

B31 = 1 << 31
N = B31 + (1 << 20) + 4099
I_MAX, I_MIN, I_NAN, I_NINF = B31 + 3, N - 2, B31 + 77, B31 + 5000
PLANTED = {I_MAX: 1000.0, I_MIN: -700.0, I_NAN: float("nan"), I_NINF: float("-inf")}
ROWS, COLS = 65440, 32832  # rows x cols = 2^31 + 1042432, row 65408 straddles 2^31
E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < (80 << 30):
        pytest.skip(f"needs 80 GiB of free device memory, {free >> 30} GiB free")
    log(f"large input: n={N} float32 ({4 * N / 2**30:.1f} GiB)")
    x = synthetic.q4dq_inputs(N, device="cuda", seed=31)
    x.clamp_(-100.0, 100.0)
    for i, v in PLANTED.items():
        x[i] = v
    torch.cuda.synchronize()
    yield x
    del x
    torch.cuda.empty_cache()


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sample_indices(seed=0, k=3000):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 3, 4, 5, B31 - 3, B31 - 2, B31 - 1, B31, B31 + 1, B31 + 2, N - 5, N - 4, N - 3, N - 2, N - 1]
    return np.unique(np.concatenate([fixed, list(PLANTED), rng.integers(0, N, k)])).astype(np.int64)


def gather(t, idx):
    return to_np(t.reshape(-1).index_select(0, torch.from_numpy(idx).to(t.device)))


def nibble(byte, i):
    """4-bit code of flat element i from its byte i / 2 (even i: the high nibble)."""
    return np.where(i % 2 == 0, byte >> 4, byte & 0xF)


def runs(starts, length=64):
    return [(s, min(s + length, N)) for s in starts]


def test_tensor_int_past_2_31(fqlib, orc, big):
    idx = sample_indices(1)
    xs = gather(big, idx)
    extremes = np.float32(list(PLANTED.values()))
    for bits, scheme in ((8, 1), (4, 0)):
        log(f"large tensor int bits={bits} scheme={scheme}")
        params, flags = fqlib.params_int(big, bits, scheme)
        ref = orc.tensor_params_int(extremes, bits, scheme)
        s, zp, lo, hi = fqlib.params_fields(params)
        assert_bits(np.float32([s, lo, hi]), np.float32([ref["scale"], ref["lo"], ref["hi"]]), "params")
        assert zp == ref["zp"] and int(flags.item()) == ref["flags"]
        codes, fq = fqlib.fake_quant_int_tensor(big, params, bits, scheme)
        rc, rf = orc.fake_quant_int(xs, bits, scheme, ref["scale"], ref["zp"])
        if bits == 8:
            assert_bits(gather(codes, idx), rc, "int8 codes")
        else:
            got = nibble(gather(codes, idx // 2).astype(np.uint8), idx)
            assert_bits(got.astype(np.uint8), (rc.astype(np.uint8) & 0xF), "int4 codes")
        assert_f32(gather(fq, idx), rf, f"int{bits} fake-quant")
        del fq
        deq = fqlib.dequantize_int_tensor(codes, N, params, bits)
        assert_f32(gather(deq, idx), orc.dequantize_int(rc, ref["scale"], ref["zp"]), f"int{bits} dequantize")
        del deq, codes
    # stochastic rounding on contiguous runs (the counter is the element index)
    params, _ = fqlib.params_int(big, 8, 1)
    ref = orc.tensor_params_int(extremes, 8, 1)
    codes, _ = fqlib.fake_quant_int_tensor_sr(big, params, seed=99, bits=8, scheme=1, want_fq=False)
    for a, b in runs([0, B31 - 40, I_NAN - 10, N - 61]):
        rc, _ = orc.fake_quant_int_sr(to_np(big[a:b]), 8, 1, ref["scale"], ref["zp"], seed=99, offset=a)
        assert_bits(to_np(codes[a:b]), rc, f"int8 stochastic codes [{a}, {b})")
    del codes
    # straight-through backward with the calibrated range (x doubles as the gradient)
    out = fqlib.ste_backward(big, big, torch.tensor([ref["lo"], ref["hi"]], dtype=torch.float32, device="cuda"))
    assert_f32(gather(out, idx), orc.ste_backward(xs, xs, ref["lo"], ref["hi"]), "STE backward")


def test_fp8_past_2_31(fqlib, orc, big):
    idx = sample_indices(2)
    xs = gather(big, idx)
    log("large fp8 scale / quantize / dequantize / stochastic")
    s, flags = fqlib.fp8_tensor_scale(big)
    amax = orc.amax_finite(np.float32(list(PLANTED.values())))
    assert amax == np.float32(1000.0)
    want = np.float32([orc.fp8_scale(amax, E4M3)[0], orc.fp8_scale(amax, E5M2)[0]])
    assert_bits(to_np(s), want, "fp8 tensor scales")
    for fmt in (E4M3, E5M2):
        q, fq = fqlib.fp8_quantize(big, fmt, s[fmt:fmt + 1])
        rq, rf = orc.fp8_quantize(xs, fmt, want[fmt])
        assert_bits(gather(q, idx), rq, f"fp8 {fmt} codes")
        assert_f32(gather(fq, idx), rf, f"fp8 {fmt} fake-quant")
        del fq
        out = fqlib.fp8_dequantize(q, fmt, s[fmt:fmt + 1])
        assert_f32(gather(out, idx), orc.fp8_dequantize(rq, fmt, want[fmt]), f"fp8 {fmt} dequantize")
        del out, q
    q, _ = fqlib.fp8_quantize_sr(big, E5M2, s[1:2], seed=7, want_fq=False)
    for a, b in runs([0, B31 - 40, I_NINF - 20, N - 61]):
        rq, _ = orc.fp8_quantize_sr(to_np(big[a:b]), E5M2, want[1], seed=7, offset=a)
        assert_bits(to_np(q[a:b]), rq, f"fp8 stochastic codes [{a}, {b})")


def test_q4dq_past_2_31(fqlib, orc, big):
    log("large 4-bit double quantization")
    r = fqlib.q4dq_quantize(big)
    torch.cuda.synchronize()
    nsb = (N + 16383) // 16384
    rng = np.random.default_rng(3)
    sbs = sorted({0, 1, B31 // 16384 - 1, B31 // 16384, I_NAN // 16384, I_NINF // 16384, I_MIN // 16384,
                  nsb - 2, nsb - 1, *rng.integers(0, nsb, 6).tolist()})
    assert int(r["flags"].item()) & fqlib.FLAG_NONFINITE, "NaN / Inf must raise the non-finite flag"
    out = fqlib.q4dq_dequantize(r["packed"], r["qscale"], r["super"], N)
    torch.cuda.synchronize()
    for sb in sbs:
        a, b = sb * 16384, min((sb + 1) * 16384, N)
        ref = orc.q4dq_quantize(to_np(big[a:b]))
        nb = (b - a + 63) // 64
        what = f"super-block {sb} [{a}, {b})"
        assert_bits(to_np(r["packed"][a // 2:(b + 1) // 2]), ref["packed"], what + " packed")
        assert_bits(to_np(r["qscale"][sb * 256:sb * 256 + nb]), ref["qscale"], what + " u8 scales")
        assert_bits(to_np(r["super"][sb:sb + 1]), ref["super"], what + " super-scale")
        assert_bits(to_np(r["block_scale"][sb * 256:sb * 256 + nb]), ref["block_scale"], what + " block scales")
        assert_f32(to_np(r["recon"][a:b]), ref["recon"], what + " reconstruction")
        assert_f32(to_np(out[a:b]), ref["recon"], what + " dequantize")


def test_nvfp4_past_2_31(fqlib, orc, big):
    log("large NVFP4")
    r = fqlib.nvfp4(big)
    torch.cuda.synchronize()
    nb = (N + 15) // 16
    rng = np.random.default_rng(4)
    # the block holding the tensor maximum first (it fixes the tensor scale), the
    # short last block last, so every other block keeps its alignment
    mid = sorted({0, B31 // 16 - 1, B31 // 16, I_NAN // 16, I_NINF // 16, *rng.integers(0, nb - 1, 8).tolist()}
                 - {I_MAX // 16, nb - 1})
    blocks = [I_MAX // 16] + mid + [nb - 1]
    xs = np.concatenate([to_np(big[b * 16:min(b * 16 + 16, N)]) for b in blocks])
    ref = orc.nvfp4(xs)
    assert_bits(to_np(r["g"]), np.float32([ref["g"]]), "tensor scale")
    got_q = np.concatenate([to_np(r["q"][b * 8:min(b * 8 + 8, (N + 1) // 2)]) for b in blocks])
    got_s = np.concatenate([to_np(r["scales"][b:b + 1]) for b in blocks])
    got_f = np.concatenate([to_np(r["fq"][b * 16:min(b * 16 + 16, N)]) for b in blocks])
    assert_bits(got_q, ref["q"], "E2M1 codes")
    assert_bits(got_s, ref["sbytes"], "E4M3 block scales")
    assert_f32(got_f, ref["fq"], "fake-quant")


def sorted_value(k):
    """Value of rank k of the multiset: integers [-2^23, 2^23) each repeated N // 2^24
    times, the first N mod 2^24 of them once more."""
    m = 1 << 24
    rep, extra = divmod(N, m)
    j = k // (rep + 1) if k < (rep + 1) * extra else extra + (k - (rep + 1) * extra) // rep
    return float(j - (1 << 23))


@pytest.mark.parametrize("cf,bits,scheme", [(0.45, 8, 1), (0.001, 4, 0)])
def test_percentile_past_2_31(fqlib, orc, big, cf, bits, scheme):
    # 0.45: about 1.6 % of the values share a prefix with a selected one (the
    # candidate slices hold them); 0.001: about 12.5 % do, and the slices overflow
    log(f"large percentile cf={cf}")
    m = 1 << 24
    base = torch.arange(m, dtype=torch.float32, device="cuda") - float(1 << 23)
    x = base.repeat(N // m + 1)[:N]
    params, flags = fqlib.params_percentile(x, cf, bits, scheme)
    last = N - 1
    lo, hi = math.floor(cf * last), math.ceil((1.0 - cf) * last)
    s_want, zp_want, f_want = orc.params_from_minmax(sorted_value(lo), sorted_value(hi), bits, scheme)
    s, zp, _, _ = fqlib.params_fields(params)
    assert_bits(np.float32([s]), np.float32([s_want]), "percentile scale")
    assert zp == zp_want and int(flags.item()) == f_want


def sample_rows(rng):
    return np.unique(np.concatenate([[0, 1, 65407, 65408, 65409, ROWS - 1], rng.integers(0, ROWS, 6)]))


def test_rows_groups_mx_past_2_31(fqlib, orc, big):
    x2 = big[:ROWS * COLS].view(ROWS, COLS)
    rows = sample_rows(np.random.default_rng(5))
    rt = torch.from_numpy(rows).cuda()
    xs = to_np(x2.index_select(0, rt))
    for bits, scheme in ((8, 1), (4, 0)):
        log(f"large rows f32 bits={bits} scheme={scheme}")
        r = fqlib.quant_rows(x2, bits, scheme)
        ref = orc.quant_rows(xs, bits, scheme)
        assert_bits(to_np(r["codes"].index_select(0, rt)), ref["codes"], "row codes")
        assert_bits(to_np(r["scale"])[rows], ref["scale"], "row scales")
        assert_bits(to_np(r["zp"])[rows], ref["zp"], "row zero-points")
        assert_f32(to_np(r["fq"].index_select(0, rt)), ref["fq"], "row fake-quant")
        del r
    for group, bits, scheme in ((128, 4, 1), (32, 8, 0)):
        log(f"large groups f32 group={group} bits={bits}")
        r = fqlib.quant_groups(x2, group, bits, scheme)
        ref = orc.quant_groups(xs, group, bits, scheme)
        assert_bits(to_np(r["codes"].index_select(0, rt)), ref["codes"], "group codes")
        assert_bits(to_np(r["scale"].index_select(0, rt)), ref["scale"], "group scales")
        assert_bits(to_np(r["zp"].index_select(0, rt)), ref["zp"], "group zero-points")
        assert_f32(to_np(r["fq"].index_select(0, rt)), ref["fq"], "group fake-quant")
        del r
    for elem in (fqlib.E2M1, fqlib.E4M3):
        log(f"large MX rows f32 elem={elem}")
        r = fqlib.mx_rows(x2, elem)
        ref = orc.mx_rows(xs, elem) if elem != fqlib.E4M3 else orc.mxfp8_rows(xs, dtype=0)
        assert_bits(to_np(r["q"].index_select(0, rt)), ref["q"], "MX codes")
        assert_bits(to_np(r["e8m0"].index_select(0, rt)), ref["e8m0"], "E8M0 scales")
        assert_f32(to_np(r["fq"].index_select(0, rt)), ref["fq"], "MX fake-quant")
        del r


def test_bf16_rows_past_2_31(fqlib, orc, big):
    xb = big[:ROWS * COLS].view(ROWS, COLS).to(torch.bfloat16)
    rows = sample_rows(np.random.default_rng(6))
    rt = torch.from_numpy(rows).cuda()
    xs = to_np(xb.index_select(0, rt)).view(np.uint16)
    log("large rows bf16 per-token int8 affine")
    r = fqlib.quant_rows(xb, 8, 1, want_fq=False)
    ref = orc.quant_rows(xs, 8, 1, dtype=1, want_fq=False)
    assert_bits(to_np(r["codes"].index_select(0, rt)), ref["codes"], "bf16 row codes")
    assert_bits(to_np(r["scale"])[rows], ref["scale"], "bf16 row scales")
    del r
    log("large groups bf16 group=128 int8")
    r = fqlib.quant_groups(xb, 128, 8, 0)
    ref = orc.quant_groups(xs, 128, 8, 0, dtype=1)
    assert_bits(to_np(r["codes"].index_select(0, rt)), ref["codes"], "bf16 group codes")
    assert_f32(to_np(r["fq"].index_select(0, rt)), ref["fq"], "bf16 group fake-quant")
    del r
    log("large MXFP8 bf16")
    r = fqlib.mxfp8_rows(xb)
    ref = orc.mxfp8_rows(xs, dtype=1)
    assert_bits(to_np(r["q"].index_select(0, rt)), ref["q"], "bf16 MXFP8 codes")
    assert_bits(to_np(r["e8m0"].index_select(0, rt)), ref["e8m0"], "bf16 E8M0 scales")


def test_cols_past_2_31(fqlib, orc, big):
    x2 = big[:ROWS * COLS].view(ROWS, COLS)
    rng = np.random.default_rng(7)
    cols = np.unique(np.concatenate([[0, 1, 2, 3, COLS - 1, I_MAX % COLS, I_NAN % COLS, I_NINF % COLS],
                                     rng.integers(0, COLS, 8)]))
    ct = torch.from_numpy(cols).cuda()
    xs = np.ascontiguousarray(to_np(x2.index_select(1, ct)))
    for bits, scheme in ((8, 0), (4, 1)):
        log(f"large cols bits={bits} scheme={scheme}")
        r = fqlib.quant_cols(x2, bits, scheme)
        ref = orc.quant_cols(xs, bits, scheme)
        assert_bits(to_np(r["scale"])[cols], ref["scale"], "column scales")
        assert_bits(to_np(r["zp"])[cols], ref["zp"], "column zero-points")
        if bits == 8:
            assert_bits(to_np(r["codes"].index_select(1, ct)), ref["codes"], "column codes")
        else:
            got = to_np(r["codes"].index_select(1, torch.from_numpy(cols // 2).cuda()))
            got = np.where(cols % 2 == 0, got >> 4, got & 0xF).astype(np.uint8)
            j = np.arange(len(cols))
            want = np.where(j % 2 == 0, ref["codes"][:, j // 2] >> 4, ref["codes"][:, j // 2] & 0xF).astype(np.uint8)
            assert_bits(got, want, "column int4 codes")
        assert_f32(to_np(r["fq"].index_select(1, ct)), ref["fq"], "column fake-quant")
        del r


def test_cols_strip_past_2_31(fqlib, orc, big):
    """The one-pass per-column kernel (4096 rows, 32776 strips of 16 columns, a
    multiple of the eight XCDs) on 2^31 + 524288 elements; the planted maximum,
    NaN and -Inf sit in its last row, past 2^31."""
    rows, cols3 = 4096, 16 * 32776
    assert I_NINF < rows * cols3 <= N
    x3 = big[:rows * cols3].view(rows, cols3)
    rng = np.random.default_rng(11)
    cols = np.unique(np.concatenate([[0, 1, 15, 16, cols3 - 1, I_MAX % cols3, I_NAN % cols3, I_NINF % cols3],
                                     rng.integers(0, cols3, 8)]))
    ct = torch.from_numpy(cols).cuda()
    xs = np.ascontiguousarray(to_np(x3.index_select(1, ct)))
    for bits, scheme in ((8, 1), (4, 0)):
        log(f"large cols strip bits={bits} scheme={scheme}")
        r = fqlib.quant_cols(x3, bits, scheme)
        ref = orc.quant_cols(xs, bits, scheme)
        assert_bits(to_np(r["scale"])[cols], ref["scale"], "strip column scales")
        assert_bits(to_np(r["zp"])[cols], ref["zp"], "strip column zero-points")
        if bits == 8:
            assert_bits(to_np(r["codes"].index_select(1, ct)), ref["codes"], "strip column codes")
        else:
            got = to_np(r["codes"].index_select(1, torch.from_numpy(cols // 2).cuda()))
            got = np.where(cols % 2 == 0, got >> 4, got & 0xF).astype(np.uint8)
            j = np.arange(len(cols))
            want = np.where(j % 2 == 0, ref["codes"][:, j // 2] >> 4, ref["codes"][:, j // 2] & 0xF).astype(np.uint8)
            assert_bits(got, want, "strip column int4 codes")
        assert_f32(to_np(r["fq"].index_select(1, ct)), ref["fq"], "strip column fake-quant")
        assert int(r["flags"].item()) == ref["flags"], "strip flags"
        del r


def test_qat_past_2_31(fqlib, orc, big):
    # the update moves no element by more than about lr, so the planted extremes
    # stay the extremes of the updated master and a sample holding them calibrates
    # as the whole tensor does
    idx = sample_indices(8)
    it = torch.from_numpy(idx).cuda()
    lr, wd = 1e-3, 0.01
    cfg = fqlib.adamw_config(lr, weight_decay=wd)
    g = torch.randn(N, generator=torch.Generator(device="cuda").manual_seed(8), device="cuda")
    m = torch.zeros_like(g)
    v = torch.zeros_like(g)
    w = big.clone()
    log("large QAT step int8 affine, nearest")
    r = fqlib.qat_step_int(w, g, m, v, 1, cfg, 8, 1, fqlib.ROUND_NEAREST, 0, 0)
    torch.cuda.synchronize()
    z = np.zeros(idx.size, np.float32)
    ref = orc.qat_step_int(to_np(big.index_select(0, it)), to_np(g.index_select(0, it)), z, z, lr, 1, bits=8,
                           scheme=1, weight_decay=wd)
    assert_f32(to_np(w.index_select(0, it)), ref["w"], "QAT master")
    assert_f32(to_np(m.index_select(0, it)), ref["m"], "QAT m")
    assert_f32(to_np(v.index_select(0, it)), ref["v"], "QAT v")
    s, zp, lo, hi = fqlib.params_fields(r["params"])
    assert_bits(np.float32([s, lo, hi]), np.float32([ref["scale"], ref["lo"], ref["hi"]]), "QAT params")
    assert zp == ref["zp"] and int(r["flags"].item()) == ref["flags"]
    assert_bits(to_np(r["codes"].index_select(0, it)), ref["codes"], "QAT codes")
    assert_f32(to_np(r["view"].index_select(0, it)), ref["view"], "QAT view")
    del r
    log("large QAT step fp8 E4M3, stochastic")
    w.copy_(big)
    m.zero_()
    v.zero_()
    r = fqlib.qat_step_fp8(w, g, m, v, 1, cfg, E4M3, fqlib.ROUND_STOCHASTIC, 11, 0)
    torch.cuda.synchronize()
    for a, b in runs([0, B31 - 40, I_MAX - 10, N - 61]):
        zr = np.zeros(b - a, np.float32)
        ref = orc.qat_step_fp8(to_np(big[a:b]), to_np(g[a:b]), zr, zr, lr, 1, fmt=E4M3, rounding=1, seed=11,
                               offset=a, weight_decay=wd)
        assert_f32(to_np(w[a:b]), ref["w"], f"QAT fp8 master [{a}, {b})")
        assert_bits(to_np(r["q"][a:b]), ref["q"], f"QAT fp8 bytes [{a}, {b})")
        assert_f32(to_np(r["view"][a:b]), ref["view"], f"QAT fp8 view [{a}, {b})")
