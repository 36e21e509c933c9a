"""GPU parity of percentile calibration ([QAT] QuantParams::per_tensor_percentile)
against the oracle: scale, zero-point, real bounds and flags bit for bit, for
every width / scheme, clip fractions from 0 to just under 1/2, sizes from one
element through several histogram workgroups and a ragged tail to the 2^24
weight and 2^26 fp8 workloads, and the cases that stress the selection: ties
across the selected rank, signed zeros, subnormals, values at the binary32
limits, one-sided data, non-finite elements (none finite at all included), an
unaligned view, and a workspace reused dirty between calls.
"""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, to_np

pytestmark = pytest.mark.gpu

CFS = [0.0, 1e-4, 0.001, 0.01, 0.1, 0.25, 0.49999]


def check(fq, orc, x_t, bits, scheme, cf, what="", ws=None):
    n = x_t.numel()
    log(f"percentile case {what} n={n} bits={bits} scheme={scheme} cf={cf}")
    if ws is None:
        params, flags = fq.params_percentile(x_t, cf, bits, scheme)
    else:
        wsb = ws.numel() * ws.element_size()
        params = torch.empty(4, dtype=torch.int32, device=x_t.device)
        flags = torch.zeros(1, dtype=torch.int32, device=x_t.device)
        fq.fq_tensor_params_percentile(x_t, n, bits, scheme, cf, ws, wsb, params, flags)
    torch.cuda.synchronize()
    ref = orc.percentile_params(to_np(x_t), bits, scheme, cf)
    s, zp, lo, hi = fq.params_fields(params)
    assert_bits(np.float32([s, lo, hi]), np.float32([ref["scale"], ref["lo"], ref["hi"]]), what + " params")
    assert zp == ref["zp"], what
    assert int(flags.item()) == ref["flags"], what
    return ref


def test_page_outlier(fqlib, orc):
    v = np.concatenate([np.arange(100) / 100.0, [1000.0]]).astype(np.float32)
    x = torch.from_numpy(v).cuda()
    ref = check(fqlib, orc, x, 8, 0, 0.02, "page outlier")
    assert ref["sel_max"] == np.float32(0.98)


@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 0), (4, 1)])
@pytest.mark.parametrize("cf", CFS)
def test_tensor_workload(fqlib, orc, bits, scheme, cf):
    x, _ = synthetic.tensor_inputs(device="cuda")
    check(fqlib, orc, x, bits, scheme, cf, "tensor 2^20")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 63, 255, 1023, 1024, 1025, 4097, 65539, (1 << 20) + 3])
def test_sizes(fqlib, orc, n):
    rng = np.random.default_rng(n)
    v = (rng.standard_t(3, n) * 0.3 + 0.05).astype(np.float32)
    x = torch.from_numpy(v).cuda()
    for cf, scheme in ((0.0, 0), (0.01, 1), (0.2, 1), (0.49999, 0)):
        check(fqlib, orc, x, 8, scheme, cf, f"n={n}")


def test_weight_full_size(fqlib, orc):
    w = synthetic.rows_f32_inputs(device="cuda").reshape(-1)
    for cf, scheme in ((0.001, 1), (0.01, 0)):
        check(fqlib, orc, w, 8, scheme, cf, "weights 2^24")


def test_fp8_workload_with_specials(fqlib, orc):
    # the 2^26 fp8 workload carries NaN / +-Inf / huge / subnormal elements
    x = synthetic.fp8_inputs(device="cuda")
    check(fqlib, orc, x, 8, 1, 0.001, "fp8 2^26")


def test_ties_and_special_values(fqlib, orc):
    rng = np.random.default_rng(11)
    cases = {
        "all equal": np.full(5000, 0.75, np.float32),
        "few levels": rng.integers(-3, 4, 100000).astype(np.float32) * 0.5,
        "signed zeros": np.where(rng.random(3001) < 0.5, -0.0, 0.0).astype(np.float32),
        "zeros and one": np.concatenate([np.zeros(999, np.float32), np.float32([-0.0, 1.0])]),
        "subnormals": (rng.standard_normal(7000) * 1e-40).astype(np.float32),
        "binary32 limits": np.float32([3.4028235e38, -3.4028235e38, 1e-45, -1e-45] * 300
                                      + list(rng.standard_normal(800))),
        "negative only": -np.abs(rng.standard_normal(9001)).astype(np.float32) - 1.0,
        "positive only": np.abs(rng.standard_normal(9001)).astype(np.float32) + 2.0,
        "near ties": (1.0 + np.arange(4096, dtype=np.float32) * np.float32(2 ** -23)).astype(np.float32),
    }
    for name, v in cases.items():
        x = torch.from_numpy(np.ascontiguousarray(v)).cuda()
        for cf in (0.0, 0.001, 0.1, 0.3):
            for bits, scheme in ((8, 0), (4, 1)):
                check(fqlib, orc, x, bits, scheme, cf, name)


def test_nonfinite(fqlib, orc):
    rng = np.random.default_rng(12)
    v = rng.standard_normal(20011).astype(np.float32)
    v[::97] = np.nan
    v[5::101] = np.inf
    v[7::103] = -np.inf
    x = torch.from_numpy(v).cuda()
    for cf in (0.0, 0.05):
        check(fqlib, orc, x, 8, 1, cf, "mixed non-finite")
    for name, w in (("all NaN", np.full(777, np.nan, np.float32)),
                    ("only infinities", np.float32([np.inf, -np.inf] * 50)),
                    ("one finite", np.float32([np.nan] * 40 + [-2.5] + [np.inf] * 40))):
        check(fqlib, orc, torch.from_numpy(w).cuda(), 8, 0, 0.1, name)
        check(fqlib, orc, torch.from_numpy(w).cuda(), 4, 1, 0.0, name)


def test_unaligned_view_and_dirty_workspace(fqlib, orc):
    rng = np.random.default_rng(13)
    base = torch.from_numpy(rng.standard_normal(50003).astype(np.float32)).cuda()
    wsb = fqlib.fq_percentile_workspace_bytes(50003)
    ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device="cuda")
    for off, n in ((1, 50001), (3, 49999), (0, 50003), (2, 7)):
        check(fqlib, orc, base[off:off + n], 8, 1, 0.01, f"view +{off}", ws=ws)
    # a second, smaller call on the workspace the larger one left behind
    check(fqlib, orc, base[:100], 4, 0, 0.1, "reuse smaller", ws=ws)


def test_candidate_slice_overflow(fqlib, orc):
    # 2^20 elements: 2^18 16-byte chunks over 128 histogram workgroups of 1024
    # threads, chunk c taken by thread c mod 131072, so workgroup 0 owns the chunks
    # with c mod 131072 < 1024.  Filling those with c mod 131072 < 256 with the
    # tensor's top value sends 2048 keys into workgroup 0's candidate slice (room
    # for 576, about 1 in 16 of its share) while the other slices stay small: the
    # third pass must fall back to x.
    n = 1 << 20
    v = (np.random.default_rng(14).standard_normal(n) * 0.1).astype(np.float32)
    chunks = v.reshape(-1, 4)
    chunks[(np.arange(chunks.shape[0]) % 131072) < 256] = 1.0
    x = torch.from_numpy(v).cuda()
    for cf, scheme in ((0.001, 1), (0.0001, 0), (0.01, 1)):
        check(fqlib, orc, x, 8, scheme, cf, "one slice overflows")


def test_many_candidates_per_slice(fqlib, orc):
    # values +-2^e (1 + u / 8) for 32 exponents e: each sign and exponent is one
    # 11-bit prefix, so the two selected prefixes hold 1/32 of the elements, about
    # 256 keys in each workgroup's candidate slice at 2^20 elements (many
    # candidates, but fewer than a slice holds, 576)
    n = 1 << 20
    rng = np.random.default_rng(21)
    e = rng.integers(0, 32, n).astype(np.float64)
    v = (np.exp2(e) * (1.0 + rng.random(n) / 8.0)).astype(np.float32)
    v[rng.random(n) < 0.5] *= -1.0
    x = torch.from_numpy(v).cuda()
    for bits, scheme, cf in ((8, 1, 0.001), (4, 0, 0.01), (8, 0, 0.3)):
        check(fqlib, orc, x, bits, scheme, cf, "many candidates per slice")


def test_selected_bins_of_known_size(fqlib, orc):
    # ranks lo and hi (cf 0.25) inside prefixes of exactly 128 keys in every
    # workgroup's share: per 8192-element share of the 128 histogram workgroups at
    # 2^20 elements (chunk c in workgroup (c mod 131072) / 1024), 2000 values in
    # [0.5, 0.75), 64 in [1, 1.25) (the bin of rank lo), 4064 in [2, 2.5), 64 in
    # [4, 5) (the bin of rank hi) and 2000 in [8, 10), so every candidate slice
    # holds exactly 128 keys
    n = 1 << 20
    rng = np.random.default_rng(22)
    wg = ((np.arange(n) // 4) % 131072) // 1024
    v = np.empty(n, np.float32)
    parts = ((2000, 0.5, 0.75), (64, 1.0, 1.25), (4064, 2.0, 2.5), (64, 4.0, 5.0), (2000, 8.0, 10.0))
    for b in range(128):
        idx = rng.permutation(np.flatnonzero(wg == b))
        k = 0
        for cnt, lo, hi in parts:
            v[idx[k:k + cnt]] = rng.uniform(lo, hi, cnt).astype(np.float32)
            k += cnt
        assert k == idx.size
    x = torch.from_numpy(v).cuda()
    ref = check(fqlib, orc, x, 8, 1, 0.25, "selected bins of known size")
    assert 1.0 <= ref["sel_min"] < 1.25 and 4.0 <= ref["sel_max"] < 5.0


# From 2^23 elements on, a sample of x (runs of 16 values from each multiple of
# n / 256) predicts the first-digit bins of both statistics, the first pass
# keeps the keys of those bins, and the second pass counts them instead of x.
# Each case below takes one branch of that path and is checked against the
# oracle like every other.
PRED_N = 1 << 23


def test_prediction_hits(fqlib, orc):
    rng = np.random.default_rng(31)
    v = (rng.standard_normal(PRED_N) * 0.05).astype(np.float32)
    x = torch.from_numpy(v).cuda()
    for bits, scheme, cf in ((8, 1, 0.001), (4, 0, 0.02)):
        check(fqlib, orc, x, bits, scheme, cf, "predicted bins hit")
    # the unaligned form of the passes
    check(fqlib, orc, x[1:], 8, 1, 0.001, "predicted bins hit, view +1")


def test_prediction_misses(fqlib, orc):
    # cf 0 (the minimum and maximum): the extremes of x lie beyond those of the
    # sample, outside the predicted bins
    rng = np.random.default_rng(31)
    v = (rng.standard_normal(PRED_N) * 0.05).astype(np.float32)
    check(fqlib, orc, torch.from_numpy(v).cuda(), 4, 0, 0.0, "extremes beyond the sample")
    # runs of 16 values from each multiple of n / 1024 (the sampled runs among
    # them) are drawn twice as wide as the rest, so the predicted tail bins lie an
    # octave out: the second pass must go back to x
    rng = np.random.default_rng(32)
    v = (rng.standard_normal(PRED_N) * 0.1).astype(np.float32)
    runs = v.reshape(1024, -1)
    runs[:, :16] = (rng.standard_normal((1024, 16)) * 0.2).astype(np.float32)
    x = torch.from_numpy(v).cuda()
    for bits, scheme, cf in ((8, 1, 0.001), (8, 0, 0.005)):
        check(fqlib, orc, x, bits, scheme, cf, "predicted bins miss")


def test_prediction_slice_overflow(fqlib, orc):
    # sorted values: the keys of the predicted lower-tail bins all fall in the
    # first chunks, so a few waves get far more than their sub-slices hold
    rng = np.random.default_rng(33)
    v = np.sort(rng.standard_normal(PRED_N).astype(np.float32))
    x = torch.from_numpy(v).cuda()
    for bits, scheme, cf in ((8, 1, 0.001), (4, 1, 0.01)):
        check(fqlib, orc, x, bits, scheme, cf, "predicted keys overflow a sub-slice")


def test_no_prediction(fqlib, orc):
    rng = np.random.default_rng(34)
    # half the values tie at zero, where the lower statistic lies: its bin holds
    # far more than 1 in 32 sampled values, so nothing is predicted
    relu = np.maximum(rng.standard_normal(PRED_N), 0.0).astype(np.float32)
    check(fqlib, orc, torch.from_numpy(relu).cuda(), 8, 1, 0.001, "tie at the lower statistic")
    # cf 0.3 of a normal tensor: the widened rank windows span heavy bins
    v = rng.standard_normal(PRED_N).astype(np.float32)
    check(fqlib, orc, torch.from_numpy(v).cuda(), 8, 0, 0.3, "heavy predicted bins")
