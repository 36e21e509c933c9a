"""GPU parity of the QAT optimizer step ([QAT] QatOptimizer::step: AdamW master
update, then the requantized view) against the oracle run in lockstep: master,
moments, parameters, codes, bytes and view bit for bit after every step, for
integer and fp8 targets, nearest and stochastic rounding, with and without
decoupled weight decay, ragged sizes, unaligned views and non-finite gradients.
"""
import numpy as np
import pytest
import torch

from conftest import log
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu


def unpack_nibbles(packed, n):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(2 * p.size, np.int8)
    hi = (p >> 4).astype(np.int16)
    lo = (p & 0xF).astype(np.int16)
    out[0::2] = np.where(hi >= 8, hi - 16, hi)
    out[1::2] = np.where(lo >= 8, lo - 16, lo)
    return out[:n]


def run_int(fq, orc, w0, grads, lr, bits, scheme, rounding, wd=0.0, seed=0, offset=0, what=""):
    n = w0.size
    cfg = fq.adamw_config(lr, weight_decay=wd)
    w = torch.from_numpy(w0.copy()).cuda()
    m = torch.zeros_like(w)
    v = torch.zeros_like(w)
    ow, om, ov = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    for t, g in enumerate(grads, start=1):
        log(f"qat int {what} n={n} bits={bits} scheme={scheme} rounding={rounding} step {t}")
        r = fq.qat_step_int(w, torch.from_numpy(g).cuda(), m, v, t, cfg, bits, scheme, rounding, seed, offset)
        torch.cuda.synchronize()
        ref = orc.qat_step_int(ow, g, om, ov, lr, t, bits=bits, scheme=scheme, rounding=rounding, seed=seed,
                               offset=offset, weight_decay=wd)
        ow, om, ov = ref["w"], ref["m"], ref["v"]
        assert_f32(to_np(w), ow, f"{what} master step {t}")
        assert_f32(to_np(m), om, f"{what} m step {t}")
        assert_f32(to_np(v), ov, f"{what} v step {t}")
        s, zp, lo, hi = fq.params_fields(r["params"])
        assert_bits(np.float32([s, lo, hi]), np.float32([ref["scale"], ref["lo"], ref["hi"]]), f"{what} params")
        assert zp == ref["zp"]
        codes = to_np(r["codes"])
        codes = unpack_nibbles(codes, n) if bits == 4 else codes.view(np.int8)
        assert_bits(codes, ref["codes"], f"{what} codes step {t}")
        assert_f32(to_np(r["view"]), ref["view"], f"{what} view step {t}")
        assert int(r["flags"].item()) == ref["flags"], what


def run_fp8(fq, orc, w0, grads, lr, fmt, rounding, wd=0.0, seed=0, offset=0, what=""):
    n = w0.size
    cfg = fq.adamw_config(lr, weight_decay=wd)
    w = torch.from_numpy(w0.copy()).cuda()
    m = torch.zeros_like(w)
    v = torch.zeros_like(w)
    ow, om, ov = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    for t, g in enumerate(grads, start=1):
        log(f"qat fp8 {what} n={n} fmt={fmt} rounding={rounding} step {t}")
        r = fq.qat_step_fp8(w, torch.from_numpy(g).cuda(), m, v, t, cfg, fmt, rounding, seed, offset)
        torch.cuda.synchronize()
        ref = orc.qat_step_fp8(ow, g, om, ov, lr, t, fmt=fmt, rounding=rounding, seed=seed, offset=offset,
                               weight_decay=wd)
        ow, om, ov = ref["w"], ref["m"], ref["v"]
        assert_f32(to_np(w), ow, f"{what} master step {t}")
        assert_f32(to_np(m), om, f"{what} m step {t}")
        assert_f32(to_np(v), ov, f"{what} v step {t}")
        assert_bits(to_np(r["q"]), ref["q"], f"{what} bytes step {t}")
        assert_f32(to_np(r["view"]), ref["view"], f"{what} view step {t}")


def test_page_examples(fqlib, orc):
    run_int(fqlib, orc, np.float32([0.12, -0.37, 0.88, -0.05, 0.51]), [np.float32([0.1, -0.2, 0.05, 0.3, -0.15])],
            0.1, 8, 0, 0, what="page int8")
    run_fp8(fqlib, orc, np.float32([0.3, -1.2, 4.0, -0.01, 2.5]), [np.float32([0.2, 0.1, -0.3, 0.4, -0.05])],
            0.05, 0, 0, what="page fp8")


def grads_for(n, steps, seed):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal(n) * 0.1 / np.sqrt(t)).astype(np.float32) for t in range(1, steps + 1)]


@pytest.mark.parametrize("bits,scheme,rounding,wd", [(8, 0, 0, 0.0), (8, 1, 1, 0.01), (4, 0, 0, 0.01), (4, 1, 1, 0.0)])
def test_int_steps(fqlib, orc, bits, scheme, rounding, wd):
    n = (1 << 16) + 3
    w0 = (np.random.default_rng(1).standard_normal(n) * 0.05).astype(np.float32)
    run_int(fqlib, orc, w0, grads_for(n, 12, 2), 1e-3, bits, scheme, rounding, wd=wd, seed=99, offset=5,
            what="steps")


@pytest.mark.parametrize("fmt,rounding,wd", [(0, 0, 0.0), (0, 1, 0.02), (1, 0, 0.02), (1, 1, 0.0)])
def test_fp8_steps(fqlib, orc, fmt, rounding, wd):
    n = (1 << 16) + 1
    w0 = (np.random.default_rng(3).standard_normal(n) * 2.0).astype(np.float32)
    run_fp8(fqlib, orc, w0, grads_for(n, 12, 4), 1e-2, fmt, rounding, wd=wd, seed=7, offset=2, what="steps")


# the last size has more reduction tiles (8192 elements each) than the 2048
# partials the requantize blocks fold, so the update workgroups loop over tiles
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 1023, (1 << 22) + 5, (1 << 24) + 40 * 8192 + 7])
def test_sizes(fqlib, orc, n):
    w0 = (np.random.default_rng(n).standard_normal(n)).astype(np.float32)
    g = grads_for(n, 2, n + 1)
    run_int(fqlib, orc, w0, g, 1e-2, 8, 1, 0, what=f"n={n}")
    run_fp8(fqlib, orc, w0, g, 1e-2, 1, 1, seed=3, what=f"n={n}")


def test_nonfinite_gradients(fqlib, orc):
    n = 4099
    rng = np.random.default_rng(6)
    w0 = rng.standard_normal(n).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    g[7] = np.nan
    g[100] = np.inf
    g[2000] = -np.inf
    z = np.zeros(n, np.float32)
    run_int(fqlib, orc, w0, [g, z], 1e-2, 8, 0, 0, what="nonfinite")
    run_fp8(fqlib, orc, w0, [g, z], 1e-2, 0, 0, what="nonfinite")


def test_unaligned_views(fqlib, orc):
    n = 5000
    rng = np.random.default_rng(8)
    base = rng.standard_normal(n + 3).astype(np.float32)
    gbase = rng.standard_normal(n + 3).astype(np.float32)
    cfg = fqlib.adamw_config(1e-2)
    for off in (1, 3):
        w = torch.from_numpy(base.copy()).cuda()[off:off + n]
        g = torch.from_numpy(gbase).cuda()[off:off + n]
        m = torch.zeros(n + 3, device="cuda")[off:off + n]
        v = torch.zeros(n + 3, device="cuda")[off:off + n]
        r = fqlib.qat_step_int(w, g, m, v, 1, cfg, 8, 0, 0)
        rf = fqlib.qat_step_fp8(w, g, m, v, 2, cfg, 0, 0)
        torch.cuda.synchronize()
        ref = orc.qat_step_int(base[off:off + n], gbase[off:off + n], np.zeros(n, np.float32),
                               np.zeros(n, np.float32), 1e-2, 1)
        ref2 = orc.qat_step_fp8(ref["w"], gbase[off:off + n], ref["m"], ref["v"], 1e-2, 2)
        assert_f32(to_np(w), ref2["w"], f"unaligned {off} master")
        assert_bits(to_np(r["codes"]).view(np.int8), ref["codes"], f"unaligned {off} codes")
        assert_bits(to_np(rf["q"]), ref2["q"], f"unaligned {off} bytes")
