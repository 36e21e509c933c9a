"""GPU parity of the 4-bit blocks + double-quantized scales against the oracle.

Workload: 2^30 float32 Student-t(4) * 0.02 (4 GiB; sampled super-blocks compared
with the oracle run on the same slices -- super-blocks are independent), plus
ragged lengths, unaligned views, the page's small and all-zero inputs, special
values and tiny blocks.
"""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu

SB = 16384


def check_q4(fq, orc, x_t, what=""):
    n = x_t.numel()
    log(f"q4dq case {what} n={n}")
    r = fq.q4dq_quantize(x_t)
    deq = fq.q4dq_dequantize(r["packed"], r["qscale"], r["super"], n)
    torch.cuda.synchronize()
    ref = orc.q4dq_quantize(to_np(x_t))
    assert_bits(to_np(r["packed"]), ref["packed"], what + " packed")
    assert_bits(to_np(r["qscale"]), ref["qscale"], what + " qscale")
    assert_bits(to_np(r["super"]), ref["super"], what + " super")
    assert_bits(to_np(r["block_scale"]), ref["block_scale"], what + " block scale")
    assert_f32(to_np(r["recon"]), ref["recon"], what + " recon")
    assert_f32(to_np(deq), ref["recon"], what + " dequant")
    assert int(r["flags"].item()) == ref["flags"], what + " flags"


def test_full_size_workload_sampled(fqlib, orc):
    n = 1 << 30
    x = synthetic.q4dq_inputs(device="cuda")
    log("q4dq full size: quantize")
    r = fqlib.q4dq_quantize(x)
    deq = fqlib.q4dq_dequantize(r["packed"], r["qscale"], r["super"], n)
    torch.cuda.synchronize()
    nsb = n // SB
    rng = np.random.default_rng(1)
    sbs = np.unique(np.concatenate([[0, nsb - 1], rng.choice(nsb, 96, replace=False)]))
    for k in sbs:
        k = int(k)
        xs = to_np(x[k * SB:(k + 1) * SB])
        ref = orc.q4dq_quantize(xs)
        w = f"super-block {k}"
        assert_bits(to_np(r["packed"][k * SB // 2:(k + 1) * SB // 2]), ref["packed"], w + " packed")
        assert_bits(to_np(r["qscale"][k * 256:(k + 1) * 256]), ref["qscale"], w + " qscale")
        assert_bits(to_np(r["super"][k:k + 1]), ref["super"], w + " super")
        assert_bits(to_np(r["block_scale"][k * 256:(k + 1) * 256]), ref["block_scale"], w + " block scale")
        assert_f32(to_np(r["recon"][k * SB:(k + 1) * SB]), ref["recon"], w + " recon")
        assert_f32(to_np(deq[k * SB:(k + 1) * SB]), ref["recon"], w + " dequant")
    assert int(r["flags"].item()) == 0
    # every super-scale is the maximum of its block scales (floored) and every
    # group's largest block has u8 code 255 -- checked over the whole tensor
    bs = r["block_scale"].view(-1, 256)
    assert torch.equal(r["super"], torch.clamp(bs.max(dim=1).values, min=np.float32(1e-8)))
    qs = r["qscale"].view(-1, 256)
    assert int(qs.max(dim=1).values.min().item()) == 255
    del x, r, deq


@pytest.mark.parametrize("n", [1, 2, 3, 63, 64, 65, 127, 4099, 16383, 16384, 16385, 3 * SB + 100, 5 * SB + 1, 8 * SB, 11 * SB + 5])
def test_ragged_sizes(fqlib, orc, n):
    x = synthetic.q4dq_inputs(n=n, device="cuda", seed=n)
    check_q4(fqlib, orc, x, what=f"ragged {n}")


def test_unaligned(fqlib, orc):
    buf = synthetic.q4dq_inputs(n=4 * SB + 9, device="cuda", seed=4)
    for off in (1, 3):
        check_q4(fqlib, orc, buf[off:off + 3 * SB], what=f"offset {off}")


def test_page_examples_and_specials(fqlib, orc):
    small = torch.tensor([1.0, -2.0, 3.0, -4.0], device="cuda")
    check_q4(fqlib, orc, small, what="page small input")
    check_q4(fqlib, orc, torch.zeros(128, device="cuda"), what="page zeros")
    check_q4(fqlib, orc, torch.arange(200, device="cuda", dtype=torch.float32) * 0.5, what="page length 200")
    i = torch.arange(4096, device="cuda", dtype=torch.float32)
    check_q4(fqlib, orc, torch.sin(i * 0.1) * 2.0, what="page sinusoid")
    rng = np.random.default_rng(2)
    x = (rng.standard_t(4, 5 * SB) * 0.02).astype(np.float32)
    x[3 * SB + 11] = np.nan        # specials in later super-blocks of a workgroup too
    x[4 * SB + 999] = np.inf
    x[100] = np.nan
    x[5000] = np.inf
    x[SB + 7] = -np.inf
    x[640:704] = 0.0
    x[1024:1088] *= np.float32(1e-25)   # tiny block scale: exact-division fallback
    x[2048:2112] = (np.arange(64) - 32 + 0.5).astype(np.float32) * np.float32(7 / 31.5)  # ties
    x[3 * 64:4 * 64] = np.float32(1e-44)
    check_q4(fqlib, orc, torch.from_numpy(x).cuda(), what="specials")
    huge = (rng.standard_normal(SB) * 1e36).astype(np.float32)
    check_q4(fqlib, orc, torch.from_numpy(huge).cuda(), what="huge")
    tiny = (rng.standard_normal(SB) * 1e-12).astype(np.float32)
    check_q4(fqlib, orc, torch.from_numpy(tiny).cuda(), what="tiny (1e-8 floor)")


def test_deterministic(fqlib):
    x = synthetic.q4dq_inputs(n=64 * SB, device="cuda")
    a = fqlib.q4dq_quantize(x)
    b = fqlib.q4dq_quantize(x)
    torch.cuda.synchronize()
    for k in ("packed", "qscale", "super", "recon"):
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k
