"""GPU parity of the kernels whose outputs go through buffer stores built from a
wave's base address (the fp8 quantize and dequantize, the 4-bit quantize's
reconstruction and the x loads of the 4-bit quantize), with every buffer placed
so that the low 32 bits of its address have bit 31 set, and again with it clear.
A base assembled from two 32-bit halves must not carry a sign extension of the
low word into the high word; these placements catch that at any allocator
layout.  Bars: bytes and codes bit-exact, float32 outputs bit-exact."""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu

ARENA = (1 << 31) + (16 << 20)  # bytes: every low-word placement is reachable


@pytest.fixture(scope="module")
def arena(fqlib):
    a = torch.empty(ARENA, dtype=torch.uint8, device="cuda")
    yield a
    del a
    torch.cuda.empty_cache()


def place(arena, nbytes, high, dtype, used):
    """A view of `nbytes` of the arena, 256-byte aligned, starting at an address
    whose bit 31 is set (high) or clear, past the bytes already `used`."""
    base = arena.data_ptr()
    off = (used + 255) // 256 * 256
    while ((base + off) >> 31 & 1) != int(high) or (base + off) % 256:
        off += 1 << 20 if ((base + off) % 256) == 0 else 256 - (base + off) % 256
    assert off + nbytes <= ARENA, "arena too small for the placement"
    v = arena[off:off + nbytes].view(dtype)
    assert ((v.data_ptr() >> 31) & 1) == int(high)
    return v, off + nbytes


@pytest.mark.parametrize("high", [True, False])
def test_fp8_outputs_at_either_half(fqlib, orc, arena, high):
    n = 1 << 20
    x = synthetic.fp8_inputs(n=n, device="cuda", seed=5, special_frac=0.01)
    xn = to_np(x)
    used = 0
    q, used = place(arena, n, high, torch.uint8, used)
    fqv, used = place(arena, 4 * n, high, torch.float32, used)
    deq, used = place(arena, 4 * n, high, torch.float32, used)
    s_t, _ = fqlib.fp8_tensor_scale(x)
    for fmt in (0, 1):
        log(f"address-bit case fp8 fmt={fmt} high={high}")
        fqlib.fq_fp8_quantize(x, n, fmt, s_t[fmt:fmt + 1], q, fqv)
        fqlib.fq_fp8_dequantize(q, n, fmt, s_t[fmt:fmt + 1], deq)
        torch.cuda.synchronize()
        s_ref, _ = orc.fp8_scale(float(orc.amax_finite(xn)), fmt)
        rq, rf = orc.fp8_quantize(xn, fmt, float(s_ref))
        assert_bits(to_np(q), rq, f"bytes fmt{fmt}")
        assert_f32(to_np(fqv), rf, f"fake-quant fmt{fmt}")
        assert_f32(to_np(deq), orc.fp8_dequantize(rq, fmt, float(s_ref)), f"dequantize fmt{fmt}")


@pytest.mark.parametrize("high", [True, False])
def test_q4dq_at_either_half(fqlib, orc, arena, high):
    n = 16384 * 8 + 100  # full super-blocks (the buffer-load / buffer-store kernel) and a partial one
    xs = synthetic.q4dq_inputs(n=n, device="cuda", seed=9)
    log(f"address-bit case q4dq high={high}")
    used = 0
    x, used = place(arena, 4 * n, high, torch.float32, used)
    x.copy_(xs)
    npk, nb, ns = fqlib.fq_q4dq_sizes(n)
    packed, used = place(arena, npk, high, torch.uint8, used)
    qs, used = place(arena, nb, high, torch.uint8, used)
    sup, used = place(arena, 4 * ns, high, torch.float32, used)
    recon, used = place(arena, 4 * n, high, torch.float32, used)
    out, used = place(arena, 4 * n, high, torch.float32, used)
    fqlib.fq_q4dq_quantize(x, n, packed, qs, sup, None, recon, None)
    fqlib.fq_q4dq_dequantize(packed, qs, sup, n, out)
    torch.cuda.synchronize()
    r = orc.q4dq_quantize(to_np(xs))
    assert_bits(to_np(packed), r["packed"], "packed codes")
    assert_bits(to_np(qs), r["qscale"], "u8 scales")
    assert_bits(to_np(sup), r["super"], "super-scales")
    assert_f32(to_np(recon), r["recon"], "reconstruction")
    assert_f32(to_np(out), r["recon"], "dequantize")
