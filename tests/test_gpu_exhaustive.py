"""Exhaustive GPU-vs-oracle checks over every binary32 bit pattern (2^32 inputs).

* fp8 cast: the product's fp8 quantize (vector path: exact quotient, then the
  CDNA4 conversion with saturation and NaN fix-ups) for E4M3 and E5M2 at scale 1
  (a plain cast) and at a non-power-of-two scale (the quotient decides the byte),
  against the oracle's unified-ULP rule ([QAT] fake_quant_fp8).
* integer codes: the product's per-tensor int8 affine quantize with given
  parameters at three scales that stress the exact-quotient path (all-ones
  significand, 2^-59 at the edge of the fast window, an odd value), against the
  oracle's quantize.

The oracle runs in host threads (ctypes releases the GIL), one slice per thread.
"""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

from conftest import log
from parity import assert_bits

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28
THREADS = max(1, min(16, os.cpu_count() or 1))


def all_patterns(c):
    return (np.arange(CHUNK, dtype=np.uint32) + np.uint32(c * CHUNK)).view(np.float32)


def parallel(fn, x, out_dtype):
    out = np.empty(x.size, out_dtype)
    step = (x.size + THREADS - 1) // THREADS
    with concurrent.futures.ThreadPoolExecutor(THREADS) as ex:
        futs = [ex.submit(fn, x[i:i + step], out[i:i + step]) for i in range(0, x.size, step)]
        for f in futs:
            f.result()
    return out


@pytest.mark.parametrize("fmt,scale_bits", [(0, 0x3F800000), (1, 0x3F800000), (0, 0x3F7FFFFF), (1, 0x40400001)])
def test_fp8_cast_every_binary32(fqlib, orc, fmt, scale_bits):
    scale = np.array([scale_bits], np.uint32).view(np.float32)
    st = torch.from_numpy(scale.copy()).cuda()
    q = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")

    def enc(xs, out):
        out[:] = orc.fp8_quantize(xs, fmt, float(scale[0]), want_q=True, want_fq=False)[0]

    for c in range(1 << 32 >> 28):
        log(f"fp8 exhaustive fmt={fmt} scale=0x{scale_bits:08x} chunk {c}")
        xh = all_patterns(c)
        xt = torch.from_numpy(xh).cuda()
        fqlib.fq_fp8_quantize(xt, CHUNK, fmt, st, q, None)
        torch.cuda.synchronize()
        ref = parallel(enc, xh, np.uint8)
        assert_bits(q.cpu().numpy(), ref, f"fp8 fmt {fmt} scale 0x{scale_bits:08x} chunk {c}")
        del xt


@pytest.mark.parametrize("scale_bits,zp", [(0x3F7FFFFF, 5), (0x22000000, 0), (0x3DF1A9FD, -77)])
def test_int8_codes_every_binary32(fqlib, orc, scale_bits, zp):
    scale = float(np.array([scale_bits], np.uint32).view(np.float32)[0])
    p = torch.tensor([0, zp, 0, 0], dtype=torch.int32)
    p.view(torch.float32)[0] = scale
    p = p.cuda()
    codes = torch.empty(CHUNK, dtype=torch.int8, device="cuda")

    def quant(xs, out):
        out[:] = orc.fake_quant_int(xs, 8, 1, scale, zp)[0]

    for c in range(1 << 32 >> 28):
        log(f"int8 exhaustive scale=0x{scale_bits:08x} zp={zp} chunk {c}")
        xh = all_patterns(c)
        xt = torch.from_numpy(xh).cuda()
        fqlib.fq_fake_quant_int_tensor(xt, CHUNK, 8, 1, p, codes, None)
        torch.cuda.synchronize()
        ref = parallel(quant, xh, np.int8)
        assert_bits(codes.cpu().numpy(), ref, f"int8 scale 0x{scale_bits:08x} chunk {c}")
        del xt
