"""GPU parity of the fused per-row calibration + quantize against the oracle.

Workloads: [4096, 4096] float32 weights with lognormal row sigmas, int8 / int4,
symmetric / affine (codes, fake-quant, scales, zero-points); [16384, 8192]
bfloat16 ReLU activations with outlier channels, per-token affine int8 (sampled
rows at full size); ragged shapes, multi-slab rows, unaligned views, special rows.
"""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu


def check_rows(fq, orc, x_t, bits, scheme, what="", rows_idx=None, want_fq=True):
    log(f"rows case {what} shape={tuple(x_t.shape)} dtype={x_t.dtype} bits={bits} scheme={scheme}")
    bf = x_t.dtype == torch.bfloat16
    r = fq.quant_rows(x_t, bits, scheme, want_fq=want_fq)
    torch.cuda.synchronize()
    if rows_idx is None:
        rows_idx = np.arange(x_t.shape[0])
    idx_t = torch.from_numpy(rows_idx).to(x_t.device)
    xs = to_np(x_t.index_select(0, idx_t))
    ref = orc.quant_rows(xs.view(np.uint16) if bf else xs, bits, scheme, dtype=1 if bf else 0, want_fq=want_fq)
    assert_bits(to_np(r["codes"].index_select(0, idx_t)), ref["codes"], what + " codes")
    assert_bits(to_np(r["scale"])[rows_idx], ref["scale"], what + " scale")
    assert_bits(to_np(r["zp"])[rows_idx], ref["zp"], what + " zp")
    if want_fq:
        assert_f32(to_np(r["fq"].index_select(0, idx_t)), ref["fq"], what + " fq")
    if len(rows_idx) == x_t.shape[0]:
        assert int(r["flags"].item()) == ref["flags"], what + " flags"
    else:
        assert int(r["flags"].item()) & ref["flags"] == ref["flags"], what + " flags"
    return r


@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 0), (4, 1)])
def test_weight_rows_full_size(fqlib, orc, bits, scheme):
    w = synthetic.rows_f32_inputs(device="cuda")
    r = check_rows(fqlib, orc, w, bits, scheme, what="W 4096x4096")
    rows, cols = w.shape
    deq = fqlib.dequantize_rows(r["codes"], rows, cols, r["scale"], r["zp"], bits)
    torch.cuda.synchronize()
    assert_bits(to_np(deq), to_np(r["fq"]), "dequantize_rows == fake-quant")


def test_activation_rows_full_size_sampled(fqlib, orc):
    a = synthetic.rows_bf16_inputs(device="cuda")
    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([[0, a.shape[0] - 1], rng.choice(a.shape[0], 254, replace=False)]))
    r = check_rows(fqlib, orc, a, 8, 1, what="A 16384x8192 bf16", rows_idx=idx, want_fq=False)
    # ReLU rows: min is 0, so every zero-point is the lowest code
    assert int(r["zp"].min().item()) == -128 and int(r["zp"].max().item()) == -128


# ragged and aligned lengths; the aligned ones hit every launch shape: a wave
# per row (<= 256 vectors, > 4 workgroup widths) and a workgroup per row with
# one to four vectors per thread (fp32: 1200, 2056, 6000, 8192 columns; bf16:
# 2056, 4096, 6000, 8192 columns)
SHAPES = [(1, 1), (3, 5), (7, 127), (2, 4095), (5, 4097), (3, 9001), (4, 12288), (9, 3), (2, 64),
          (3, 1200), (3, 2056), (2, 4096), (3, 6000), (2, 8192)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bf16", [False, True])
def test_ragged_shapes(fqlib, orc, shape, bf16):
    rows, cols = shape
    w = synthetic.rows_f32_inputs(rows, cols, device="cuda", seed=rows * 7 + cols)
    if bf16:
        w = w.to(torch.bfloat16)
    for bits, scheme in [(8, 0), (8, 1), (4, 0), (4, 1)]:
        check_rows(fqlib, orc, w, bits, scheme, what=f"ragged {shape} bf16={bf16}")


def test_long_bf16_rows(fqlib, orc):
    a = synthetic.rows_bf16_inputs(6, 20000, device="cuda", seed=5)
    for bits, scheme in [(8, 1), (4, 0)]:
        check_rows(fqlib, orc, a, bits, scheme, what="bf16 20000 cols")


def test_unaligned_views(fqlib, orc):
    w = synthetic.rows_f32_inputs(8, 1030, device="cuda", seed=2)
    flat = w.reshape(-1)
    v = flat[1:1 + 8 * 1024].reshape(8, 1024)  # 4-byte offset: not 16-byte aligned
    for bits, scheme in [(8, 0), (4, 1)]:
        check_rows(fqlib, orc, v, bits, scheme, what="offset view")


@pytest.mark.parametrize("cols", [300, 1200, 4096, 6000, 8192])
def test_special_rows(fqlib, orc, cols):
    """Zero, NaN, Inf, tiny, huge, one-signed and -0 rows through every launch
    shape (a wave per row at 300 columns, a workgroup per row above)."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((10, cols)) * np.exp(rng.normal(-3, 0.5, (10, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1, 5] = np.nan
    x[1, -3] = np.nan           # also in the last vector a thread holds
    x[2, 7] = np.inf
    x[2, -1] = -np.inf
    x[3] = np.nan
    x[4] *= np.float32(1e-33)   # tiny scale -> exact-division fallback
    x[5] = np.abs(x[5]) + 1.0   # all positive
    x[6] = -np.abs(x[6]) - 1.0  # all negative
    x[7, :] = -0.0
    x[8] *= np.float32(1e30)
    x[9, ::2] = -np.inf
    xt = torch.from_numpy(x).cuda()
    for bits in (8, 4):
        for scheme in (0, 1):
            check_rows(fqlib, orc, xt, bits, scheme, what=f"special rows {cols}")
            check_rows(fqlib, orc, xt.to(torch.bfloat16), bits, scheme, what=f"special rows bf16 {cols}")


def test_deterministic(fqlib):
    w = synthetic.rows_f32_inputs(device="cuda")
    a = fqlib.quant_rows(w, 4, 1)
    b = fqlib.quant_rows(w, 4, 1)
    torch.cuda.synchronize()
    for k in ("codes", "fq", "scale", "zp"):
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k
