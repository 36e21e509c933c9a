"""GPU parity of per-column (axis 1) calibration + quantize against the oracle:
codes, fake-quant, scales, zero-points and flags for the [4096, 4096] fp32
weight workload (all four widths / schemes), a bf16 activation-shaped tensor,
ragged shapes (aligned and unaligned paths, one to many row chunks), special
columns and unaligned views."""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu


def check_cols(fq, orc, x_t, bits, scheme, what=""):
    log(f"cols case {what} shape={tuple(x_t.shape)} dtype={x_t.dtype} bits={bits} scheme={scheme}")
    bf = x_t.dtype == torch.bfloat16
    r = fq.quant_cols(x_t, bits, scheme)
    torch.cuda.synchronize()
    xs = to_np(x_t)
    ref = orc.quant_cols(xs.view(np.uint16) if bf else xs, bits, scheme, dtype=1 if bf else 0)
    assert_bits(to_np(r["codes"]), ref["codes"], what + " codes")
    assert_bits(to_np(r["scale"]), ref["scale"], what + " scale")
    assert_bits(to_np(r["zp"]), ref["zp"], what + " zp")
    assert_f32(to_np(r["fq"]), ref["fq"], what + " fq")
    assert int(r["flags"].item()) == ref["flags"], what + " flags"


@pytest.mark.parametrize("bits,scheme", [(8, 0), (8, 1), (4, 0), (4, 1)])
def test_weight_full_size(fqlib, orc, bits, scheme):
    w = synthetic.rows_f32_inputs(device="cuda")
    check_cols(fqlib, orc, w, bits, scheme, "weights [4096, 4096]")


def test_bf16_activation_shape(fqlib, orc):
    a = synthetic.rows_bf16_inputs(4096, 8192, device="cuda")
    check_cols(fqlib, orc, a, 8, 1, "bf16 [4096, 8192]")


SHAPES = [(1, 1), (3, 5), (7, 127), (2, 4095), (5, 4097), (64, 3), (65, 9), (130, 1000), (1000, 7), (300, 256)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bf16", [False, True])
def test_ragged_shapes(fqlib, orc, shape, bf16):
    rows, cols = shape
    w = synthetic.rows_f32_inputs(rows, cols, device="cuda", seed=rows * 13 + cols)
    if bf16:
        w = w.to(torch.bfloat16)
    for bits, scheme in ((8, 1), (4, 0)):
        check_cols(fqlib, orc, w, bits, scheme, f"ragged {shape}")


def test_special_columns(fqlib, orc):
    rng = np.random.default_rng(1)
    rows, cols = 200, 24
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.normal(-3, 0.5, (1, cols)))).astype(np.float32)
    x[:, 0] = 0.0
    x[5, 1] = np.nan
    x[7, 2] = np.inf
    x[:, 3] = np.nan
    x[:, 4] *= np.float32(1e-33)
    x[:, 5] = np.abs(x[:, 5]) + 1.0
    x[:, 6] = -np.abs(x[:, 6]) - 1.0
    x[:, 7] = -0.0
    x[:, 8] *= np.float32(1e30)
    x[::2, 9] = -np.inf
    xt = torch.from_numpy(x).cuda()
    for bits in (8, 4):
        for scheme in (0, 1):
            check_cols(fqlib, orc, xt, bits, scheme, "special columns")
            check_cols(fqlib, orc, xt.to(torch.bfloat16), bits, scheme, "special columns bf16")


def test_unaligned_view(fqlib, orc):
    buf = synthetic.rows_f32_inputs(1, 100 * 64 + 3, device="cuda").reshape(-1)
    x = buf[3:].reshape(100, 64)
    check_cols(fqlib, orc, x, 8, 1, "unaligned")


def test_bf16_quantize_vectors(fqlib, orc):
    # the quantize pass reads four bf16 columns (8 bytes) per lane, the min / max
    # pass eight (16 bytes): a column count that is a multiple of four but not of
    # eight, and views 8-byte aligned (vector quantize, element min / max) and
    # 4-byte aligned (element loads in both)
    w = synthetic.rows_f32_inputs(300, 260, device="cuda", seed=260).to(torch.bfloat16)
    for bits, scheme in ((8, 1), (4, 0), (4, 1)):
        check_cols(fqlib, orc, w, bits, scheme, "bf16 cols % 8 == 4")
    buf = synthetic.rows_f32_inputs(1, 130 * 512 + 8, device="cuda", seed=7).reshape(-1).to(torch.bfloat16)
    for off in (4, 2):
        x = buf[off:off + 130 * 512].reshape(130, 512)
        for bits, scheme in ((8, 0), (4, 1)):
            check_cols(fqlib, orc, x, bits, scheme, f"bf16 view at element {off}")


# fp32 shapes of the one-pass strip kernel (1024 < rows <= 4096, cols a multiple
# of 16 with at least half as many 16-column strips as compute units): smallest
# and largest row counts, rows that leave a partial 256-row load, and each way of
# dealing strips to workgroups: groups of eight adjacent strips (a strip count
# divisible by 64), a contiguous run per XCD (136 strips: divisible by 8, not by
# 64), strip b on workgroup b (130 and 129 strips), more strips than compute units
STRIP_SHAPES = [(1025, 2048), (4096, 2080), (2500, 4096), (4095, 8192), (1536, 2064), (2000, 2176)]


@pytest.mark.parametrize("shape", STRIP_SHAPES)
def test_strip_path_shapes(fqlib, orc, shape):
    rows, cols = shape
    w = synthetic.rows_f32_inputs(rows, cols, device="cuda", seed=rows + cols)
    for bits, scheme in ((8, 0), (8, 1), (4, 0), (4, 1)):
        check_cols(fqlib, orc, w, bits, scheme, f"strip {shape}")


# bf16 shapes of the one-pass strip kernel (1024 < rows <= 4096, cols a multiple
# of 32 with at least half as many 32-column strips as compute units): smallest
# and largest row counts, rows that leave a partial 128-row load, strip counts
# dealt in groups of eight (128, 256), as a contiguous run per XCD (136) and one
# per workgroup (129); then column counts the strip kernel does not take (a
# multiple of 4 but not of 32, too few strips), which go through the three-launch
# path
STRIP_SHAPES_BF16 = [(1025, 4096), (4096, 4128), (2500, 8192), (4095, 4096), (1999, 4352), (3000, 4100),
                     (2048, 4064)]


@pytest.mark.parametrize("shape", STRIP_SHAPES_BF16)
def test_strip_path_shapes_bf16(fqlib, orc, shape):
    rows, cols = shape
    w = synthetic.rows_f32_inputs(rows, cols, device="cuda", seed=rows + cols).to(torch.bfloat16)
    for bits, scheme in ((8, 0), (8, 1), (4, 0), (4, 1)):
        check_cols(fqlib, orc, w, bits, scheme, f"bf16 {shape}")


def test_strip_special_columns(fqlib, orc):
    """Special columns spread over several strips of the one-pass kernel, with the
    wave-uniform fast path taken by some strips and not by others."""
    rng = np.random.default_rng(2)
    rows, cols = 1100, 2048
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.normal(-3, 0.5, (1, cols)))).astype(np.float32)
    x[:, 0] = 0.0
    x[5, 17] = np.nan
    x[1099, 40] = np.inf
    x[:, 63] = np.nan
    x[:, 100] *= np.float32(1e-33)
    x[:, 129] = np.abs(x[:, 129]) + 1.0
    x[:, 130] = -np.abs(x[:, 130]) - 1.0
    x[:, 511] = -0.0
    x[:, 777] *= np.float32(1e30)
    x[::2, 1500] = -np.inf
    x[:, 2047] = np.float32(3.0)
    xt = torch.from_numpy(x).cuda()
    for bits in (8, 4):
        for scheme in (0, 1):
            check_cols(fqlib, orc, xt, bits, scheme, "strip special columns")
    # the same columns in bf16, 4096 wide
    xb = torch.from_numpy(np.concatenate([x, x[:, ::-1]], axis=1).copy()).cuda().to(torch.bfloat16)
    for bits in (8, 4):
        for scheme in (0, 1):
            check_cols(fqlib, orc, xb, bits, scheme, "bf16 special columns")
