"""GPU parity of the FP4 / FP6 block formats ([CS] demo 4 block_scaled) against
the oracle, bit for bit: MXFP4 (E2M1) and MXFP6 (E2M3, E3M2) with E8M0 scales
per 32 elements along rows -- codes, scale bytes and fake-quant values -- on the
[4096, 4096] fp32 and [4096, 8192] bf16 shapes, short rows of multiples of 32
(the wide layout ending mid-wave), ragged and odd row lengths, unaligned views
and special values; and NVFP4 (E2M1, E4M3 block scales of 16,
fp32 tensor scale) on the 2^20 tensor, the 2^26 fp8 workload with its NaN / Inf /
zero elements, short and ragged lengths, an unaligned view and the zero tensor.
"""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu

ELEMS = {"E2M1": 2, "E2M3": 3, "E3M2": 4}


def check_mx(fq, orc, x_t, elem, what=""):
    log(f"mx case {what} shape={tuple(x_t.shape)} dtype={x_t.dtype} elem={elem}")
    bf = x_t.dtype == torch.bfloat16
    r = fq.mx_rows(x_t, elem)
    torch.cuda.synchronize()
    xs = to_np(x_t)
    ref = orc.mx_rows(xs.view(np.uint16) if bf else xs, elem, dtype=1 if bf else 0)
    assert_bits(to_np(r["q"]), ref["q"], what + " codes")
    assert_bits(to_np(r["e8m0"]), ref["e8m0"], what + " e8m0")
    assert_f32(to_np(r["fq"]), ref["fq"], what + " fq")


def check_nv(fq, orc, x_t, what=""):
    log(f"nvfp4 case {what} n={x_t.numel()}")
    r = fq.nvfp4(x_t)
    torch.cuda.synchronize()
    ref = orc.nvfp4(to_np(x_t))
    assert_bits(to_np(r["g"]), np.float32([ref["g"]]), what + " tensor scale")
    assert_bits(to_np(r["scales"]), ref["sbytes"], what + " block scales")
    assert_bits(to_np(r["q"]), ref["q"], what + " codes")
    assert_f32(to_np(r["fq"]), ref["fq"], what + " fq")


@pytest.mark.parametrize("elem", list(ELEMS.values()), ids=list(ELEMS))
def test_mx_weights_full_size(fqlib, orc, elem):
    w = synthetic.rows_f32_inputs(device="cuda")
    check_mx(fqlib, orc, w, elem, "weights [4096, 4096]")


@pytest.mark.parametrize("elem", list(ELEMS.values()), ids=list(ELEMS))
def test_mx_bf16_activation_shape(fqlib, orc, elem):
    a = synthetic.rows_bf16_inputs(4096, 8192, device="cuda")
    check_mx(fqlib, orc, a, elem, "bf16 [4096, 8192]")


@pytest.mark.parametrize("cols", [1, 7, 31, 33, 100, 257])
@pytest.mark.parametrize("elem", list(ELEMS.values()), ids=list(ELEMS))
def test_mx_ragged_rows(fqlib, orc, cols, elem):
    rng = np.random.default_rng(cols * 10 + elem)
    x = (rng.standard_t(5, (23, cols)) * 0.02).astype(np.float32)
    check_mx(fqlib, orc, torch.from_numpy(x).cuda(), elem, f"cols {cols}")
    check_mx(fqlib, orc, torch.from_numpy(x).to(torch.bfloat16).cuda(), elem, f"bf16 cols {cols}")


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 32), (23, 64), (7, 96), (5, 160), (33, 1056)])
@pytest.mark.parametrize("elem", list(ELEMS.values()), ids=list(ELEMS))
def test_mx_wide_layout_shapes(fqlib, orc, rows, cols, elem):
    # rows a multiple of 32 wide: sixteen elements per lane, a lane pair per block;
    # these sizes end mid-wave and mid-workgroup
    rng = np.random.default_rng(rows * 1000 + cols + elem)
    x = (rng.standard_t(5, (rows, cols)) * np.exp(rng.standard_normal((rows, 1)))).astype(np.float32)
    check_mx(fqlib, orc, torch.from_numpy(x).cuda(), elem, f"wide {rows}x{cols}")
    check_mx(fqlib, orc, torch.from_numpy(x).to(torch.bfloat16).cuda(), elem, f"wide bf16 {rows}x{cols}")


@pytest.mark.parametrize("elem", list(ELEMS.values()), ids=list(ELEMS))
def test_mx_special_values(fqlib, orc, elem):
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((12, 128)) * 3).astype(np.float32)
    x[0, :32] = 0.0
    x[1, 5] = np.nan
    x[2, 40] = np.inf
    x[3, 70] = -np.inf
    x[4, :32] = np.nan
    x[5, 10] = 3.4e38
    x[6, :] = rng.standard_normal(128) * 1e-40
    x[7, 1::2] = -0.0
    x[8, :] = rng.standard_normal(128) * 1e-38
    x[9, :64] = 2.0 ** -126
    x[10, :] = 7.25
    x[11, 3] = 1e30
    check_mx(fqlib, orc, torch.from_numpy(x).cuda(), elem, "specials")


def test_mx_unaligned_and_e4m3_forward(fqlib, orc):
    rng = np.random.default_rng(22)
    base = torch.from_numpy(rng.standard_normal(64 * 96 + 3).astype(np.float32)).cuda()
    for off in (1, 2):
        x = base[off:off + 64 * 96].view(64, 96)
        for elem in ELEMS.values():
            check_mx(fqlib, orc, x, elem, f"unaligned +{off}")
    # FQ_E4M3 runs the MXFP8 path
    x = torch.from_numpy(rng.standard_normal((8, 64)).astype(np.float32)).cuda()
    r = fqlib.mx_rows(x, fqlib.E4M3)
    torch.cuda.synchronize()
    ref = orc.mxfp8_rows(to_np(x), dtype=0)
    assert_bits(to_np(r["q"]), ref["q"], "e4m3 codes")
    assert_f32(to_np(r["fq"]), ref["fq"], "e4m3 fq")


def test_nvfp4_tensor_workload(fqlib, orc):
    x, _ = synthetic.tensor_inputs(device="cuda")
    check_nv(fqlib, orc, x, "tensor 2^20")


def test_nvfp4_fp8_workload_with_specials(fqlib, orc):
    check_nv(fqlib, orc, synthetic.fp8_inputs(device="cuda"), "fp8 2^26")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 15, 16, 17, 31, 33, 1000, 4099, (1 << 20) + 7])
def test_nvfp4_lengths(fqlib, orc, n):
    rng = np.random.default_rng(n)
    x = (rng.standard_t(5, n) * 0.02).astype(np.float32)
    check_nv(fqlib, orc, torch.from_numpy(x).cuda(), f"n={n}")


def test_nvfp4_edges(fqlib, orc):
    rng = np.random.default_rng(23)
    check_nv(fqlib, orc, torch.zeros(4096, device="cuda"), "zero tensor")
    x = (rng.standard_normal(8192) * 1e-3).astype(np.float32)
    x[::16] *= 1e4          # one large element per block
    x[100:116] = 0.0        # a zero block
    x[200:216] = 1e-20      # a block far below the tensor scale (E4M3 scale 0 -> X = 1)
    x[300] = np.nan
    x[400] = -np.inf
    x[500:516] = -0.0
    check_nv(fqlib, orc, torch.from_numpy(x).cuda(), "edges")
    base = torch.from_numpy(rng.standard_normal(5003).astype(np.float32)).cuda()
    check_nv(fqlib, orc, base[1:5001], "unaligned view")
    tiny = torch.from_numpy(np.float32([1e-42, -3e-43, 2e-44, 0.0] * 8)).cuda()
    check_nv(fqlib, orc, tiny, "subnormal tensor")
