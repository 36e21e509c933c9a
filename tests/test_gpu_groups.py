"""GPU parity of group-wise quantization ([CS] demo 3 "granularity", each group
a [QAT] channel) against the oracle: codes, fake-quant, scales, zero-points and
flags bit for bit, on every path of the entry point -- groups of 1..64 lanes in
registers (groups of 4..256 elements, fp32 and bf16) at the full
[4096, 4096] fp32 and [4096, 8192] bf16 shapes, other dividing sizes through the
per-row path, and the generic path for ragged last groups and odd groups with
4-bit codes -- plus special values, unaligned views and group >= cols."""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu


def check(fq, orc, x_t, group, bits, scheme, what=""):
    log(f"groups case {what} shape={tuple(x_t.shape)} dtype={x_t.dtype} group={group} bits={bits} scheme={scheme}")
    bf = x_t.dtype == torch.bfloat16
    r = fq.quant_groups(x_t, group, bits, scheme)
    torch.cuda.synchronize()
    xs = to_np(x_t)
    ref = orc.quant_groups(xs.view(np.uint16) if bf else xs, group, bits, scheme, dtype=1 if bf else 0)
    assert_bits(to_np(r["codes"]), ref["codes"], what + " codes")
    assert_bits(to_np(r["scale"]), ref["scale"], what + " scale")
    assert_bits(to_np(r["zp"]), ref["zp"], what + " zp")
    assert_f32(to_np(r["fq"]), ref["fq"], what + " fq")
    assert int(r["flags"].item()) == ref["flags"], what + " flags"


@pytest.mark.parametrize("group,bits,scheme", [(128, 4, 0), (32, 8, 0), (128, 8, 1), (32, 4, 1)])
def test_weight_full_size(fqlib, orc, group, bits, scheme):
    w = synthetic.rows_f32_inputs(device="cuda")
    check(fqlib, orc, w, group, bits, scheme, "weights [4096, 4096]")


@pytest.mark.parametrize("group,bits,scheme", [(128, 8, 0), (32, 4, 1)])
def test_bf16_activation_shape(fqlib, orc, group, bits, scheme):
    a = synthetic.rows_bf16_inputs(4096, 8192, device="cuda")
    check(fqlib, orc, a, group, bits, scheme, "bf16 [4096, 8192]")


@pytest.mark.parametrize("group", [4, 8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("bits,scheme", [(8, 0), (4, 1)])
def test_register_groups_fp32(fqlib, orc, group, bits, scheme):
    # 1..64 lanes per group; rows x cols chosen so the grid ends mid-block
    rng = np.random.default_rng(group)
    x = (rng.standard_normal((37, 512)) * np.exp(rng.standard_normal((37, 1)))).astype(np.float32)
    check(fqlib, orc, torch.from_numpy(x).cuda(), group, bits, scheme, f"fp32 group {group}")


@pytest.mark.parametrize("group", [4, 8, 16, 32, 64, 128, 256, 512])
def test_register_groups_bf16(fqlib, orc, group):
    rng = np.random.default_rng(group + 1)
    x = torch.from_numpy((rng.standard_normal((19, 1024)) * 3).astype(np.float32)).to(torch.bfloat16).cuda()
    check(fqlib, orc, x, group, 8, 1, f"bf16 group {group}")
    check(fqlib, orc, x, group, 4, 0, f"bf16 group {group}")


@pytest.mark.parametrize("group,cols", [(48, 480), (512, 2048), (2, 64), (6, 60), (1, 40), (1024, 4096)])
@pytest.mark.parametrize("bits", [8, 4])
def test_dividing_groups_via_rows(fqlib, orc, group, cols, bits):
    rng = np.random.default_rng(group * 7 + cols)
    x = rng.standard_normal((33, cols)).astype(np.float32)
    check(fqlib, orc, torch.from_numpy(x).cuda(), group, bits, 0, f"group {group} of {cols}")


@pytest.mark.parametrize("group,cols,bits", [(32, 100, 8), (32, 100, 4), (33, 100, 4), (33, 99, 4), (7, 50, 8),
                                             (5, 21, 4), (128, 300, 4), (3, 3, 4), (10, 7, 8)])
def test_generic_path(fqlib, orc, group, cols, bits):
    rng = np.random.default_rng(group + cols + bits)
    x = (rng.standard_normal((21, cols)) * 2).astype(np.float32)
    for scheme in (0, 1):
        check(fqlib, orc, torch.from_numpy(x).cuda(), group, bits, scheme, f"ragged group {group} of {cols}")
    xb = torch.from_numpy(x).to(torch.bfloat16).cuda()
    check(fqlib, orc, xb, group, bits, 1, f"ragged bf16 group {group} of {cols}")


@pytest.mark.parametrize("group", [32, 30, 33])
def test_special_values(fqlib, orc, group):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 264)).astype(np.float32)
    x[0, :] = 0.0                      # degenerate groups
    x[1, 5] = np.nan
    x[2, 40] = np.inf
    x[3, 70] = -np.inf
    x[4, :group] = np.nan              # a group with no finite value
    x[5, 10] = 3.4e38
    x[6, :] = rng.standard_normal(264) * 1e-40   # subnormals
    x[7, 1::2] = -0.0
    x[8, :] = 7.25                     # constant rows
    for bits, scheme in ((8, 0), (8, 1), (4, 0), (4, 1)):
        check(fqlib, orc, torch.from_numpy(x).cuda(), group, bits, scheme, f"specials group {group}")


def test_unaligned_views(fqlib, orc):
    rng = np.random.default_rng(9)
    base = torch.from_numpy(rng.standard_normal(64 * 256 + 3).astype(np.float32)).cuda()
    for off in (1, 3):
        x = base[off:off + 64 * 256].view(64, 256)
        check(fqlib, orc, x, 32, 8, 0, f"unaligned +{off}")
        check(fqlib, orc, x, 64, 4, 1, f"unaligned +{off}")


def test_group_at_least_cols_is_per_row(fqlib, orc):
    x = torch.from_numpy(np.random.default_rng(2).standard_normal((9, 77)).astype(np.float32)).cuda()
    for group in (77, 78, 1000):
        r = fqlib.quant_groups(x, group, 8, 1)
        rr = fqlib.quant_rows(x, 8, 1)
        torch.cuda.synchronize()
        assert_bits(to_np(r["codes"]), to_np(rr["codes"]), f"group {group} codes")
        assert_bits(to_np(r["scale"]).reshape(-1), to_np(rr["scale"]), f"group {group} scale")


@pytest.mark.parametrize("group,bits", [(16, 8), (32, 8), (128, 8), (64, 4), (256, 4)])
def test_four_element_path(fqlib, orc, group, bits):
    # codes 4-byte (int8) / 2-byte (int4) but not 16 / 8-byte aligned: the groups run
    # four elements per lane instead of sixteen
    rng = np.random.default_rng(group + bits)
    rows, cols = 24, 512
    x = torch.from_numpy((rng.standard_normal((rows, cols)) * 2).astype(np.float32)).cuda()
    nb = rows * cols if bits == 8 else rows * cols // 2
    off = 4 if bits == 8 else 2
    codes = torch.empty(nb + off, dtype=torch.uint8, device="cuda")[off:]
    fqo = torch.empty(rows * cols, dtype=torch.float32, device="cuda")
    ng = cols // group
    scale = torch.empty(rows * ng, dtype=torch.float32, device="cuda")
    zp = torch.empty(rows * ng, dtype=torch.int32, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    fqlib.fq_quant_groups(x, fqlib.F32, rows, cols, group, bits, 1, codes, fqo, scale, zp, flags)
    torch.cuda.synchronize()
    ref = orc.quant_groups(to_np(x), group, bits, 1)
    assert_bits(to_np(codes), ref["codes"].reshape(-1), "codes")
    assert_bits(to_np(scale), ref["scale"].reshape(-1), "scale")
    assert_f32(to_np(fqo), ref["fq"].reshape(-1), "fq")
