"""GPU parity of the 32-element E4M3 blocks with power-of-two (E8M0) scales.

Workload: [16384, 8192] bfloat16 ReLU activations with outlier channels (sampled
rows at full size); ragged column counts (partial blocks), float32 input,
unaligned views and special values.
"""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu


def check_mx(fq, orc, x_t, what="", rows_idx=None, want_fq=True):
    log(f"mx case {what} shape={tuple(x_t.shape)} dtype={x_t.dtype}")
    bf = x_t.dtype == torch.bfloat16
    r = fq.mxfp8_rows(x_t, want_fq=want_fq)
    torch.cuda.synchronize()
    if rows_idx is None:
        rows_idx = np.arange(x_t.shape[0])
    it = torch.from_numpy(rows_idx).to(x_t.device)
    xs = to_np(x_t.index_select(0, it))
    ref = orc.mxfp8_rows(xs.view(np.uint16) if bf else xs, dtype=1 if bf else 0, want_fq=want_fq)
    assert_bits(to_np(r["q"].index_select(0, it)), ref["q"], what + " bytes")
    assert_bits(to_np(r["e8m0"].index_select(0, it)), ref["e8m0"], what + " e8m0")
    if want_fq:
        assert_f32(to_np(r["fq"].index_select(0, it)), ref["fq"], what + " fq")


def test_full_size_sampled(fqlib, orc):
    a = synthetic.rows_bf16_inputs(device="cuda")
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([[0, a.shape[0] - 1], rng.choice(a.shape[0], 254, replace=False)]))
    check_mx(fqlib, orc, a, what="A 16384x8192", rows_idx=idx, want_fq=False)
    check_mx(fqlib, orc, a[:512], what="A first 512 rows with fq")


@pytest.mark.parametrize("cols", [1, 31, 32, 33, 100, 4096 + 17])
@pytest.mark.parametrize("bf16", [True, False])
def test_ragged_cols(fqlib, orc, cols, bf16):
    a = synthetic.rows_bf16_inputs(5, cols, device="cuda", seed=cols)
    x = a if bf16 else a.float() * torch.randn(5, cols, device="cuda")
    check_mx(fqlib, orc, x, what=f"cols {cols} bf16={bf16}")


def test_float32_rows(fqlib, orc):
    w = synthetic.rows_f32_inputs(64, 4096, device="cuda", seed=6)
    check_mx(fqlib, orc, w, what="f32 64x4096")


def test_unaligned_and_specials(fqlib, orc):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((6, 256)) * 10.0 ** rng.integers(-30, 30, (6, 1))).astype(np.float32)
    x[0, :32] = 0.0
    x[1, 3] = np.nan
    x[1, 40] = np.inf
    x[2, 64:96] = np.float32(1e-42)
    x[3, :] = np.float32(3e38)
    x[4, 100] = -np.inf
    x[5, ::3] = -0.0
    xt = torch.from_numpy(x).cuda()
    check_mx(fqlib, orc, xt, what="specials f32")
    check_mx(fqlib, orc, xt.to(torch.bfloat16), what="specials bf16")
    flat = synthetic.rows_bf16_inputs(1, 8 * 256 + 8, device="cuda", seed=1).reshape(-1)
    check_mx(fqlib, orc, flat[8 - 1:8 - 1 + 8 * 256].reshape(8, 256), what="offset view bf16")
