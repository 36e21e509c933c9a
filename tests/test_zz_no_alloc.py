"""GPU check of the workspace-free per-tensor calibration + fake-quant
(fq_calibrate_fake_quant_int_tensor_noalloc, for callers that cannot allocate)
against the entry point it varies, fq_calibrate_fake_quant_int_tensor with a
caller workspace: params, codes, fake-quant values and flags bit for bit, on two
calls in a row of which the second is smaller (the static scratch keeps the
first call's partials).  The tensors cover both launch paths of the call: up to
512 reduction partials (two launches) and beyond (three launches)."""
import numpy as np
import pytest
import torch

from conftest import log
from fake_quant_amd import synthetic
from parity import assert_bits, assert_f32, to_np

pytestmark = pytest.mark.gpu


def run_both(fq, x, bits, scheme):
    n = x.numel()
    cb = n if bits == 8 else (n + 1) // 2
    dev = x.device
    outs = []
    for noalloc in (False, True):
        params = torch.full((4,), -1, dtype=torch.int32, device=dev)
        codes = torch.full((cb,), 0x55, dtype=torch.uint8, device=dev)
        fqv = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
        flags = torch.zeros(1, dtype=torch.int32, device=dev)
        if noalloc:
            fq.fq_calibrate_fake_quant_int_tensor_noalloc(x, n, bits, scheme, params, codes, fqv, flags)
        else:
            wsb = fq.fq_workspace_bytes(n)
            ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
            fq.fq_calibrate_fake_quant_int_tensor(x, n, bits, scheme, ws, wsb, params, codes, fqv, flags)
        torch.cuda.synchronize()
        outs.append((to_np(params), to_np(codes), to_np(fqv), int(flags.item())))
    return outs


def inputs(n, seed, special):
    x, _ = synthetic.tensor_inputs(n, device="cuda", seed=seed)
    if special:
        x[n // 3] = float("inf")
        x[n // 2] = float("nan")
    return x


@pytest.mark.parametrize("sizes", [(3_000_005, 4099), ((1 << 22) + 8197, 70_001), ((1 << 22) + 4, 1)])
@pytest.mark.parametrize("bits,scheme", [(8, 0), (4, 1)])
def test_noalloc_matches_workspace_entry_point(fqlib, sizes, bits, scheme):
    for k, n in enumerate(sizes):
        log(f"noalloc case sizes={sizes} call={k} n={n} bits={bits} scheme={scheme}")
        x = inputs(n, seed=11 + k, special=(k == 1 and n > 4))
        (p0, c0, f0, g0), (p1, c1, f1, g1) = run_both(fqlib, x, bits, scheme)
        assert_bits(p1, p0, f"params n={n}")
        assert_bits(c1, c0, f"codes n={n}")
        assert_f32(f1, f0, f"fake-quant n={n}")
        assert g1 == g0, f"flags n={n}"
        if k == 1 and n > 4:
            assert g1 & fqlib.FLAG_NONFINITE


def test_noalloc_zero_tensor_after_data(fqlib):
    """A degenerate (all-zero) tensor after a call on data: scale 0, codes 0,
    fake-quant +0 and the DEGENERATE flag, as the workspace entry point gives."""
    for k, n in enumerate((1 << 20, 5000)):
        log(f"noalloc zero case call={k} n={n}")
        x = inputs(n, seed=3, special=False) if k == 0 else torch.zeros(n, dtype=torch.float32, device="cuda")
        (p0, c0, f0, g0), (p1, c1, f1, g1) = run_both(fqlib, x, 8, 1)
        assert_bits(p1, p0, "params")
        assert_bits(c1, c0, "codes")
        assert_f32(f1, f0, "fake-quant")
        assert g1 == g0
    assert g1 & fqlib.FLAG_DEGENERATE
    assert np.all(c1 == 0) and np.all(f1.view(np.uint32) == 0)
