"""check=True on the GPU: the calibrating calls synchronise and raise FqFlagError
for the conditions the pages report as InvalidState (a calibration group with a
non-finite value, or with no usable range), and stay silent otherwise; the
outputs are written either way."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_check_raises_on_flags(fqlib):
    ok = torch.randn(4, 256, device="cuda")
    nan = ok.clone()
    nan[1, 3] = float("nan")
    zero = torch.zeros(4, 256, device="cuda")
    fqlib.params_int(ok.reshape(-1), check=True)
    fqlib.quant_rows(ok, check=True)
    fqlib.quant_groups(ok, 32, check=True)
    fqlib.quant_cols(ok, check=True)
    fqlib.params_percentile(ok.reshape(-1), 0.01, check=True)
    for call in (lambda x: fqlib.params_int(x.reshape(-1), check=True),
                 lambda x: fqlib.quant_rows(x, check=True),
                 lambda x: fqlib.quant_groups(x, 32, check=True),
                 lambda x: fqlib.quant_cols(x, check=True),
                 lambda x: fqlib.params_percentile(x.reshape(-1), 0.01, check=True)):
        with pytest.raises(fqlib.FqFlagError) as e:
            call(nan)
        assert e.value.status & fqlib.FLAG_NONFINITE
        with pytest.raises(fqlib.FqFlagError) as e:
            call(zero)
        assert e.value.status & fqlib.FLAG_DEGENERATE
    # the fp8 scale skips non-finite values without flagging them; a zero scale is flagged
    fqlib.fp8_tensor_scale(nan.reshape(-1), check=True)
    with pytest.raises(fqlib.FqFlagError) as e:
        fqlib.fp8_tensor_scale(zero.reshape(-1), check=True)
    assert e.value.status == fqlib.FLAG_DEGENERATE
    # without check the same calls return the flag word
    r = fqlib.quant_rows(nan)
    torch.cuda.synchronize()
    assert int(r["flags"].item()) == fqlib.FLAG_NONFINITE
    assert np.isfinite(r["scale"].cpu().numpy()).all()
