"""The benchmark's measurement helpers (include/fq_bench.h) on the GPU: the copy
reproduces its input bit for bit, the flush reads without writing anything but
its sink (which no ordinary buffer triggers)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_copy_f32_bitwise(fqlib):
    n = (1 << 20) + 4
    x = torch.randn(n, device="cuda")
    x[:8] = torch.tensor([float("nan"), float("inf"), -float("inf"), -0.0, 0.0, 1e-45, -3.5, 7.0])
    y = torch.full_like(x, 123.0)
    fqlib.fqb_copy_f32(x, y, n)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_flush_leaves_buffers_alone(fqlib):
    torch.manual_seed(0)
    s = torch.randn(1 << 22, device="cuda")
    before = s.clone()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    fqlib.fqb_flush(s, s.numel() * 4, sink)
    torch.cuda.synchronize()
    assert torch.equal(before, s)
    assert int(sink.item()) == 0
