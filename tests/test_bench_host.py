"""Host-side checks of bench.py and of the binding's pre-launch guards (CPU only:
no kernel runs; the library's compute entry points are replaced by a recorder)."""
import pytest
import torch

import bench
from fake_quant_amd import fq, synthetic

TINY = {
    "tensor": dict(n=1000),
    "rows_f32": dict(rows=8, cols=40),
    "fp8": dict(n=3001),
    "q4dq": dict(n=20001),
    "rows_bf16": dict(rows=4, cols=64),
}


class RecordingLib:
    """Stands in for libfq.so: host-only helpers go to the real library, compute
    entry points are recorded and report success without launching anything."""

    def __init__(self, real):
        self.real = real
        self.calls = []

    def __getattr__(self, name):
        if name in ("fq_workspace_bytes", "fq_q4dq_sizes", "fq_status_string", "fq_version",
                    "fq_cols_workspace_bytes", "fq_percentile_workspace_bytes"):
            return getattr(self.real, name)

        def rec(*args):
            self.calls.append(name)
            return 0
        return rec


def cpu_need(name, what, t, nbytes):
    if t is None or isinstance(t, int):
        return
    assert t.is_contiguous(), (name, what)
    have = t.numel() * t.element_size()
    assert have >= nbytes, f"{name}: {what} holds {have} bytes, the call touches {nbytes}"


def test_every_bench_op_passes_buffers_that_fit(monkeypatch):
    monkeypatch.setattr(synthetic, "FULL", TINY)
    recorder = RecordingLib(fq.lib())
    monkeypatch.setattr(fq, "_lib", recorder)
    monkeypatch.setattr(fq, "_need", cpu_need)
    monkeypatch.setattr(fq, "_stream", lambda stream=None: None)
    ops = bench.build_ops(fq, synthetic, torch, None, dev="cpu")
    assert len(ops) == 15
    # built largest first, timed in WORKLOADS order
    assert sorted(bench.BUILD_ORDER) == sorted(bench.WORKLOADS)
    groups = [op.name.split(".")[0] for op in ops]
    assert [g for i, g in enumerate(groups) if i == 0 or groups[i - 1] != g] == list(bench.WORKLOADS)
    for op in ops:
        op.fn()
    assert len(recorder.calls) == 15
    assert sum(op.nbytes for op in ops) > 0


def test_next_rows_pass_buffers_that_fit(monkeypatch):
    monkeypatch.setattr(synthetic, "FULL", TINY)
    recorder = RecordingLib(fq.lib())
    monkeypatch.setattr(fq, "_lib", recorder)
    monkeypatch.setattr(fq, "_need", cpu_need)
    monkeypatch.setattr(fq, "_stream", lambda stream=None: None)
    groups = bench.build_next_ops(fq, synthetic, torch, dev="cpu")
    ops = [op for g in groups.values() for op in g]
    assert [op.name for op in ops] == ["tensor.params_int8_sym", "tensor.fake_quant_int8", "sr.fake_quant_int8", "sr.fp8_quantize_e4m3", "sr.fp8_quantize_e5m2",
                                       "qat.step_int8_sym", "qat.step_fp8_e4m3", "cols.int8_sym", "cols.int4_affine",
                                       "cols.bf16_int8_affine",
                                       "percentile.tensor_2^20", "percentile.weights_2^24",
                                       "groups.f32_int4_g128", "groups.f32_int8_g32", "groups.bf16_int8_g128",
                                       "block.mxfp4_e2m1", "block.mxfp6_e2m3", "block.nvfp4"]
    before = len(recorder.calls)
    for op in ops:
        op.fn()
    assert recorder.calls[before:] == ["fq_tensor_params_int", "fq_fake_quant_int_tensor", "fq_fake_quant_int_tensor_sr", "fq_fp8_quantize_sr", "fq_fp8_quantize_sr",
                                       "fq_qat_step_int", "fq_qat_step_fp8", "fq_quant_cols", "fq_quant_cols", "fq_quant_cols",
                                       "fq_tensor_params_percentile", "fq_tensor_params_percentile",
                                       "fq_quant_groups", "fq_quant_groups", "fq_quant_groups",
                                       "fq_mx_rows", "fq_mx_rows", "fq_nvfp4"]


def test_binding_guards_reject_bad_buffers():
    x = torch.zeros(16)
    with pytest.raises(fq.FqError, match="not a GPU tensor"):
        fq.fq_fp8_quantize(x, 16, fq.E4M3, x[:1], None, x)
    fq_need = fq._need
    # size and contiguity checks (checked ahead of the device check on a fake view)
    class Fake:
        is_cuda = True
        def __init__(self, n, contig=True):
            self.n, self.contig = n, contig
        def is_contiguous(self):
            return self.contig
        def numel(self):
            return self.n
        def element_size(self):
            return 4
    with pytest.raises(fq.FqError, match="holds 60 bytes"):
        fq_need("f", "out", Fake(15), 64)
    with pytest.raises(fq.FqError, match="not contiguous"):
        fq_need("f", "out", Fake(16, contig=False), 64)
    fq_need("f", "out", Fake(16), 64)


def test_raise_on_flags_maps_bits_to_errors():
    # the flag word read on the host: no bit -> no error; each bit -> FqFlagError
    fq.raise_on_flags("op", torch.zeros(1, dtype=torch.int32))
    with pytest.raises(fq.FqFlagError, match="Inf or NaN") as e:
        fq.raise_on_flags("op", torch.tensor([fq.FLAG_NONFINITE], dtype=torch.int32))
    assert e.value.status == fq.FLAG_NONFINITE
    with pytest.raises(fq.FqFlagError, match="no usable range"):
        fq.raise_on_flags("op", torch.tensor([fq.FLAG_DEGENERATE], dtype=torch.int32))
    with pytest.raises(fq.FqFlagError, match="Inf or NaN; .*no usable range"):
        fq.raise_on_flags("op", torch.tensor([3], dtype=torch.int32))
    assert issubclass(fq.FqFlagError, fq.FqError)
