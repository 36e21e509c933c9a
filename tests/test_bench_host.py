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


def _fill_with_oracle(ops, orc):
    """Write into every step op's output tensors what the oracle gives for its
    inputs, one serial call per op (as a GPU that matches would have)."""
    import numpy as np
    by = {op.name: op for op in ops}

    def put(op, key, arr):
        t = by[op].outs[key]
        t.view(-1).view(torch.uint8).copy_(torch.from_numpy(np.ascontiguousarray(arr).reshape(-1).view(np.uint8)))

    x = by["tensor.calibrate_fake_quant_int8"].ins["x"].numpy()
    g = by["tensor.ste_backward"].ins["g"].numpy()
    p = orc.tensor_params_int(x, 8, orc.SYM)
    c, f = orc.fake_quant_int(x, 8, orc.SYM, float(p["scale"]), p["zp"])
    put("tensor.calibrate_fake_quant_int8", "params",
        np.array([np.float32(p["scale"]).view(np.int32), p["zp"], np.float32(p["lo"]).view(np.int32),
                  np.float32(p["hi"]).view(np.int32)], np.int32))
    put("tensor.calibrate_fake_quant_int8", "flags", np.array([p["flags"]], np.int32))
    put("tensor.calibrate_fake_quant_int8", "codes", c)
    put("tensor.calibrate_fake_quant_int8", "fq", f)
    put("tensor.ste_backward", "grad_in", orc.ste_backward(g, x, float(p["lo"]), float(p["hi"])))
    for name in [k for k in by if k.startswith("rows_f32.")]:
        w = by[name].ins["x"].numpy()
        r = orc.quant_rows(w, 8 if "int8" in name else 4, orc.SYM if name.endswith("_sym") else orc.AFFINE)
        for k in ("codes", "fq", "scale", "zp"):
            put(name, k, r[k])
        put(name, "flags", np.array([r["flags"]], np.int32))
    y = by["fp8.tensor_scale"].ins["x"].numpy()
    amax = float(orc.amax_finite(y))
    sc = [orc.fp8_scale(amax, fmt) for fmt in (orc.E4M3, orc.E5M2)]
    put("fp8.tensor_scale", "scales", np.array([sc[0][0], sc[1][0]], np.float32))
    put("fp8.tensor_scale", "flags", np.array([sc[0][1] | sc[1][1]], np.int32))
    for fmt, fname in ((orc.E4M3, "e4m3"), (orc.E5M2, "e5m2")):
        q, fv = orc.fp8_quantize(y, fmt, float(sc[fmt][0]))
        put(f"fp8.quantize_{fname}", "q", q)
        put(f"fp8.quantize_{fname}", "fq", fv)
        put(f"fp8.dequantize_{fname}", "out", orc.fp8_dequantize(q, fmt, float(sc[fmt][0])))
    z = by["q4dq.quantize_recon"].ins["x"].numpy()
    r = orc.q4dq_quantize(z)
    for k in ("packed", "qscale", "super", "recon"):
        put("q4dq.quantize_recon", k, r[k])
    put("q4dq.quantize_recon", "flags", np.array([r["flags"]], np.int32))
    put("q4dq.dequantize", "out", orc.q4dq_dequantize(r["packed"], r["qscale"], r["super"], z.size))
    a = synthetic.bf16_bits(by["rows_bf16.int8_affine"].ins["x"])
    r = orc.quant_rows(a, 8, orc.AFFINE, dtype=orc.BF16, want_fq=False)
    for k in ("codes", "scale", "zp"):
        put("rows_bf16.int8_affine", k, r[k])
    put("rows_bf16.int8_affine", "flags", np.array([r["flags"]], np.int32))
    m = orc.mxfp8_rows(a, dtype=orc.BF16, want_fq=False)
    put("rows_bf16.mxfp8_e4m3", "q", m["q"])
    put("rows_bf16.mxfp8_e4m3", "e8m0", m["e8m0"])


def test_oracle_leg_checks_every_output(monkeypatch, orc):
    """The bench's oracle leg, split over three threads, finds outputs equal to
    the serial oracle's equal (parity ok, split == serial), and a single flipped
    byte, a 2-ulp float and a wrong flag word each fail their own workload only."""
    monkeypatch.setattr(synthetic, "FULL", TINY)
    recorder = RecordingLib(fq.lib())
    monkeypatch.setattr(fq, "_lib", recorder)
    monkeypatch.setattr(fq, "_need", cpu_need)
    monkeypatch.setattr(fq, "_stream", lambda stream=None: None)
    monkeypatch.setattr(bench, "oracle_threads", lambda: 3)
    ops = bench.build_ops(fq, synthetic, torch, None, dev="cpu")
    assert all(op.outs for op in ops)
    _fill_with_oracle(ops, orc)
    cpu, parity = bench.cpu_baseline_and_parity(orc, ops)
    assert parity["ok"], parity["mismatches"]
    assert set(parity["workloads"]) == set(bench.WORKLOADS)
    assert cpu["cores"] == 3 and cpu["split_equals_serial"]
    assert set(cpu["per_op"]) == {op.name for op in ops}
    assert all("seconds_1thread" in cpu["per_workload"][w] for w in bench.SINGLE_THREAD_ROWS)
    by = {op.name: op for op in ops}
    by["q4dq.quantize_recon"].outs["packed"][17] ^= 1
    rec = by["fp8.quantize_e5m2"].outs["fq"].view(torch.int32)
    rec[5] = rec[5] + 2 if rec[5] != 0 else 2
    by["rows_f32.int4_affine"].outs["flags"][0] ^= 2
    cpu, parity = bench.cpu_baseline_and_parity(orc, ops)
    assert not parity["ok"]
    bad = {w for w, ok in parity["workloads"].items() if not ok}
    assert bad == {"q4dq", "fp8", "rows_f32"}
    assert parity["mismatches"]["q4dq.quantize_recon"]["packed"] == 1
    assert parity["mismatches"]["fp8.quantize_e5m2"]["fq"] == 1
    assert parity["mismatches"]["rows_f32.int4_affine"]["flags"] == 1


def test_ranges_cover_and_align():
    for n, parts, align in [(1, 16, 1), (20001, 3, 16384), (1 << 20, 16, 1), (4096, 16, 1), (5, 16, 1)]:
        rs = bench._ranges(n, parts, align)
        assert rs[0][0] == 0 and rs[-1][1] == n and len(rs) <= parts
        assert all(a[1] == b[0] for a, b in zip(rs, rs[1:]))
        assert all(a % align == 0 for a, _ in rs)


def test_sources_sha_ignores_comments_only():
    # editing a comment or the layout keeps the hash that ties the counter summary
    # to the kernel sources; editing code changes it
    import bench
    base = 'int f(int a) { return a + 1; } // one\n/* two */ const char* s = "/* kept */";\n'
    same = '// header\nint f(int a)\n{\n    return a + 1;  /* changed */\n}\nconst char* s = "/* kept */";'
    other = 'int f(int a) { return a + 2; }\nconst char* s = "/* kept */";'
    strv = 'int f(int a) { return a + 1; } const char* s = "/*  kept */";'
    assert bench.code_only(base) == bench.code_only(same)
    assert bench.code_only(base) != bench.code_only(other)
    assert bench.code_only(base) != bench.code_only(strv)  # string contents are code
