#!/usr/bin/env python3
"""Benchmark of the fake-quant hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME ...] [--no-cpu] [--no-cold] [--no-next] [--copy-ref]

One step runs every operation of the path once, each on the full-size synthetic
input of its workload (all inputs resident in HBM before timing starts):

  tensor    per-tensor symmetric int8 of 2^20 N(0,1) fp32: calibration and fake-quant
            (codes + fq) in one call, STE backward
  rows_f32  per-row int8 / int4, symmetric / affine of a [4096, 4096] fp32 weight
            (codes + fq + scale + zero-point)
  fp8       finite-amax scale, E4M3 and E5M2 quantize (bytes + fq) and dequantize
            of 2^26 log-uniform fp32 with +-Inf / NaN / zeros
  q4dq      64-element 4-bit blocks + double-quantized scales of 2^30 Student-t
            fp32 (packed + u8 scales + super-scales + reconstruction), dequantize
  rows_bf16 per-token affine int8 and 32-element E4M3 blocks with E8M0 scales of a
            [16384, 8192] bf16 ReLU activation with outlier channels

`value` = algorithmic bytes of the step (each contract input read once, each
output written once) / measured step time, in GB/s; `roofline` is the dominant
kernel's achieved bandwidth against the 8 TB/s HBM peak; `kernels` gives every
op's share of the timed steps; `per_op_cold_warm` times each op on its own with
its inputs evicted from the caches (cold) and back to back (warm);
`copy_f32_ceiling` is a plain device copy timed the same ways (also at the smaller
workloads' input sizes, under `by_size`); `next_rows`
times the rows beyond the step (the per-tensor calibration and fake-quant as two
separate calls, stochastic rounding, the QAT optimizer step, per-column,
percentile and group-wise calibration, the FP4 / FP6 block formats)
the same ways, outside `value`; `cpu_baseline` is the CPU oracle over every step
workload at full size on the host's cores (the per-tensor and per-row ones also on
one thread), and `parity` compares every step op's GPU outputs with its results
(`value` is null when any differs).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "effective GB/s of quantize/fake-quant kernels; % of MI355X HBM peak"
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_SUMMARY = "bench_step_all_workloads_hbm_traffic.txt"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", nargs="*", default=None,
                    help="restrict to workloads: tensor rows_f32 fp8 q4dq rows_bf16 (step), "
                         "tensor_calls stochastic_rounding qat_step per_column percentile group_wise block_formats "
                         "(beside the step)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-cold", action="store_true", help="skip the per-op cold / warm timings")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the rows beyond the step (stochastic rounding, QAT step, calibration variants, "
                         "block formats), timed cold / warm on their own")
    ap.add_argument("--copy-ref", action="store_true",
                    help="only run COPY_REF_LAUNCHES plain device copies of COPY_REF_BYTES each, torch's and then "
                         "the library's copy kernel (the known-size reference that scales HBM counter readings) "
                         "and exit")
    return ap.parse_args()


COPY_REF_BYTES = 1 << 30
COPY_REF_LAUNCHES = 3


def copy_reference(torch, fq):
    """Plain copies of a known size: each launch reads and writes exactly
    COPY_REF_BYTES, so the FETCH_SIZE / WRITE_SIZE counters read for it give the
    factor from counter units to bytes.  First torch's device copy, then the
    library's plain copy kernel (fqb_copy_f32, the achievable-bandwidth reference
    that other counters of the kernels are compared with)."""
    src = torch.ones(COPY_REF_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(COPY_REF_LAUNCHES):
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy {i} of {COPY_REF_BYTES} bytes done")
    for i in range(COPY_REF_LAUNCHES):
        fq.fqb_copy_f32(src, dst, COPY_REF_BYTES // 4)
        torch.cuda.synchronize()
        log(f"fqb_copy_f32 {i} of {COPY_REF_BYTES} bytes done")
    print(json.dumps({"copy_ref_bytes": COPY_REF_BYTES, "launches": COPY_REF_LAUNCHES,
                      "kernels": ["torch device copy", "fqb_copy_f32"]}))


class Op:
    """One timed call: `fn` enqueues it, `nbytes` are its algorithmic bytes; `ins`
    and `outs` name its GPU input and output tensors (the parity check reads
    them after the timings)."""
    def __init__(self, name, kernel, fn, nbytes, ins=None, outs=None):
        self.name, self.kernel, self.fn, self.nbytes = name, kernel, fn, nbytes
        self.ins, self.outs = ins or {}, outs or {}


def ops_tensor(fq, syn, torch, dev):
    n = syn.FULL["tensor"]["n"]
    x, g = syn.tensor_inputs(n, device=dev)
    wsb = fq.fq_workspace_bytes(n)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    params = torch.empty(4, dtype=torch.int32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    codes = torch.empty(n, dtype=torch.int8, device=dev)
    fqo = torch.empty(n, dtype=torch.float32, device=dev)
    gin = torch.empty(n, dtype=torch.float32, device=dev)
    bounds = params.view(torch.float32)[2:4]
    # calibration (reduction + parameters) and fake-quant in the one call that
    # does both in two launches; the STE reads the bounds that call stores
    return [
        Op("tensor.calibrate_fake_quant_int8", "k_reduce_partial+k_fq_int_tensor_fold",
           lambda: fq.fq_calibrate_fake_quant_int_tensor(x, n, 8, fq.SYM, ws, wsb, params, codes, fqo, flags),
           4 * n + 16 + n + 4 * n, ins=dict(x=x), outs=dict(params=params, codes=codes, fq=fqo, flags=flags)),
        Op("tensor.ste_backward", "k_ste", lambda: fq.fq_ste_backward(g, n, x, n, bounds, gin), 12 * n,
           ins=dict(x=x, g=g), outs=dict(grad_in=gin)),
    ]


def ops_next_tensor_calls(fq, syn, torch, dev):
    """The per-tensor calibration and fake-quant of the step as two separate calls
    (three launches), measured beside the step."""
    n = syn.FULL["tensor"]["n"]
    x, _ = syn.tensor_inputs(n, device=dev)
    wsb = fq.fq_workspace_bytes(n)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    params = torch.empty(4, dtype=torch.int32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    codes = torch.empty(n, dtype=torch.int8, device=dev)
    fqo = torch.empty(n, dtype=torch.float32, device=dev)
    return [
        Op("tensor.params_int8_sym", "k_reduce_partial+k_params_int_final",
           lambda: fq.fq_tensor_params_int(x, n, 8, fq.SYM, ws, wsb, params, flags), 4 * n + 16),
        Op("tensor.fake_quant_int8", "k_fq_int_tensor",
           lambda: fq.fq_fake_quant_int_tensor(x, n, 8, fq.SYM, params, codes, fqo), 4 * n + n + 4 * n),
    ]


def op_rows_f32(fq, torch, w, r, c, bits, scheme, sname, dev):
    cb = r * c if bits == 8 else r * ((c + 1) // 2)
    codes = torch.empty(cb, dtype=torch.uint8, device=dev)
    fqo = torch.empty(r * c, dtype=torch.float32, device=dev)
    sc = torch.empty(r, dtype=torch.float32, device=dev)
    zp = torch.empty(r, dtype=torch.int32, device=dev)
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    return Op(f"rows_f32.int{bits}_{sname}", "k_rows_wg",
              lambda: fq.fq_quant_rows(w, fq.F32, r, c, bits, scheme, codes, fqo, sc, zp, fl),
              4 * r * c + cb + 4 * r * c + 8 * r, ins=dict(x=w),
              outs=dict(codes=codes, fq=fqo, scale=sc, zp=zp, flags=fl))


def ops_rows_f32(fq, syn, torch, dev):
    r, c = syn.FULL["rows_f32"]["rows"], syn.FULL["rows_f32"]["cols"]
    w = syn.rows_f32_inputs(r, c, device=dev)
    return [op_rows_f32(fq, torch, w, r, c, bits, scheme, sname, dev)
            for bits in (8, 4) for scheme, sname in ((fq.SYM, "sym"), (fq.AFFINE, "affine"))]


def ops_fp8_format(fq, torch, x, n, scales, fmt, fname, dev):
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    fqo = torch.empty(n, dtype=torch.float32, device=dev)
    deq = torch.empty(n, dtype=torch.float32, device=dev)
    s = scales[fmt:fmt + 1]
    return [Op(f"fp8.quantize_{fname}", "k_fp8_quant", lambda: fq.fq_fp8_quantize(x, n, fmt, s, q, fqo),
               4 * n + n + 4 * n, ins=dict(x=x), outs=dict(q=q, fq=fqo)),
            Op(f"fp8.dequantize_{fname}", "k_fp8_dequant_w", lambda: fq.fq_fp8_dequantize(q, n, fmt, s, deq),
               n + 4 * n, outs=dict(out=deq))]


def ops_fp8(fq, syn, torch, dev):
    n = syn.FULL["fp8"]["n"]
    x = syn.fp8_inputs(n, device=dev)
    wsb = fq.fq_workspace_bytes(n)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    scales = torch.empty(2, dtype=torch.float32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    ops = [Op("fp8.tensor_scale", "k_reduce_partial+k_fp8_scale_final",
              lambda: fq.fq_fp8_tensor_scale(x, n, ws, wsb, scales[0:1], scales[1:2], flags), 4 * n + 8,
              ins=dict(x=x), outs=dict(scales=scales, flags=flags))]
    for fmt, fname in ((fq.E4M3, "e4m3"), (fq.E5M2, "e5m2")):
        ops += ops_fp8_format(fq, torch, x, n, scales, fmt, fname, dev)
    return ops


def ops_q4dq(fq, syn, torch, dev):
    n = syn.FULL["q4dq"]["n"]
    x = syn.q4dq_inputs(n, device=dev)
    npk, nb, ns = fq.fq_q4dq_sizes(n)
    packed = torch.empty(npk, dtype=torch.uint8, device=dev)
    qs = torch.empty(nb, dtype=torch.uint8, device=dev)
    sup = torch.empty(ns, dtype=torch.float32, device=dev)
    recon = torch.empty(n, dtype=torch.float32, device=dev)
    deq = torch.empty(n, dtype=torch.float32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    return [
        Op("q4dq.quantize_recon", "k_q4dq_full",
           lambda: fq.fq_q4dq_quantize(x, n, packed, qs, sup, None, recon, flags),
           4 * n + npk + nb + 4 * ns + 4 * n, ins=dict(x=x),
           outs=dict(packed=packed, qscale=qs, super=sup, recon=recon, flags=flags)),
        Op("q4dq.dequantize", "k_q4dq_dequant_full",
           lambda: fq.fq_q4dq_dequantize(packed, qs, sup, n, deq), npk + nb + 4 * ns + 4 * n, outs=dict(out=deq)),
    ]


def ops_rows_bf16(fq, syn, torch, dev):
    r, c = syn.FULL["rows_bf16"]["rows"], syn.FULL["rows_bf16"]["cols"]
    a = syn.rows_bf16_inputs(r, c, device=dev)
    codes = torch.empty(r * c, dtype=torch.int8, device=dev)
    sc = torch.empty(r, dtype=torch.float32, device=dev)
    zp = torch.empty(r, dtype=torch.int32, device=dev)
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    q = torch.empty(r * c, dtype=torch.uint8, device=dev)
    e8 = torch.empty(r * ((c + 31) // 32), dtype=torch.uint8, device=dev)
    return [
        Op("rows_bf16.int8_affine", "k_rows_wg",
           lambda: fq.fq_quant_rows(a, fq.BF16, r, c, 8, fq.AFFINE, codes, None, sc, zp, fl),
           2 * r * c + r * c + 8 * r, ins=dict(x=a), outs=dict(codes=codes, scale=sc, zp=zp, flags=fl)),
        Op("rows_bf16.mxfp8_e4m3", "k_mx_wide",
           lambda: fq.fq_mxfp8_rows(a, fq.BF16, r, c, q, e8, None), 2 * r * c + r * c + r * c // 32,
           ins=dict(x=a), outs=dict(q=q, e8m0=e8)),
    ]


WORKLOADS = {"tensor": ops_tensor, "rows_f32": ops_rows_f32, "fp8": ops_fp8, "q4dq": ops_q4dq,
             "rows_bf16": ops_rows_bf16}


def ops_next_sr(fq, syn, torch, dev):
    """Stochastic rounding ([QAT] RoundingMode::Stochastic), measured beside the
    step but not part of it: per-tensor int8 fake-quant of the 2^20 tensor and
    fp8 E4M3 / E5M2 quantize of the 2^26 fp8 workload; the parameters and scales
    are calibrated once at set-up."""
    n1 = syn.FULL["tensor"]["n"]
    x1, _ = syn.tensor_inputs(n1, device=dev)
    wsb1 = fq.fq_workspace_bytes(n1)
    ws1 = torch.empty(wsb1 // 4, dtype=torch.float32, device=dev)
    params = torch.empty(4, dtype=torch.int32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    fq.fq_tensor_params_int(x1, n1, 8, fq.SYM, ws1, wsb1, params, flags)
    codes = torch.empty(n1, dtype=torch.int8, device=dev)
    fq1 = torch.empty(n1, dtype=torch.float32, device=dev)
    n = syn.FULL["fp8"]["n"]
    x = syn.fp8_inputs(n, device=dev)
    wsb = fq.fq_workspace_bytes(n)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    scales = torch.empty(2, dtype=torch.float32, device=dev)
    fq.fq_fp8_tensor_scale(x, n, ws, wsb, scales[0:1], scales[1:2], flags)
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    fqo = torch.empty(n, dtype=torch.float32, device=dev)
    seed = 0x5EED
    ops = [Op("sr.fake_quant_int8", "k_fq_int_tensor_sr",
              lambda: fq.fq_fake_quant_int_tensor_sr(x1, n1, 8, fq.SYM, params, seed, 0, codes, fq1), 9 * n1)]
    for fmt, fname in ((fq.E4M3, "e4m3"), (fq.E5M2, "e5m2")):
        s = scales[fmt:fmt + 1]
        ops.append(Op(f"sr.fp8_quantize_{fname}", "k_fp8_quant_sr",
                      lambda s=s, fmt=fmt: fq.fq_fp8_quantize_sr(x, n, fmt, s, seed, 0, q, fqo), 9 * n))
    return ops


def ops_next_qat(fq, syn, torch, dev):
    """One QAT optimizer step ([QAT] QatOptimizer::step) on the [4096, 4096] fp32
    weight workload as master: AdamW update, then the int8 symmetric view
    (recalibrated per tensor) or the fp8 E4M3 view.  Contract bytes per element:
    read master, grad, m, v (16); write master, m, v, view (16) and the codes or
    bytes (1)."""
    r, c = syn.FULL["rows_f32"]["rows"], syn.FULL["rows_f32"]["cols"]
    n = r * c
    w = syn.rows_f32_inputs(r, c, device=dev).reshape(-1)
    g = syn.rows_f32_inputs(r, c, device=dev, seed=7).reshape(-1)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    v = torch.zeros(n, dtype=torch.float32, device=dev)
    cfg = fq.adamw_config(1e-4, weight_decay=0.01)
    wsb = fq.fq_workspace_bytes(n)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    params = torch.empty(4, dtype=torch.int32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    codes = torch.empty(n, dtype=torch.int8, device=dev)
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    view = torch.empty(n, dtype=torch.float32, device=dev)
    t = 10
    return [
        Op("qat.step_int8_sym", "k_adamw_minmax+k_fq_int_tensor_fold_gs",
           lambda: fq.fq_qat_step_int(w, g, m, v, n, cfg, t, 8, fq.SYM, fq.ROUND_NEAREST, 0, 0, ws, wsb, params,
                                      codes, view, flags), 33 * n),
        Op("qat.step_fp8_e4m3", "k_adamw_fp8",
           lambda: fq.fq_qat_step_fp8(w, g, m, v, n, cfg, t, fq.E4M3, fq.ROUND_NEAREST, 0, 0, q, view), 33 * n),
    ]


def ops_next_cols(fq, syn, torch, dev):
    """Per-column (axis 1) calibration + int8 / int4 quantize of the [4096, 4096]
    fp32 weight workload (codes, fake-quant, scale and zero-point per column)."""
    r, c = syn.FULL["rows_f32"]["rows"], syn.FULL["rows_f32"]["cols"]
    w = syn.rows_f32_inputs(r, c, device=dev)
    wsb = fq.fq_cols_workspace_bytes(r, c)
    ws = torch.empty(max(wsb // 4, 1), dtype=torch.float32, device=dev)
    fqo = torch.empty(r * c, dtype=torch.float32, device=dev)
    scale = torch.empty(c, dtype=torch.float32, device=dev)
    zp = torch.empty(c, dtype=torch.int32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    ops = []
    for bits, scheme, name in ((8, fq.SYM, "int8_sym"), (4, fq.AFFINE, "int4_affine")):
        nb = r * c if bits == 8 else r * ((c + 1) // 2)
        codes = torch.empty(nb, dtype=torch.uint8, device=dev)
        ops.append(Op(f"cols.{name}", "k_cols_strip",
                      lambda bits=bits, scheme=scheme, codes=codes: fq.fq_quant_cols(
                          w, fq.F32, r, c, bits, scheme, ws, wsb, codes, fqo, scale, zp, flags),
                      4 * r * c + nb + 4 * r * c + 8 * c))
    # per-channel int8 of a bf16 activation: 4096 tokens of the [*, 8192] ReLU
    # workload with its outlier channels
    ra, ca = 4096, syn.FULL["rows_bf16"]["cols"]
    a = syn.rows_bf16_inputs(ra, ca, device=dev)
    wsba = fq.fq_cols_workspace_bytes(ra, ca)
    wsa = torch.empty(max(wsba // 4, 1), dtype=torch.float32, device=dev)
    fqa = torch.empty(ra * ca, dtype=torch.float32, device=dev)
    sca = torch.empty(ca, dtype=torch.float32, device=dev)
    zpa = torch.empty(ca, dtype=torch.int32, device=dev)
    ca8 = torch.empty(ra * ca, dtype=torch.uint8, device=dev)
    ops.append(Op("cols.bf16_int8_affine", "k_cols_strip",
                  lambda: fq.fq_quant_cols(a, fq.BF16, ra, ca, 8, fq.AFFINE, wsa, wsba, ca8, fqa, sca, zpa, flags),
                  2 * ra * ca + ra * ca + 4 * ra * ca + 8 * ca))
    return ops


def ops_next_percentile(fq, syn, torch, dev):
    """Percentile calibration ([QAT] QuantParams::per_tensor_percentile, clip
    fraction 0.001, int8 affine) of the 2^20 tensor and of the [4096, 4096] fp32
    weights flattened; the algorithmic bytes are one read of the tensor, which the
    radix selection reads twice at 2^20 and once at 2^24 (where a sample predicts
    the candidates)."""
    params = torch.empty(4, dtype=torch.int32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    n1 = syn.FULL["tensor"]["n"]
    x1, _ = syn.tensor_inputs(n1, device=dev)
    r, c = syn.FULL["rows_f32"]["rows"], syn.FULL["rows_f32"]["cols"]
    w = syn.rows_f32_inputs(r, c, device=dev)
    ops = []
    for name, x, n in (("tensor_2^20", x1, n1), ("weights_2^24", w, r * c)):
        wsb = fq.fq_percentile_workspace_bytes(n)
        ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
        ops.append(Op(f"percentile.{name}", "k_pct_init+k_pct_first+k_pct_second+k_pct_third+k_pct_final",
                      lambda x=x, n=n, ws=ws, wsb=wsb: fq.fq_tensor_params_percentile(
                          x, n, 8, fq.AFFINE, 0.001, ws, wsb, params, flags),
                      4 * n + 16))
    return ops


def ops_next_groups(fq, syn, torch, dev):
    """Group-wise quantization along rows ([CS] demo 3 granularity): the
    [4096, 4096] fp32 weights in INT4 groups of 128 and INT8 groups of 32, and
    the bf16 activations in INT8 groups of 128 (codes, fake-quant, and a scale
    and zero-point per group)."""
    ops = []
    r, c = syn.FULL["rows_f32"]["rows"], syn.FULL["rows_f32"]["cols"]
    w = syn.rows_f32_inputs(r, c, device=dev)
    rb, cb = syn.FULL["rows_bf16"]["rows"], syn.FULL["rows_bf16"]["cols"]
    a = syn.rows_bf16_inputs(rb, cb, device=dev)
    for name, x, dt, rows, cols, group, bits in (("f32_int4_g128", w, fq.F32, r, c, 128, 4),
                                                 ("f32_int8_g32", w, fq.F32, r, c, 32, 8),
                                                 ("bf16_int8_g128", a, fq.BF16, rb, cb, 128, 8)):
        ng = (cols + group - 1) // group
        nb = rows * cols if bits == 8 else rows * ((cols + 1) // 2)
        codes = torch.empty(nb, dtype=torch.uint8, device=dev)
        fqo = torch.empty(rows * cols, dtype=torch.float32, device=dev)
        scale = torch.empty(rows * ng, dtype=torch.float32, device=dev)
        zp = torch.empty(rows * ng, dtype=torch.int32, device=dev)
        flags = torch.zeros(1, dtype=torch.int32, device=dev)
        esz = 4 if dt == fq.F32 else 2
        ops.append(Op(f"groups.{name}", "k_groups_wide",
                      lambda x=x, dt=dt, rows=rows, cols=cols, group=group, bits=bits, codes=codes, fqo=fqo,
                      scale=scale, zp=zp, flags=flags: fq.fq_quant_groups(
                          x, dt, rows, cols, group, bits, fq.SYM, codes, fqo, scale, zp, flags),
                      esz * rows * cols + nb + 4 * rows * cols + 8 * rows * ng))
    return ops


def ops_next_block_formats(fq, syn, torch, dev):
    """FP4 / FP6 block formats ([CS] demo 4): MXFP4 (E2M1) and MXFP6 (E2M3) with
    E8M0 scales per 32 on the [16384, 8192] bf16 activations, and NVFP4 (E2M1,
    E4M3 scales per 16, fp32 tensor scale) on the 2^26 fp8-workload tensor (its
    tensor amax pass counted as one more read)."""
    ops = []
    rb, cb = syn.FULL["rows_bf16"]["rows"], syn.FULL["rows_bf16"]["cols"]
    a = syn.rows_bf16_inputs(rb, cb, device=dev)
    fqo = torch.empty(rb * cb, dtype=torch.float32, device=dev)
    e8 = torch.empty(rb * ((cb + 31) // 32), dtype=torch.uint8, device=dev)
    for name, elem, qb in (("mxfp4_e2m1", fq.E2M1, rb * ((cb + 1) // 2)), ("mxfp6_e2m3", fq.E2M3, rb * cb)):
        q = torch.empty(qb, dtype=torch.uint8, device=dev)
        ops.append(Op(f"block.{name}", "k_mxn_wide",
                      lambda elem=elem, q=q: fq.fq_mx_rows(a, fq.BF16, rb, cb, elem, q, e8, fqo),
                      2 * rb * cb + qb + rb * ((cb + 31) // 32) + 4 * rb * cb))
    n = syn.FULL["fp8"]["n"]
    x = syn.fp8_inputs(n, device=dev)
    wsb = fq.fq_workspace_bytes(n)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    q4 = torch.empty((n + 1) // 2, dtype=torch.uint8, device=dev)
    sb = torch.empty((n + 15) // 16, dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    fqn = torch.empty(n, dtype=torch.float32, device=dev)
    ops.append(Op("block.nvfp4", "k_reduce_partial+k_amax_final+k_nvfp4_wide",
                  lambda: fq.fq_nvfp4(x, n, ws, wsb, q4, sb, g, fqn),
                  4 * n + 4 * n + (n + 1) // 2 + (n + 15) // 16 + 4 * n))
    return ops


NEXT_WORKLOADS = {"tensor_calls": ops_next_tensor_calls, "stochastic_rounding": ops_next_sr, "qat_step": ops_next_qat, "per_column": ops_next_cols,
                  "percentile": ops_next_percentile, "group_wise": ops_next_groups,
                  "block_formats": ops_next_block_formats}


def build_next_ops(fq, syn, torch, only=None, dev="cuda"):
    """The rows beyond the step (measured on their own, not counted in `value`),
    those named in `only` if given."""
    return {name: make(fq, syn, torch, dev) for name, make in NEXT_WORKLOADS.items()
            if only is None or name in only}


# Workloads are built largest first: the 4-bit workload's 4 GiB buffers, placed
# after the others, made its quantize kernel measurably slower (1575 against
# 1520 us on MI355X, the same kernel and bytes).  The ops run in WORKLOADS order.
BUILD_ORDER = ["q4dq", "rows_bf16", "fp8", "rows_f32", "tensor"]


def build_ops(fq, syn, torch, only, dev="cuda"):
    """Draw inputs and allocate outputs on the GPU, one workload per function (each
    op's closure owns that workload's buffers); return the timed ops in WORKLOADS
    order."""
    built = {}
    for name in BUILD_ORDER:
        if only is None or name in only:
            built[name] = WORKLOADS[name](fq, syn, torch, dev)
    return [op for name in WORKLOADS for op in built.get(name, [])]


FLUSH_BYTES = 1 << 30
COLD_REPS, WARM_REPS, PRE_REPS = 20, 20, 5


def _median_min(ms):
    ms = sorted(ms)
    return ms[len(ms) // 2], ms[0]


def _timed_reps(fn, reps, torch, stream, before=None):
    """HIP events around each of `reps` launches of fn (after `before`, if given),
    enqueued back to back and read after one synchronisation."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        if before is not None:
            before()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def cold_warm(ops, fq, torch, stream, ceiling=True):
    """Every op on its own, cold (a 1 GiB read of scratch before each repetition
    evicts its inputs from L2 and the Infinity Cache) and warm (back to back);
    median and minimum over the repetitions.  Also the plain-copy ceiling."""
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    flush = lambda: fq.fqb_flush(scratch, FLUSH_BYTES, sink)
    res = {}
    for op in ops:
        for _ in range(PRE_REPS):
            op.fn()
        warm = _timed_reps(op.fn, WARM_REPS, torch, stream)
        cold = _timed_reps(op.fn, COLD_REPS, torch, stream, before=flush)
        (cm, cmin), (wm, wmin) = _median_min(cold), _median_min(warm)
        res[op.name] = dict(cold_us=round(cm * 1e3, 2), cold_us_min=round(cmin * 1e3, 2),
                            cold_gbs=round(op.nbytes / (cm * 1e-3) / 1e9, 1),
                            cold_frac=round(op.nbytes / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            warm_us=round(wm * 1e3, 2), warm_us_min=round(wmin * 1e3, 2),
                            warm_gbs=round(op.nbytes / (wm * 1e-3) / 1e9, 1),
                            warm_frac=round(op.nbytes / (wm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        res[op.name]["kernel"] = op.kernel
        res[op.name]["bytes"] = op.nbytes
    if not ceiling:
        del scratch
        return res, None
    n = COPY_REF_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copy = lambda: fq.fqb_copy_f32(src, dst, n)
    for _ in range(PRE_REPS):
        copy()
    nbytes = 2 * COPY_REF_BYTES
    (cm, _), (wm, _) = (_median_min(_timed_reps(copy, COLD_REPS, torch, stream, before=flush)),
                        _median_min(_timed_reps(copy, WARM_REPS, torch, stream)))
    ceiling = dict(kernel="fqb_copy_f32", bytes=nbytes, cold_gbs=round(nbytes / (cm * 1e-3) / 1e9, 1),
                   warm_gbs=round(nbytes / (wm * 1e-3) / 1e9, 1),
                   cold_frac=round(nbytes / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    # the same copy at the input sizes of the smaller workloads (2^20 f32 tensor,
    # [4096, 4096] f32 rows, 2^26 f32 fp8 tensor): what a plain stream of that size
    # reaches, launch and ramp included
    by_size = {}
    for k in (20, 24, 26):
        m = 1 << k
        copy_m = lambda m=m: fq.fqb_copy_f32(src, dst, m)
        for _ in range(PRE_REPS):
            copy_m()
        (cm, _), (wm, _) = (_median_min(_timed_reps(copy_m, COLD_REPS, torch, stream, before=flush)),
                            _median_min(_timed_reps(copy_m, WARM_REPS, torch, stream)))
        nb = 8 * m
        by_size[f"2^{k} f32"] = dict(bytes=nb, cold_us=round(cm * 1e3, 2), warm_us=round(wm * 1e3, 2),
                                     cold_frac=round(nb / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                     warm_frac=round(nb / (wm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    ceiling["by_size"] = by_size
    del scratch, src, dst
    return res, ceiling


def _ranges(n, parts, align=1):
    """[lo, hi) ranges covering [0, n): at most `parts` of them, every boundary
    but the last a multiple of `align`."""
    step = -(-n // max(parts, 1))
    step = max(align, -(-step // align) * align)
    return [(lo, min(n, lo + step)) for lo in range(0, n, step)]


def oracle_threads():
    """Host cores the oracle leg uses: those this process may run on, at most 16
    (one GPU's share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


class OracleLeg:
    """Runs the CPU oracle over the step's workloads and checks the GPU outputs
    against it.  Work is split over `threads` host threads by rows, elements or
    16384-element super-blocks: every output of the oracle depends only on its
    own row, element or super-block (the per-tensor reductions are max / min, and
    the max of the ranges' maxima is the maximum), so the split gives the serial
    result; the per-tensor and per-row workloads also run on one thread and are
    compared with the split run.  ctypes releases the GIL around each oracle
    call, so the threads run in parallel."""

    def __init__(self, orc, threads):
        from concurrent.futures import ThreadPoolExecutor
        self.orc, self.threads = orc, threads
        self.pool = ThreadPoolExecutor(threads)
        self.times = {}        # op -> dict(bytes, seconds[, seconds_1thread])
        self.checks = {}       # op -> {output: mismatches}
        self.serial_same = {}  # op -> split run identical to the single-thread run

    def split(self, n, align, fn, threads=None):
        T = threads or self.threads
        rs = _ranges(n, T, align)
        if T == 1:
            return [fn(a, b) for a, b in rs]
        return list(self.pool.map(lambda r: fn(*r), rs))

    def timed(self, op, fn, key="seconds"):
        t0 = time.perf_counter()
        out = fn()
        self.times.setdefault(op.name, dict(bytes=op.nbytes))[key] = time.perf_counter() - t0
        return out

    # --- comparisons (the stated bars: bytes and integers bit-exact; binary32
    # outputs within 1 ulp with +0 == -0 and NaN == NaN; the kernels aim at
    # bit-exact, which is counted as well) ---
    def _chunks(self, n, fn):
        return sum(self.split(n, 1 << 22, fn))

    def exact(self, op, what, gpu, ref):
        import numpy as np
        a = np.ascontiguousarray(gpu).reshape(-1).view(np.uint8)
        e = np.ascontiguousarray(ref).reshape(-1).view(np.uint8)
        if a.size != e.size:
            bad = -1  # a size mismatch counts as a failure
        else:
            bad = self._chunks(a.size, lambda lo, hi: int(np.count_nonzero(a[lo:hi] != e[lo:hi])))
        self.checks.setdefault(op.name, {})[what] = bad

    def f32(self, op, what, gpu, ref):
        import numpy as np
        a = np.ascontiguousarray(gpu, dtype=np.float32).reshape(-1).view(np.uint32)
        e = np.ascontiguousarray(ref, dtype=np.float32).reshape(-1).view(np.uint32)
        if a.size != e.size:
            self.checks.setdefault(op.name, {})[what] = -1
            return

        def count(lo, hi):
            x, y = a[lo:hi], e[lo:hi]
            xn = (x & 0x7FFFFFFF) > 0x7F800000
            yn = (y & 0x7FFFFFFF) > 0x7F800000
            diff = ~((x == y) | (xn & yn))
            idx = np.nonzero(diff)[0]
            if idx.size == 0:
                return 0, 0
            xi, yi = x[idx].astype(np.int64), y[idx].astype(np.int64)
            ox = np.where(xi >= 1 << 31, (1 << 31) - xi, xi)  # order-preserving, +0 == -0
            oy = np.where(yi >= 1 << 31, (1 << 31) - yi, yi)
            far = (xn[idx] != yn[idx]) | (np.abs(ox - oy) > 1)
            return int(idx.size), int(np.count_nonzero(far))

        rs = self.split(a.size, 1 << 22, count)
        not_exact, beyond = sum(r[0] for r in rs), sum(r[1] for r in rs)
        rec = self.checks.setdefault(op.name, {})
        rec[what] = beyond
        if not_exact:
            rec[what + "_not_bit_exact"] = not_exact

    def ok(self, op):
        return all(v == 0 for k, v in self.checks.get(op.name, {"missing": 1}).items()
                   if not k.endswith("_not_bit_exact"))


def _host(t):
    return t.detach().cpu().numpy()


def oracle_tensor(leg, ops):
    import numpy as np
    orc = leg.orc
    opc, ops_ = ops["tensor.calibrate_fake_quant_int8"], ops["tensor.ste_backward"]
    x, g = _host(opc.ins["x"]), _host(ops_.ins["g"])
    n = x.size

    def calibrate_fq(T):
        p = orc.tensor_params_int(x, 8, orc.SYM)
        codes, fqv = np.empty(n, np.int8), np.empty(n, np.float32)
        leg.split(n, 1, lambda a, b: orc.fake_quant_int(x[a:b], 8, orc.SYM, float(p["scale"]), p["zp"],
                                                         codes=codes[a:b], fq=fqv[a:b]), T)
        return p, codes, fqv

    def ste(p, T):
        out = np.empty(n, np.float32)
        leg.split(n, 1, lambda a, b: orc.ste_backward(g[a:b], x[a:b], float(p["lo"]), float(p["hi"]), out=out[a:b]), T)
        return out

    p, codes, fqv = leg.timed(opc, lambda: calibrate_fq(leg.threads))
    p1, codes1, fqv1 = leg.timed(opc, lambda: calibrate_fq(1), key="seconds_1thread")
    gin = leg.timed(ops_, lambda: ste(p, leg.threads))
    gin1 = leg.timed(ops_, lambda: ste(p, 1), key="seconds_1thread")
    leg.serial_same[opc.name] = bool(np.array_equal(codes, codes1) and np.array_equal(fqv.view(np.uint32),
                                                                                       fqv1.view(np.uint32)))
    leg.serial_same[ops_.name] = bool(np.array_equal(gin.view(np.uint32), gin1.view(np.uint32)))
    want = np.array([np.float32(p["scale"]).view(np.int32), p["zp"], np.float32(p["lo"]).view(np.int32),
                     np.float32(p["hi"]).view(np.int32)], np.int32)
    leg.exact(opc, "params", _host(opc.outs["params"]), want)
    leg.exact(opc, "flags", _host(opc.outs["flags"]), np.array([p["flags"]], np.int32))
    leg.exact(opc, "codes", _host(opc.outs["codes"]), codes)
    leg.f32(opc, "fq", _host(opc.outs["fq"]), fqv)
    leg.f32(ops_, "grad_in", _host(ops_.outs["grad_in"]), gin)


def oracle_rows_f32(leg, ops):
    import numpy as np
    orc = leg.orc
    names = [k for k in ops if k.startswith("rows_f32.")]
    x = _host(ops[names[0]].ins["x"])
    rows, cols = x.shape
    for name in names:
        op = ops[name]
        bits = 8 if "int8" in name else 4
        scheme = orc.SYM if name.endswith("_sym") else orc.AFFINE

        def run(T, bits=bits, scheme=scheme):
            cw = cols if bits == 8 else (cols + 1) // 2
            codes = np.empty((rows, cw), np.int8 if bits == 8 else np.uint8)
            fqv = np.empty((rows, cols), np.float32)
            sc, zp = np.empty(rows, np.float32), np.empty(rows, np.int32)
            fl = leg.split(rows, 1, lambda a, b: orc.quant_rows(x[a:b], bits, scheme, codes=codes[a:b], fq=fqv[a:b],
                                                                 scale=sc[a:b], zp=zp[a:b])["flags"], T)
            return codes, fqv, sc, zp, int(np.bitwise_or.reduce(fl))

        codes, fqv, sc, zp, fl = leg.timed(op, lambda: run(leg.threads))
        r1 = leg.timed(op, lambda: run(1), key="seconds_1thread")
        leg.serial_same[name] = bool(all(np.array_equal(u.view(np.uint8), v.view(np.uint8))
                                         for u, v in zip((codes, fqv, sc, zp), r1[:4])) and fl == r1[4])
        leg.exact(op, "codes", _host(op.outs["codes"]), codes)
        leg.f32(op, "fq", _host(op.outs["fq"]), fqv)
        leg.exact(op, "scale", _host(op.outs["scale"]), sc)
        leg.exact(op, "zp", _host(op.outs["zp"]), zp)
        leg.exact(op, "flags", _host(op.outs["flags"]), np.array([fl], np.int32))


def oracle_fp8(leg, ops):
    import numpy as np
    orc = leg.orc
    ops_ = ops["fp8.tensor_scale"]
    x = _host(ops_.ins["x"])
    n = x.size

    def scales():
        amax = max(leg.split(n, 1, lambda a, b: float(orc.amax_finite(x[a:b]))))
        return [orc.fp8_scale(amax, fmt) for fmt in (orc.E4M3, orc.E5M2)]

    sc = leg.timed(ops_, scales)
    leg.exact(ops_, "scales", _host(ops_.outs["scales"]), np.array([sc[0][0], sc[1][0]], np.float32))
    leg.exact(ops_, "flags", _host(ops_.outs["flags"]), np.array([sc[0][1] | sc[1][1]], np.int32))
    for fmt, fname in ((orc.E4M3, "e4m3"), (orc.E5M2, "e5m2")):
        s = float(sc[fmt][0])
        opq, opd = ops[f"fp8.quantize_{fname}"], ops[f"fp8.dequantize_{fname}"]
        q, fqv, deq = np.empty(n, np.uint8), np.empty(n, np.float32), np.empty(n, np.float32)
        leg.timed(opq, lambda: leg.split(n, 1, lambda a, b: orc.fp8_quantize(x[a:b], fmt, s, q=q[a:b], fq=fqv[a:b])))
        leg.timed(opd, lambda: leg.split(n, 1, lambda a, b: orc.fp8_dequantize(q[a:b], fmt, s, out=deq[a:b])))
        leg.exact(opq, "q", _host(opq.outs["q"]), q)
        leg.f32(opq, "fq", _host(opq.outs["fq"]), fqv)
        leg.f32(opd, "out", _host(opd.outs["out"]), deq)
        del q, fqv, deq


def oracle_q4dq(leg, ops):
    import numpy as np
    orc = leg.orc
    opq, opd = ops["q4dq.quantize_recon"], ops["q4dq.dequantize"]
    x = _host(opq.ins["x"])
    n = x.size
    npk, nb, ns = orc.q4dq_sizes(n)
    packed, qs = np.empty(npk, np.uint8), np.empty(nb, np.uint8)
    sup, recon = np.empty(ns, np.float32), np.empty(n, np.float32)
    SB = 16384  # a super-block: 256 blocks of 64

    def quant(a, b):
        return orc.q4dq_quantize(x[a:b], want_block_scale=False, packed=packed[a // 2:(b + 1) // 2],
                                 qscale=qs[a // 64:(b + 63) // 64], sup=sup[a // SB:(b + SB - 1) // SB],
                                 recon=recon[a:b])["flags"]

    fl = leg.timed(opq, lambda: leg.split(n, SB, quant))
    deq = np.empty(n, np.float32)
    leg.timed(opd, lambda: leg.split(n, SB, lambda a, b: orc.q4dq_dequantize(
        packed[a // 2:(b + 1) // 2], qs[a // 64:(b + 63) // 64], sup[a // SB:(b + SB - 1) // SB], b - a,
        out=deq[a:b])))
    leg.exact(opq, "packed", _host(opq.outs["packed"]), packed)
    leg.exact(opq, "qscale", _host(opq.outs["qscale"]), qs)
    leg.exact(opq, "super", _host(opq.outs["super"]), sup)
    leg.exact(opq, "flags", _host(opq.outs["flags"]), np.array([int(np.bitwise_or.reduce(fl))], np.int32))
    leg.f32(opq, "recon", _host(opq.outs["recon"]), recon)
    del recon
    leg.f32(opd, "out", _host(opd.outs["out"]), deq)


def oracle_rows_bf16(leg, ops):
    import numpy as np
    import torch
    orc = leg.orc
    opr, opm = ops["rows_bf16.int8_affine"], ops["rows_bf16.mxfp8_e4m3"]
    a = _host(opr.ins["x"].view(torch.int16)).view(np.uint16)
    rows, cols = a.shape
    codes, sc, zp = np.empty((rows, cols), np.int8), np.empty(rows, np.float32), np.empty(rows, np.int32)
    fl = leg.timed(opr, lambda: leg.split(rows, 1, lambda lo, hi: orc.quant_rows(
        a[lo:hi], 8, orc.AFFINE, dtype=orc.BF16, want_fq=False, codes=codes[lo:hi], scale=sc[lo:hi],
        zp=zp[lo:hi])["flags"]))
    leg.exact(opr, "codes", _host(opr.outs["codes"]), codes)
    leg.exact(opr, "scale", _host(opr.outs["scale"]), sc)
    leg.exact(opr, "zp", _host(opr.outs["zp"]), zp)
    leg.exact(opr, "flags", _host(opr.outs["flags"]), np.array([int(np.bitwise_or.reduce(fl))], np.int32))
    q, e8 = np.empty((rows, cols), np.uint8), np.empty((rows, (cols + 31) // 32), np.uint8)
    leg.timed(opm, lambda: leg.split(rows, 1, lambda lo, hi: orc.mxfp8_rows(
        a[lo:hi], dtype=orc.BF16, want_fq=False, q=q[lo:hi], e8m0=e8[lo:hi])))
    leg.exact(opm, "q", _host(opm.outs["q"]), q)
    leg.exact(opm, "e8m0", _host(opm.outs["e8m0"]), e8)


ORACLE = {"tensor": oracle_tensor, "rows_f32": oracle_rows_f32, "fp8": oracle_fp8, "q4dq": oracle_q4dq,
          "rows_bf16": oracle_rows_bf16}
SINGLE_THREAD_ROWS = ("tensor", "rows_f32")


def cpu_baseline_and_parity(orc, ops):
    """The oracle over every step workload at full size (about 13 s of CPU work),
    on the host's cores, and the parity of every step op's GPU outputs against
    it.  Returns (cpu_baseline, parity)."""
    leg = OracleLeg(orc, oracle_threads())
    by_wl = {}
    for op in ops:
        by_wl.setdefault(op.name.split(".")[0], {})[op.name] = op
    for wl, wops in by_wl.items():
        log(f"oracle + parity: {wl}")
        ORACLE[wl](leg, wops)
    leg.pool.shutdown()
    total_b = sum(t["bytes"] for t in leg.times.values())
    total_s = sum(t["seconds"] for t in leg.times.values())
    per_op = {}
    for name, t in leg.times.items():
        rec = dict(seconds=round(t["seconds"], 4), gbs=round(t["bytes"] / t["seconds"] / 1e9, 3))
        if "seconds_1thread" in t:
            rec.update(seconds_1thread=round(t["seconds_1thread"], 4),
                       gbs_1thread=round(t["bytes"] / t["seconds_1thread"] / 1e9, 3))
        per_op[name] = rec
    per_wl = {}
    for wl, wops in by_wl.items():
        b = sum(leg.times[n]["bytes"] for n in wops)
        sec = sum(leg.times[n]["seconds"] for n in wops)
        per_wl[wl] = dict(seconds=round(sec, 4), gbs=round(b / sec / 1e9, 3))
        if wl in SINGLE_THREAD_ROWS:
            s1 = sum(leg.times[n]["seconds_1thread"] for n in wops)
            per_wl[wl].update(seconds_1thread=round(s1, 4), gbs_1thread=round(b / s1 / 1e9, 3))
    cpu = dict(value=round(total_b / total_s / 1e9, 4), unit="GB/s", cores=leg.threads, kind="oracle",
               sample=f"every step workload at full size ({', '.join(by_wl)}), split over {leg.threads} host "
                      f"threads by rows, elements or 16384-element super-blocks ({total_s:.1f} s wall); the "
                      f"per-tensor and per-row workloads also on one thread",
               seconds=round(total_s, 3), per_workload=per_wl, per_op=per_op,
               split_equals_serial=all(leg.serial_same.values()), host=host_cpu())
    parity = dict(ok=all(leg.ok(op) for op in ops),
                  workloads={wl: all(leg.ok(op) for op in wops.values()) for wl, wops in by_wl.items()},
                  mismatches=leg.checks,
                  bar="codes, bytes, nibbles, u8 scales, params and flags bit-exact; float32 outputs within "
                      "1 ulp (+0 == -0, NaN == NaN), counts of not bit-exact ones kept beside")
    return cpu, parity


def host_cpu():
    """The host the oracle ran on: cores this process may use, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(cores_available=len(os.sched_getaffinity(0)), cpu_model=model)


SMI_KEYS = ("clock", "temperature", "power", "serial", "perf")


def smi_snapshot():
    """The GPU's clocks, temperatures, power limit and serial as rocm-smi reports
    them (the fields of card 0 whose names mention one of SMI_KEYS), or None
    where rocm-smi is missing or fails.  Read from sysfs by a child process; it
    does not touch the GPU's queues."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showtemp", "--showmaxpower", "--showpower",
                            "--showserial", "--showperflevel", "--json"],
                           capture_output=True, text=True, timeout=20)
        card = json.loads(r.stdout).get("card0", {})
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    return {k: v for k, v in card.items() if any(w in k.lower() for w in SMI_KEYS)} or None


def device_info(torch):
    """Static properties of cuda:0 as torch reports them."""
    p = torch.cuda.get_device_properties(0)
    return dict(name=p.name, arch=getattr(p, "gcnArchName", None), compute_units=p.multi_processor_count,
                total_memory=p.total_memory)


def traffic_record(kernel):
    """HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE, scaled by the
    copy reference) from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(PROFILES, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != sources_sha(kernel):
        return None
    try:
        return float(rec[f"hbm_bytes_per_launch[{kernel}]"])
    except (KeyError, ValueError):
        return None


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/|\s+', re.S)


def code_only(text):
    """C / C++ source with its comments removed and every run of whitespace
    folded to one space (string and character literals kept as they are), so
    that editing a comment does not count as a change of the kernel."""
    def keep(m):
        t = m.group(0)
        if t[0] in "\"'":
            return t
        return "\0"
    return re.sub("\0+", " ", _CODE_TOKENS.sub(keep, text)).strip()


def sources_sha(kernel):
    """sha256 over the code (comments and layout left out) of the sources
    `kernel` is built from: the .hip file(s) that define it, every header of the
    package and the public header."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fake_quant_amd", "csrc")
    files = []
    for f in sorted(os.listdir(csrc)):
        p = os.path.join(csrc, f)
        if f.endswith(".h") or (f.endswith(".hip") and kernel.encode() in open(p, "rb").read()):
            files.append(p)
    files.append(os.path.join(ROOT, "include", "fq.h"))
    for p in files:
        h.update(os.path.basename(p).encode())
        h.update(code_only(open(p, encoding="utf-8").read()).encode())
    return h.hexdigest()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (there is no multi-GPU path); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from fake_quant_amd import fq
    from fake_quant_amd import synthetic as syn

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_ref:
        copy_reference(torch, fq)
        return
    log("drawing inputs and allocating outputs")
    ops = build_ops(fq, syn, torch, args.only)
    if not ops:
        # only rows beyond the step were asked for
        next_rows = {name: cold_warm(nops, fq, torch, torch.cuda.current_stream(), ceiling=False)[0]
                     for name, nops in build_next_ops(fq, syn, torch, args.only).items()}
        print(json.dumps({"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1,
                          "config": {"workload": "only " + ",".join(args.only)}, "next_rows": next_rows}),
              flush=True)
        return
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"{len(ops)} ops per step; warmup {args.warmup}")
    for op in ops:  # first pass one op at a time, so a failure names its op
        log(f"first call: {op.name}")
        op.fn()
        torch.cuda.synchronize()
    smi_before = smi_snapshot()  # before the warm-up steps, which bring the clocks back up
    for _ in range(args.warmup):
        for op in ops:
            op.fn()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_wall = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, op in enumerate(ops):
            op.fn()
            ev[s][i + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    smi_after = smi_snapshot()
    total_ms = start.elapsed_time(end)
    per_op_ms = [sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
                 for i in range(len(ops))]
    step_bytes = sum(op.nbytes for op in ops)
    ms_step = total_ms / args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9

    kernels = {}
    for op, ms in zip(ops, per_op_ms):
        gbs = op.nbytes / (ms * 1e-3) / 1e9
        kernels[op.name] = dict(kernel=op.kernel, bytes=op.nbytes, us=round(ms * 1e3, 2), gbs=round(gbs, 1),
                                frac=round(gbs / HBM_PEAK_GBS, 4))
    dom_i = max(range(len(ops)), key=lambda i: per_op_ms[i])
    dom = ops[dom_i]
    achieved = dom.nbytes / (per_op_ms[dom_i] * 1e-3) / 1e9
    roofline = dict(bound="hbm", kernel=dom.kernel, op=dom.name, achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic_record(dom.kernel),
                    avg_launch_us=round(per_op_ms[dom_i] * 1e3, 2), bytes_per_launch=dom.nbytes)

    per_op, copy_ceiling = None, None
    if not args.no_cold:
        log("per-op cold / warm timings and the copy ceiling")
        per_op, copy_ceiling = cold_warm(ops, fq, torch, stream)
    next_rows = None
    if not args.no_next and (args.only is None or any(w in NEXT_WORKLOADS for w in args.only)):
        log("rows beyond the step, cold / warm")
        next_rows = {name: cold_warm(nops, fq, torch, stream, ceiling=False)[0]
                     for name, nops in build_next_ops(fq, syn, torch, args.only).items()}
        torch.cuda.synchronize()

    cpu, parity = None, None
    n_ops = len(ops)
    if not args.no_cpu:
        from oracle import oracle as orc
        log("the CPU oracle over every step workload, and the parity of the GPU outputs against it")
        cpu, parity = cpu_baseline_and_parity(orc, ops)
        if not parity["ok"]:
            log(f"PARITY FAILED: {parity['mismatches']}")

    workloads = "tensor 2^20 f32 int8 calibrate + fake-quant + STE; rows_f32 [4096,4096] int8/int4 sym/affine; fp8 2^26 E4M3/E5M2; " \
                "q4dq 2^30 f32 4-bit + double-quant; rows_bf16 [16384,8192] per-token int8 + 32-block E4M3/E8M0"
    if args.only:
        workloads = "only " + ",".join(args.only)
    out = {
        "metric": METRIC,
        # a step whose outputs differ from the oracle's has no valid throughput
        "value": round(value, 1) if parity is None or parity["ok"] else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "config": {"workload": workloads, "bytes_per_step": step_bytes, "ops_per_step": n_ops,
                   "wall_s_timed": round(t_wall, 3)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "kernels": kernels,
        "per_op_cold_warm": per_op,
        "copy_f32_ceiling": copy_ceiling,
        "next_rows": next_rows,
        # what the box reported before the warm-up steps and right after the timed ones
        "device": dict(device_info(torch), smi_before=smi_before, smi_after_timed=smi_after),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
