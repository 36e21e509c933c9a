"""Seeded synthetic inputs for the five workloads (shared by tests and bench).

This module draws random numbers and nothing else: it holds none of the
quantization arithmetic, and it imports neither the HIP binding nor the CPU
oracle.  Every generator takes a ``device``; a workload is drawn with a
``torch.Generator`` seeded on that device, so the same seed gives the same
tensor on every run on the same kind of device.  Parity checks copy the drawn
tensor to the host for the oracle, so both sides always see identical bytes.

Shapes and value distributions follow the synthetic data the pages themselves
use (CS349E 05_quantization_basics.py demos 1, 3 and 4: ReLU activations,
lognormal per-row weight scales, outlier channels, Student-t weights):

* per-tensor int8 ("tensor"): x, g ~ N(0, 1), 2^20 float32 each.
* per-row weights ("rows_f32"): row r ~ N(0, sigma_r^2), sigma_r = exp(N(-3, 0.5^2)),
  [4096, 4096] float32.
* fp8 cast ("fp8"): sign * 2^u, u ~ U(-20, 20), 2^26 float32, then 0.1 % each of
  +-Inf, NaN and exact zeros at random positions.
* 4-bit double quant ("q4dq"): Student-t(4) * 0.02, 2^30 float32; t(4) is drawn
  as z / sqrt(c / 4) with z ~ N(0, 1) and c = -2 ln(u1 u2) ~ chi-square(4).
* per-token activations ("rows_bf16"): ReLU(N(0, 1)) [16384, 8192], 1 % of the
  channels (82 of 8192) scaled by 50, rounded to bfloat16 (round-to-nearest-even).
"""
from __future__ import annotations

import torch

SEED = 0

FULL = {
    "tensor": dict(n=1 << 20),
    "rows_f32": dict(rows=4096, cols=4096),
    "fp8": dict(n=1 << 26),
    "q4dq": dict(n=1 << 30),
    "rows_bf16": dict(rows=16384, cols=8192),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def tensor_inputs(n: int = 1 << 20, device="cpu", seed: int = SEED):
    """Per-tensor workload: (x, g), both ~N(0, 1) float32 of length n."""
    gen = _gen(device, seed)
    x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    g = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    return x, g


def rows_f32_inputs(rows: int = 4096, cols: int = 4096, device="cpu", seed: int = SEED):
    """Per-row weight matrix with lognormal row sigmas (median sigma ~ 0.05)."""
    gen = _gen(device, seed)
    sigma = torch.exp(torch.randn(rows, 1, generator=gen, device=device) * 0.5 - 3.0)
    w = torch.randn(rows, cols, generator=gen, device=device, dtype=torch.float32)
    return (w * sigma).contiguous()


def fp8_inputs(n: int = 1 << 26, device="cpu", seed: int = SEED, special_frac: float = 0.001):
    """Log-uniform magnitudes 2^U(-20, 20) with random signs, then special values."""
    gen = _gen(device, seed)
    u = torch.rand(n, generator=gen, device=device) * 40.0 - 20.0
    sign = torch.randint(0, 2, (n,), generator=gen, device=device).to(torch.float32) * 2.0 - 1.0
    x = (sign * torch.exp2(u)).to(torch.float32)
    k = int(round(special_frac * n))
    if k > 0:
        perm = torch.randperm(n, generator=gen, device=device)[: 3 * k]
        inf_pos, nan_pos, zero_pos = perm[:k], perm[k:2 * k], perm[2 * k:]
        x[inf_pos] = sign[inf_pos] * float("inf")
        x[nan_pos] = float("nan")
        x[zero_pos] = 0.0
    return x


def q4dq_inputs(n: int = 1 << 30, device="cpu", seed: int = SEED, chunk: int = 1 << 26):
    """Student-t(4) * 0.02, drawn chunk by chunk to bound temporaries."""
    gen = _gen(device, seed)
    out = torch.empty(n, device=device, dtype=torch.float32)
    tiny = torch.finfo(torch.float32).tiny
    for start in range(0, n, chunk):
        m = min(chunk, n - start)
        z = torch.randn(m, generator=gen, device=device)
        u1 = torch.rand(m, generator=gen, device=device)
        u2 = torch.rand(m, generator=gen, device=device)
        chi2 = -2.0 * (torch.log1p(-u1) + torch.log1p(-u2))
        chi2.clamp_(min=tiny)
        out[start:start + m] = z / torch.sqrt(chi2 / 4.0) * 0.02
    return out


def rows_bf16_inputs(rows: int = 16384, cols: int = 8192, device="cpu", seed: int = SEED,
                     outlier_frac: float = 0.01, outlier_gain: float = 50.0):
    """ReLU(N(0,1)) activations with outlier channels, as bfloat16 [rows, cols]."""
    gen = _gen(device, seed)
    a = torch.relu(torch.randn(rows, cols, generator=gen, device=device, dtype=torch.float32))
    k = int(round(outlier_frac * cols))
    if k > 0:
        chans = torch.randperm(cols, generator=gen, device=device)[:k]
        a[:, chans] *= outlier_gain
    return a.to(torch.bfloat16).contiguous()


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bfloat16 tensor's bits (host copy)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view("uint16")
