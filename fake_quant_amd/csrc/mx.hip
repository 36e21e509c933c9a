// mx.hip -- 32-element fp8 E4M3 blocks with power-of-two (E8M0) scales along rows.
//
// [CS] CS349E 05_quantization_basics.py, demo 4 `block_scaled(x, FP8_E4M3, 32,
// "e8m0")`: per block, amax (0 treated as 1), k = frexp exponent of amax,
// X = 2^(k - 1 - emax) with emax = 8 for E4M3 (448 = 1.75 * 2^8); elements go
// through the saturating E4M3 cast of x / X and come back as cast * X.
// The E4M3 cast is the one of [QAT] fake_quant_fp8 (optirs-gpu quantization.rs).
//
// Dividing by X = 2^e is a pure exponent shift, so fl(x / X) = ldexp(x, -e) and
// fl(decode * X) = ldexp(decode, e): no division runs here.
//
// Vector path (cols a multiple of 32, aligned buffers): the wide layout, sixteen
// elements per lane and a block of 32 per lane pair, over a grid covering the
// flattened tensor; against one 16-byte vector per lane it runs the [16384, 8192]
// bf16 workload in 62.9 instead of 70.9 us (cold).
#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;
constexpr int kMx = 32;
constexpr int kE4M3Emax = 8;

// exponent of X for a block whose finite amax has bits `am`
__device__ __forceinline__ int mx_exp(uint32_t am) {
    float A = am == 0u ? 1.0f : as_f(am);
    int k = __builtin_amdgcn_frexp_expf(A);
    return max(k - 1 - kE4M3Emax, -127);
}

__device__ __forceinline__ float mx_value(uint32_t b, int xe) {
    float v = __builtin_amdgcn_ldexpf(fp8_decode_finite<0>(b), xe);
    return b == 0x7Fu ? __builtin_nanf("") : v;
}

// Wide layout (cols a multiple of 32, aligned buffers): lane v holds elements
// 16 v .. 16 v + 15, a block is a lane pair reduced with one DPP exchange; codes
// leave as 16 bytes per lane, the fake-quant values through the LDS transpose.
// Every thread of the grid reaches the reduction and the barrier.
template <int DT>
__global__ __launch_bounds__(kB) void k_mx_wide(const void* __restrict__ x, int64_t nw, uint8_t* __restrict__ q,
                                                uint8_t* __restrict__ e8, float* __restrict__ fq) {
    __shared__ float4 s_out[kB / kWave][kWave * kWidePad / 4];
    const int64_t v = (int64_t)blockIdx.x * kB + threadIdx.x;
    const bool in = v < nw;
    float xe[kWide];
    if (in) {
        load16<DT == FQ_BF16, true>(x, v, xe);
    } else {
#pragma unroll
        for (int i = 0; i < kWide; ++i) xe[i] = 0.0f;
    }
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < kWide; ++i) am = max(am, finite_abs_bits(xe[i]));
    am = max(am, dpp_u<kQuadXor1>(am));
    const int xe_exp = mx_exp(am);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = fp8_encode4_hw<0>(__builtin_amdgcn_ldexpf(xe[4 * k], -xe_exp), __builtin_amdgcn_ldexpf(xe[4 * k + 1], -xe_exp),
                                 __builtin_amdgcn_ldexpf(xe[4 * k + 2], -xe_exp), __builtin_amdgcn_ldexpf(xe[4 * k + 3], -xe_exp));
    if (in) {
        // codes with the nontemporal hint: measured over the bench step (three runs
        // each, one box), the ops after this one find fewer dirty lines to write
        // back and the step took 2.8645-2.8651 ms against 2.8713-2.8779 ms with plain
        // stores, though this op alone, cold, slowed from 75.9 to 72.5 % of 8 TB/s
        __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(q) + v);
        if ((v & 1) == 0) e8[v >> 1] = (uint8_t)(xe_exp + 127);
    }
    if (fq) {
        // decode * X = ldexp(decode, xe); the NaN code decodes to NaN
        float o[kWide];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float d[4];
            fp8_decode4_hw<0>(w[k], d);
#pragma unroll
            for (int i = 0; i < 4; ++i) o[4 * k + i] = __builtin_amdgcn_ldexpf(d[i], xe_exp);
        }
        store16_staged(reinterpret_cast<float4*>(fq), v, nw, o, s_out[threadIdx.x / kWave]);
    }
}

// Any shape / alignment: one thread per block of a row (partial block at the end).
template <int DT>
__global__ __launch_bounds__(kB) void k_mx_any(const void* __restrict__ x, int64_t rows, int64_t cols,
                                               uint8_t* __restrict__ q, uint8_t* __restrict__ e8,
                                               float* __restrict__ fq) {
    const int64_t nbr = (cols + kMx - 1) / kMx;
    const int64_t total = rows * nbr;
    for (int64_t g = (int64_t)blockIdx.x * kB + threadIdx.x; g < total; g += (int64_t)gridDim.x * kB) {
        const int64_t r = g / nbr, b = g % nbr;
        const int64_t c0 = b * kMx;
        const int64_t c1 = c0 + kMx < cols ? c0 + kMx : cols;
        auto ld = [&](int64_t c) -> float {
            int64_t i = r * cols + c;
            if (DT == FQ_F32) return reinterpret_cast<const float*>(x)[i];
            return as_f((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
        };
        uint32_t am = 0;
        for (int64_t c = c0; c < c1; ++c) am = max(am, finite_abs_bits(ld(c)));
        const int xe_exp = mx_exp(am);
        e8[g] = (uint8_t)(xe_exp + 127);
        for (int64_t c = c0; c < c1; ++c) {
            uint32_t byte = fp8_encode<0>(__builtin_amdgcn_ldexpf(ld(c), -xe_exp));
            q[r * cols + c] = (uint8_t)byte;
            if (fq) fq[r * cols + c] = mx_value(byte, xe_exp);
        }
    }
}

}  // namespace

extern "C" {

int fq_mxfp8_rows(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q, uint8_t* e8m0,
                  float* fq, hipStream_t stream) {
    if (!fqh::valid_dtype(dtype)) return FQ_E_UNSUPPORTED;
    if (!x || rows < 1 || cols < 1 || !q || !e8m0) return FQ_E_INVALID;
    if (!fqh::aligned(x, dtype == FQ_F32 ? 4 : 2) || !fqh::aligned(fq, 4)) return FQ_E_INVALID;
    const int64_t nw = rows * cols / kWide;
    const bool al = (cols % kMx == 0) && fqh::aligned(x, 16) && fqh::aligned(q, 16) && fqh::aligned(fq, 16);
    if (al && nw / kB < 0x7FFFFFFFLL) {
        const unsigned G = (unsigned)((nw + kB - 1) / kB);
        if (dtype == FQ_F32) k_mx_wide<FQ_F32><<<G, kB, 0, stream>>>(x, nw, q, e8m0, fq);
        else k_mx_wide<FQ_BF16><<<G, kB, 0, stream>>>(x, nw, q, e8m0, fq);
    } else {
        const int64_t total = rows * ((cols + kMx - 1) / kMx);
        const unsigned G = fqh::grid_for(total, kB, 8);
        if (dtype == FQ_F32) k_mx_any<FQ_F32><<<G, kB, 0, stream>>>(x, rows, cols, q, e8m0, fq);
        else k_mx_any<FQ_BF16><<<G, kB, 0, stream>>>(x, rows, cols, q, e8m0, fq);
    }
    return fqh::launched();
}

}  // extern "C"
