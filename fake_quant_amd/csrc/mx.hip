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
// Vector path (cols a multiple of 32, aligned buffers): a block is 64 bytes of
// bf16 = four 16-byte lane loads (a DPP quad) or 128 bytes of fp32 = eight lanes;
// one 16-byte vector per thread over a grid covering the flattened tensor.
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

__device__ __forceinline__ uint32_t fin_abs(float v) {
    uint32_t a = as_u(v) & 0x7FFFFFFFu;
    return a < 0x7F800000u ? a : 0u;
}

template <int DT>
__global__ __launch_bounds__(kB) void k_mx_vec(const void* __restrict__ x, int64_t nvec,
                                               uint8_t* __restrict__ q, uint8_t* __restrict__ e8,
                                               float* __restrict__ fq) {
    constexpr int N = DT == FQ_F32 ? 4 : 8;       // elements per lane
    constexpr int L = kMx / N;                     // lanes per block
    const int64_t stride = (int64_t)gridDim.x * kB;
    for (int64_t gv = (int64_t)blockIdx.x * kB + threadIdx.x; gv < nvec; gv += stride) {
        float xe[N];
        if (DT == FQ_F32) {
            float4 v = reinterpret_cast<const float4*>(x)[gv];
            xe[0] = v.x; xe[1] = v.y; xe[2] = v.z; xe[3] = v.w;
        } else {
            uint4 w = reinterpret_cast<const uint4*>(x)[gv];
            xe[0] = bf16_lo(w.x); xe[1] = bf16_hi(w.x); xe[2] = bf16_lo(w.y); xe[3] = bf16_hi(w.y);
            xe[4] = bf16_lo(w.z); xe[5] = bf16_hi(w.z); xe[6] = bf16_lo(w.w); xe[7] = bf16_hi(w.w);
        }
        uint32_t am = 0;
#pragma unroll
        for (int e = 0; e < N; ++e) am = max(am, fin_abs(xe[e]));
        am = quad_max_u(am);
        if (L == 8) am = max(am, dpp_u<kHalfMirror>(am));
        const int xe_exp = mx_exp(am);
        uint32_t w[N / 4];
#pragma unroll
        for (int e = 0; e < N; e += 4)
            w[e / 4] = fp8_encode4_hw<0>(__builtin_amdgcn_ldexpf(xe[e], -xe_exp),
                                         __builtin_amdgcn_ldexpf(xe[e + 1], -xe_exp),
                                         __builtin_amdgcn_ldexpf(xe[e + 2], -xe_exp),
                                         __builtin_amdgcn_ldexpf(xe[e + 3], -xe_exp));
        if (DT == FQ_F32) {
            reinterpret_cast<uint32_t*>(q)[gv] = w[0];
        } else {
            reinterpret_cast<uint2*>(q)[gv] = make_uint2(w[0], w[(N / 4) - 1]);
        }
        if ((gv % L) == 0) e8[gv / L] = (uint8_t)(xe_exp + 127);
        if (fq) {
            // decode * X = ldexp(decode, xe); the NaN code decodes to NaN
            float4* fv = reinterpret_cast<float4*>(fq) + gv * (N / 4);
#pragma unroll
            for (int h = 0; h < N / 4; ++h) {
                float d[4];
                fp8_decode4_hw<0>(w[h], d);
                store_nt(fv + h, make_float4(__builtin_amdgcn_ldexpf(d[0], xe_exp), __builtin_amdgcn_ldexpf(d[1], xe_exp),
                                             __builtin_amdgcn_ldexpf(d[2], xe_exp), __builtin_amdgcn_ldexpf(d[3], xe_exp)));
            }
        }
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
        for (int64_t c = c0; c < c1; ++c) am = max(am, fin_abs(ld(c)));
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
    const int N = dtype == FQ_F32 ? 4 : 8;
    const bool al = (cols % kMx == 0) && fqh::aligned(x, 16) && fqh::aligned(q, dtype == FQ_F32 ? 4 : 8) &&
                    fqh::aligned(fq, 16);
    if (al) {
        const int64_t nvec = rows * cols / N;
        const unsigned G = fqh::grid_all(nvec, kB);
        if (dtype == FQ_F32) k_mx_vec<FQ_F32><<<G, kB, 0, stream>>>(x, nvec, q, e8m0, fq);
        else k_mx_vec<FQ_BF16><<<G, kB, 0, stream>>>(x, nvec, q, e8m0, fq);
    } else {
        const int64_t total = rows * ((cols + kMx - 1) / kMx);
        const unsigned G = fqh::grid_for(total, kB, 8);
        if (dtype == FQ_F32) k_mx_any<FQ_F32><<<G, kB, 0, stream>>>(x, rows, cols, q, e8m0, fq);
        else k_mx_any<FQ_BF16><<<G, kB, 0, stream>>>(x, rows, cols, q, e8m0, fq);
    }
    return fqh::launched();
}

}  // extern "C"
