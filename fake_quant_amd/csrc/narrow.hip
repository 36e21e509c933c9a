// narrow.hip -- block-scaled FP4 / FP6 elements: MXFP4 / MXFP6 (E8M0 scale per
// 32 elements along rows) and NVFP4 (E4M3 scale per 16 elements with an fp32
// tensor scale).
//
// [CS] CS349E 05_quantization_basics.py, demo 4 `block_scaled(x, elem, block,
// scale_kind)`:
//   "e8m0": X = 2^(k - 1 - emax) with k the frexp exponent of the block amax
//           (amax 0 taken as 1); elements elem(x / X) * X;
//   "e4m3": g = amax(x) / (elem max * 448); X = E4M3(amax_block / elem max / g)
//           * g with saturation, 1 where that is not > 0; elements elem(x / X) * X.
// The FP4 / FP6 element formats follow the fp8 minifloat rule of [QAT]
// optirs-gpu quantization.rs (fp8_quantize_magnitude: binade step, ties to even,
// saturation) with every code finite: E2M1 (max 6, emax 2, as the demo states),
// E2M3 (max 7.5, emax 2), E3M2 (max 28, emax 4).  Their tables are not on the
// pages; a NaN element becomes +0 (they have no NaN code), +-Inf saturates.
//
// Both run in the wide layout (sixteen consecutive elements per lane, outputs
// through an LDS transpose), so the per-block work is shared by sixteen
// elements: measured against four elements per lane, MXFP4 150 -> 136 us,
// MXFP6 155 -> 143 us, NVFP4 150 -> 137 us on [16384, 8192] bf16 / 2^26 fp32.
// MX: a block of 32 = a lane pair, reduced with one DPP exchange; the
// power-of-two scaling is exact, so x / X is a multiplication by 2^-e.
// NVFP4: a block of 16 = one lane; the tensor amax comes from the shared
// two-pass reduction; x / X is a true quotient (ExactDiv).
#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr float pow2f(int e) {
    float r = 1.0f;
    for (int i = 0; i < e; ++i) r *= 2.0f;
    return r;
}

constexpr int kB = fqh::kBlock;
constexpr int kMxBlock = 32;
constexpr int kNvBlock = 16;

// Element format with EB exponent and MB mantissa bits, bias 2^(EB-1) - 1, all
// codes finite.
template <int EB, int MB>
struct Narrow {
    static constexpr int kBias = (1 << (EB - 1)) - 1;
    static constexpr int kEmax = (1 << EB) - 1 - kBias;
    static constexpr uint32_t kEminField = 127u + 1u - kBias;  // binary32 exponent field of 2^emin
    static constexpr uint32_t kMaxCode = (1u << (EB + MB)) - 1u;
    static constexpr uint32_t kSign = 1u << (EB + MB);
    static constexpr float kMax = (float)((2 << MB) - 1) / (float)(1 << MB) * (float)(1 << kEmax);
    static constexpr float kRebias = pow2f(127 - kBias);

    // sign | magnitude code of y: |y| clamped to the maximum (saturation; a NaN
    // clamps too and is patched below), binade from the exponent field (at least
    // emin), the exact scaled magnitude rounded to even; a rounding carry runs
    // into the exponent field.
    __device__ __forceinline__ static uint32_t encode(float y) {
        const float a = fminf(fabsf(y), kMax);
        const uint32_t E = max(as_u(a) >> 23, kEminField);
        const float k = rintf(__builtin_amdgcn_ldexpf(a, (int)(127u + MB) - (int)E));
        const uint32_t mag = min((uint32_t)k + ((E - kEminField) << MB), kMaxCode);
        const uint32_t code = mag | ((as_u(y) >> 31) << (EB + MB));
        return (y != y) ? 0u : code;
    }
    // value of a code: the magnitude bits under the binary32 exponent field give
    // 2^(E - 127) (1 + M / 2^MB) (a binary32 subnormal for E = 0), and the
    // multiplication by 2^(127 - bias) rebiases exactly
    __device__ __forceinline__ static float decode(uint32_t c) {
        const float v = as_f((c & kMaxCode) << (23 - MB)) * kRebias;
        return as_f(as_u(v) | ((c & kSign) ? 0x80000000u : 0u));
    }
};
using E2M1 = Narrow<2, 1>;
using E2M3 = Narrow<2, 3>;
using E3M2 = Narrow<3, 2>;
static_assert(E2M1::kMax == 6.0f && E2M3::kMax == 7.5f && E3M2::kMax == 28.0f, "format maxima");

// exponent of X = 2^(k - 1 - emax) for a block whose finite amax has bits am
template <class F>
__device__ __forceinline__ int mx_exp(uint32_t am) {
    const float A = am == 0u ? 1.0f : as_f(am);
    return max(__builtin_amdgcn_frexp_expf(A) - 1 - F::kEmax, -127);
}

// MX in the wide layout (cols a multiple of 32, aligned buffers): lane v holds
// elements 16 v .. 16 v + 15, a block is a lane pair.  FP4 codes leave as 8
// bytes per lane, FP6 as 16; the fake-quant values through the LDS transpose.
// Every thread of the grid reaches the reduction and the barrier.
template <int DT, class F>
__global__ __launch_bounds__(kB) void k_mxn_wide(const void* __restrict__ x, int64_t nvec, uint8_t* __restrict__ q,
                                                 uint8_t* __restrict__ e8, float* __restrict__ fq) {
    __shared__ float4 s_out[kB / kWave][kWave * kWidePad / 4];
    const int64_t v = (int64_t)blockIdx.x * kB + threadIdx.x;
    const bool in = v < nvec;
    float e[kWide];
    if (in) {
        load16<DT == FQ_BF16>(x, v, e);
    } else {
#pragma unroll
        for (int i = 0; i < kWide; ++i) e[i] = 0.0f;
    }
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < kWide; ++i) am = max(am, finite_abs_bits(e[i]));
    am = max(am, dpp_u<kQuadXor1>(am));
    const int xe = mx_exp<F>(am);
    const float X = __builtin_amdgcn_ldexpf(1.0f, xe), inv = __builtin_amdgcn_ldexpf(1.0f, -xe);
    uint32_t c[kWide];
    float o[kWide];
#pragma unroll
    for (int i = 0; i < kWide; ++i) {
        c[i] = F::encode(e[i] * inv);
        o[i] = F::decode(c[i]) * X;
    }
    if (in) {
        if constexpr (F::kMaxCode == 7u) {
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int k = 0; k < 8; ++k) w[k / 4] |= ((c[2 * k] << 4) | c[2 * k + 1]) << (8 * (k % 4));
            reinterpret_cast<uint2*>(q)[v] = make_uint2(w[0], w[1]);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = c[4 * k] | (c[4 * k + 1] << 8) | (c[4 * k + 2] << 16) | (c[4 * k + 3] << 24);
            reinterpret_cast<uint4*>(q)[v] = make_uint4(w[0], w[1], w[2], w[3]);
        }
        if ((v & 1) == 0) e8[v >> 1] = (uint8_t)(xe + 127);
    }
    if (fq) store16_staged(reinterpret_cast<float4*>(fq), v, nvec, o, s_out[threadIdx.x / kWave]);
}

// MX, any shape or alignment: one thread per block of a row (a short block at
// the row end); FP4 codes go out a byte at a time, and a block starts on a byte.
template <int DT, class F>
__global__ __launch_bounds__(kB) void k_mxn_any(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                uint8_t* __restrict__ q, uint8_t* __restrict__ e8,
                                                float* __restrict__ fq) {
    const int64_t nbr = (cols + kMxBlock - 1) / kMxBlock;
    const int64_t pstride = (cols + 1) / 2;
    for (int64_t g = (int64_t)blockIdx.x * kB + threadIdx.x; g < rows * nbr; g += (int64_t)gridDim.x * kB) {
        const int64_t r = g / nbr, c0 = (g % nbr) * kMxBlock;
        const int64_t c1 = c0 + kMxBlock < cols ? c0 + kMxBlock : cols;
        uint32_t am = 0;
        for (int64_t c = c0; c < c1; ++c) am = max(am, finite_abs_bits(load_elem<DT == FQ_BF16>(x, r * cols + c)));
        const int xe = mx_exp<F>(am);
        const float X = __builtin_amdgcn_ldexpf(1.0f, xe), inv = __builtin_amdgcn_ldexpf(1.0f, -xe);
        e8[g] = (uint8_t)(xe + 127);
        uint32_t hold = 0;
        for (int64_t c = c0; c < c1; ++c) {
            const uint32_t code = F::encode(load_elem<DT == FQ_BF16>(x, r * cols + c) * inv);
            if (fq) fq[r * cols + c] = F::decode(code) * X;
            if constexpr (F::kMaxCode == 7u) {
                if ((c & 1) == 0) {
                    hold = code << 4;
                    if (c == cols - 1) q[r * pstride + c / 2] = (uint8_t)hold;
                } else {
                    q[r * pstride + c / 2] = (uint8_t)(hold | code);
                }
            } else {
                q[r * cols + c] = (uint8_t)code;
            }
        }
    }
}

template <int DT, class F>
int launch_mx(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* e8, float* fq, hipStream_t st) {
    constexpr bool fp4 = F::kMaxCode == 7u;  // eight code bytes per lane, else sixteen
    const bool al = cols % kMxBlock == 0 && fqh::aligned(x, 16) && fqh::aligned(fq, 16) && fqh::aligned(q, fp4 ? 8 : 16);
    const int64_t nw = rows * (cols / kWide);
    if (al && nw / kB < 0x7FFFFFFFLL) {
        k_mxn_wide<DT, F><<<(unsigned)((nw + kB - 1) / kB), kB, 0, st>>>(x, nw, q, e8, fq);
    } else {
        const int64_t blocks = rows * ((cols + kMxBlock - 1) / kMxBlock);
        k_mxn_any<DT, F><<<fqh::grid_for(blocks, kB, 8), kB, 0, st>>>(x, rows, cols, q, e8, fq);
    }
    return fqh::launched();
}

template <int DT>
int launch_mx_elem(const void* x, int64_t rows, int64_t cols, int elem, uint8_t* q, uint8_t* e8, float* fq,
                   hipStream_t st) {
    if (elem == FQ_E2M1) return launch_mx<DT, E2M1>(x, rows, cols, q, e8, fq, st);
    if (elem == FQ_E2M3) return launch_mx<DT, E2M3>(x, rows, cols, q, e8, fq, st);
    return launch_mx<DT, E3M2>(x, rows, cols, q, e8, fq, st);
}

// ---------------------------------------------------------------------------
// NVFP4
// ---------------------------------------------------------------------------

// scale of a block from its finite amax and the tensor amax, in the page's
// order; *sb gets the E4M3 byte of the block scale
__device__ __forceinline__ float nv_scale(float amax, float tmax, uint32_t* sb) {
    const float g = tmax / (6.0f * 448.0f);
    const float ratio = amax / 6.0f / g;
    *sb = fp8_encode<0>(ratio);
    const float X = fp8_decode<0>(*sb) * g;
    return X > 0.0f ? X : 1.0f;
}

// full blocks of 16 in the wide layout, aligned buffers: lane v holds block v,
// whose scale it derives alone; codes leave as 8 bytes per lane, the fake-quant
// values through the LDS transpose; the first lane also stores the tensor scale.
// Every thread of the grid reaches the barrier.
__global__ __launch_bounds__(kB) void k_nvfp4_wide(const float* __restrict__ x, int64_t nblk,
                                                   const uint32_t* __restrict__ tmax_bits, uint8_t* __restrict__ q,
                                                   uint8_t* __restrict__ sbytes, float* __restrict__ g_out,
                                                   float* __restrict__ fq) {
    __shared__ float4 s_out[kB / kWave][kWave * kWidePad / 4];
    const int64_t v = (int64_t)blockIdx.x * kB + threadIdx.x;
    const bool in = v < nblk;
    float e[kWide];
    if (in) {
        load16<false>(x, v, e);
    } else {
#pragma unroll
        for (int i = 0; i < kWide; ++i) e[i] = 0.0f;
    }
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < kWide; ++i) am = max(am, finite_abs_bits(e[i]));
    const float tmax = as_f(*tmax_bits);
    if (v == 0) *g_out = tmax / (6.0f * 448.0f);
    uint32_t sb;
    const float X = nv_scale(as_f(am), tmax, &sb);
    const ExactDiv d(X);
    uint32_t c[kWide];
    float o[kWide];
#pragma unroll
    for (int i = 0; i < kWide; ++i) {
        c[i] = E2M1::encode(d(e[i]));
        o[i] = E2M1::decode(c[i]) * X;
    }
    if (in) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k / 4] |= ((c[2 * k] << 4) | c[2 * k + 1]) << (8 * (k % 4));
        reinterpret_cast<uint2*>(q)[v] = make_uint2(w[0], w[1]);
        sbytes[v] = (uint8_t)sb;
    }
    if (fq) store16_staged(reinterpret_cast<float4*>(fq), v, nblk, o, s_out[threadIdx.x / kWave]);
}

// blocks [b0, nblocks) of the flat tensor, any alignment: one thread per block
// (the last one short when n % 16 != 0)
__global__ __launch_bounds__(kB) void k_nvfp4_any(const float* __restrict__ x, int64_t n, int64_t b0,
                                                  const uint32_t* __restrict__ tmax_bits, uint8_t* __restrict__ q,
                                                  uint8_t* __restrict__ sbytes, float* __restrict__ g_out,
                                                  float* __restrict__ fq) {
    const int64_t nb = (n + kNvBlock - 1) / kNvBlock;
    const float tmax = as_f(*tmax_bits);
    for (int64_t b = b0 + (int64_t)blockIdx.x * kB + threadIdx.x; b < nb; b += (int64_t)gridDim.x * kB) {
        if (b == 0) *g_out = tmax / (6.0f * 448.0f);
        const int64_t i0 = b * kNvBlock, i1 = i0 + kNvBlock < n ? i0 + kNvBlock : n;
        uint32_t am = 0;
        for (int64_t i = i0; i < i1; ++i) am = max(am, finite_abs_bits(x[i]));
        uint32_t sb;
        const float X = nv_scale(as_f(am), tmax, &sb);
        const ExactDiv d(X);
        sbytes[b] = (uint8_t)sb;
        uint32_t hold = 0;
        for (int64_t i = i0; i < i1; ++i) {
            const uint32_t code = E2M1::encode(d(x[i]));
            if (fq) fq[i] = E2M1::decode(code) * X;
            if ((i & 1) == 0) {
                hold = code << 4;
                if (i == n - 1) q[i / 2] = (uint8_t)hold;
            } else {
                q[i / 2] = (uint8_t)(hold | code);
            }
        }
    }
}

}  // namespace

extern "C" {

int fq_mx_rows(const void* x, int dtype, int64_t rows, int64_t cols, int elem, uint8_t* q, uint8_t* e8m0,
               float* fq, hipStream_t stream) {
    if (elem == FQ_E4M3) return fq_mxfp8_rows(x, dtype, rows, cols, q, e8m0, fq, stream);
    if (!fqh::valid_dtype(dtype) || !(elem == FQ_E2M1 || elem == FQ_E2M3 || elem == FQ_E3M2)) return FQ_E_UNSUPPORTED;
    if (!x || rows < 1 || cols < 1 || !q || !e8m0) return FQ_E_INVALID;
    if (!fqh::aligned(x, dtype == FQ_F32 ? 4 : 2) || !fqh::aligned(fq, 4)) return FQ_E_INVALID;
    if (dtype == FQ_F32) return launch_mx_elem<FQ_F32>(x, rows, cols, elem, q, e8m0, fq, stream);
    return launch_mx_elem<FQ_BF16>(x, rows, cols, elem, q, e8m0, fq, stream);
}

int fq_nvfp4(const float* x, int64_t n, void* workspace, size_t workspace_bytes, uint8_t* q, uint8_t* scales,
             float* tensor_scale, float* fq, hipStream_t stream) {
    if (!x || n < 1 || !workspace || !q || !scales || !tensor_scale) return FQ_E_INVALID;
    if (workspace_bytes < fq_workspace_bytes(n) || !fqh::aligned(workspace, 16)) return FQ_E_INVALID;
    if (!fqh::aligned(x, 4) || !fqh::aligned(fq, 4) || !fqh::aligned(tensor_scale, 4)) return FQ_E_INVALID;
    int rc = fqh::tensor_amax(x, n, workspace, stream);
    if (rc != FQ_OK) return rc;
    const uint32_t* tmax = reinterpret_cast<const uint32_t*>(workspace);
    const int64_t nfull = n / kNvBlock;  // whole blocks
    int64_t b0 = 0;
    if (nfull > 0 && fqh::aligned(x, 16) && fqh::aligned(fq, 16) && fqh::aligned(q, 8) && nfull / kB < 0x7FFFFFFFLL) {
        k_nvfp4_wide<<<(unsigned)((nfull + kB - 1) / kB), kB, 0, stream>>>(x, nfull, tmax, q, scales, tensor_scale, fq);
        b0 = nfull;
    }
    const int64_t nb = (n + kNvBlock - 1) / kNvBlock;
    if (b0 < nb)
        k_nvfp4_any<<<fqh::grid_for(nb - b0, kB, 8), kB, 0, stream>>>(x, n, b0, tmax, q, scales, tensor_scale, fq);
    return fqh::launched();
}

}  // extern "C"
