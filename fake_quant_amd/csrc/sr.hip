// sr.hip -- stochastic rounding for the per-tensor integer and fp8 paths.
//
// [QAT] optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
// Training (QAT) primitives": module docs "Rounding modes" and
// RoundingMode::Stochastic (round_to_int: floor(t) + 1 with probability equal to
// the fractional part, floor(t) otherwise; unbiased), used by quantize and by
// fp8_quantize_magnitude.
//
// The uniform variate of element index i is word i mod 4 of Philox4x32-10
// (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC'11) at counter (floor(i/4) low 32 bits, high 32 bits, 0, 0) under key
// (seed low, seed high), as a binary32 with 24 random bits: (word >> 8) 2^-24.
// Element x[k] of a call has index offset + k, so any split of a tensor draws
// the same numbers.  Rounding: up iff the draw is below fl(t - floor(t)).
//
// Layout: one chunk of four elements per thread (one 16-byte load of x) over a
// grid covering the tensor; a chunk needs one Philox block when the offset is a
// multiple of four, two otherwise (a launch-uniform choice).
#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;

// ---------------------------------------------------------------------------
// integer grid: code = clamp(round_sr(x / s), qmin - zp, qmax - zp) + zp
// ---------------------------------------------------------------------------
enum { kZero = 0, kQuick = 1, kTrue = 2 };

template <int MODE>
__device__ __forceinline__ float int_offset_sr(float x, const IntQ& q, uint32_t j) {
    if (MODE == kZero) return q.nan_off;
    const float t = MODE == kQuick ? q.div.quick(x) : x / q.div.s;
    const float r = fminf(fmaxf(round_sr(t, j), q.lo), q.hi) + 0.0f;  // code offset 0 is +0
    return (t != t) ? q.nan_off : r;
}

template <int BITS, int MODE>
__device__ __forceinline__ void int_sr_chunk(const float (&xe)[4], int cnt, const uint32_t (&j)[4], const IntQ& q,
                                             float scale, int zp, int64_t c, uint8_t* __restrict__ codes,
                                             float* __restrict__ fq, bool vec) {
    float o[4];
    int code[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o[e] = int_offset_sr<MODE>(xe[e], q, j[e]);
        code[e] = (int)o[e] + zp;
    }
    if (vec) {
        if (codes) {
            if (BITS == 8) reinterpret_cast<uint32_t*>(codes)[c] = pack4(code[0], code[1], code[2], code[3]);
            else reinterpret_cast<uint16_t*>(codes)[c] = (uint16_t)(nib2(code[0], code[1]) | (nib2(code[2], code[3]) << 8));
        }
        if (fq) store_nt(reinterpret_cast<float4*>(fq) + c, make_float4(o[0] * scale, o[1] * scale, o[2] * scale, o[3] * scale));
        return;
    }
    for (int e = 0; e < cnt; ++e) {
        if (fq) fq[4 * c + e] = o[e] * scale;
        if (codes && BITS == 8) codes[4 * c + e] = (uint8_t)code[e];
    }
    if (codes && BITS == 4) {
        codes[2 * c] = (uint8_t)nib2(code[0], cnt > 1 ? code[1] : 0);
        if (cnt > 2) codes[2 * c + 1] = (uint8_t)nib2(code[2], cnt > 3 ? code[3] : 0);
    }
}

template <int BITS, int MODE, bool AL>
__device__ __forceinline__ void int_sr_loop(const float* __restrict__ x, int64_t n, const IntQ& q, float scale,
                                            int zp, const Draws& d, uint8_t* __restrict__ codes,
                                            float* __restrict__ fq) {
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    for (int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x; c <= nfull; c += stride) {
        const int cnt = c < nfull ? 4 : (int)(n & 3);
        if (cnt == 0) break;
        float xe[4] = {0.f, 0.f, 0.f, 0.f};
        if (AL && cnt == 4) {
            const float4 v = reinterpret_cast<const float4*>(x)[c];
            xe[0] = v.x;
            xe[1] = v.y;
            xe[2] = v.z;
            xe[3] = v.w;
        } else {
            for (int e = 0; e < cnt; ++e) xe[e] = x[4 * c + e];
        }
        uint32_t j[4];
        d.get(c, j);
        int_sr_chunk<BITS, MODE>(xe, cnt, j, q, scale, zp, c, codes, fq, AL && cnt == 4);
    }
}

template <int BITS, bool AL>
__global__ __launch_bounds__(kB) void k_fq_int_tensor_sr(const float* __restrict__ x, int64_t n, int affine,
                                                         const fq_int_params* __restrict__ p, Draws d,
                                                         uint8_t* __restrict__ codes, float* __restrict__ fq) {
    const fq_int_params P = *p;
    const IntRange rg = int_range(BITS, affine != 0);
    const IntQ q(P.scale, P.zero_point, rg);
    if (q.zero) int_sr_loop<BITS, kZero, AL>(x, n, q, P.scale, P.zero_point, d, codes, fq);
    else if (q.div.fast) int_sr_loop<BITS, kQuick, AL>(x, n, q, P.scale, P.zero_point, d, codes, fq);
    else int_sr_loop<BITS, kTrue, AL>(x, n, q, P.scale, P.zero_point, d, codes, fq);
}

template <int FMT>
__device__ __forceinline__ float fp8_value_sr(uint32_t b, float scale) {
    const float v = fp8_decode_finite<FMT>(b) * scale;
    return b == 0x7Fu ? __builtin_nanf("") : v;
}

template <int FMT, int MODE, bool AL>
__device__ __forceinline__ void fp8_sr_loop(const float* __restrict__ x, int64_t n, const ExactDiv& dv, float scale,
                                            const Draws& d, uint8_t* __restrict__ q, float* __restrict__ fq) {
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    for (int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x; c <= nfull; c += stride) {
        const int cnt = c < nfull ? 4 : (int)(n & 3);
        if (cnt == 0) break;
        float xe[4] = {0.f, 0.f, 0.f, 0.f};
        if (AL && cnt == 4) {
            const float4 v = reinterpret_cast<const float4*>(x)[c];
            xe[0] = v.x;
            xe[1] = v.y;
            xe[2] = v.z;
            xe[3] = v.w;
        } else {
            for (int e = 0; e < cnt; ++e) xe[e] = x[4 * c + e];
        }
        uint32_t j[4];
        d.get(c, j);
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (MODE == kZero) {
                b[e] = 0u;
            } else {
                const float y = MODE == kQuick ? dv.quick(xe[e]) : xe[e] / dv.s;
                b[e] = fp8_encode_sr<FMT>(y, j[e]);
            }
        }
        if (AL && cnt == 4) {
            const uint32_t w = pack4(b[0], b[1], b[2], b[3]);
            if (q) reinterpret_cast<uint32_t*>(q)[c] = w;
            if (fq) {
                // the codes above are never Inf codes; their NaN code decodes to NaN
                float d[4];
                fp8_decode4_hw<FMT>(w, d);
                store_nt(reinterpret_cast<float4*>(fq) + c,
                         make_float4(d[0] * scale, d[1] * scale, d[2] * scale, d[3] * scale));
            }
        } else {
            for (int e = 0; e < cnt; ++e) {
                if (q) q[4 * c + e] = (uint8_t)b[e];
                if (fq) fq[4 * c + e] = fp8_value_sr<FMT>(b[e], scale);
            }
        }
    }
}

template <int FMT, bool AL>
__global__ __launch_bounds__(kB) void k_fp8_quant_sr(const float* __restrict__ x, int64_t n,
                                                     const float* __restrict__ scale_p, Draws d,
                                                     uint8_t* __restrict__ q, float* __restrict__ fq) {
    const float s = *scale_p;
    const ExactDiv dv(s == 0.0f ? 1.0f : s);
    if (s == 0.0f) fp8_sr_loop<FMT, kZero, AL>(x, n, dv, s, d, q, fq);
    else if (dv.fast) fp8_sr_loop<FMT, kQuick, AL>(x, n, dv, s, d, q, fq);
    else fp8_sr_loop<FMT, kTrue, AL>(x, n, dv, s, d, q, fq);
}

}  // namespace

extern "C" {

int fq_fake_quant_int_tensor_sr(const float* x, int64_t n, int bits, int scheme, const fq_int_params* params,
                                uint64_t seed, uint64_t offset, void* codes, float* fq, hipStream_t stream) {
    if (!fqh::valid_bits(bits) || !fqh::valid_scheme(scheme)) return FQ_E_UNSUPPORTED;
    if (!x || n < 1 || !params || (!codes && !fq)) return FQ_E_INVALID;
    if (!fqh::aligned(x, 4) || !fqh::aligned(params, 4) || !fqh::aligned(fq, 4)) return FQ_E_INVALID;
    const bool al = fqh::aligned(x, 16) && fqh::aligned(fq, 16) && fqh::aligned(codes, bits == 8 ? 4 : 2);
    const unsigned G = fqh::grid_all(n / 4 + 1, kB);
    const Draws d = Draws::make(seed, offset);
    uint8_t* cd = (uint8_t*)codes;
    const int aff = scheme == FQ_AFFINE;
    if (bits == 8) {
        if (al) k_fq_int_tensor_sr<8, true><<<G, kB, 0, stream>>>(x, n, aff, params, d, cd, fq);
        else k_fq_int_tensor_sr<8, false><<<G, kB, 0, stream>>>(x, n, aff, params, d, cd, fq);
    } else {
        if (al) k_fq_int_tensor_sr<4, true><<<G, kB, 0, stream>>>(x, n, aff, params, d, cd, fq);
        else k_fq_int_tensor_sr<4, false><<<G, kB, 0, stream>>>(x, n, aff, params, d, cd, fq);
    }
    return fqh::launched();
}

int fq_fp8_quantize_sr(const float* x, int64_t n, int fmt, const float* scale, uint64_t seed, uint64_t offset,
                       uint8_t* q, float* fq, hipStream_t stream) {
    if (!fqh::valid_fmt(fmt)) return FQ_E_UNSUPPORTED;
    if (!x || n < 1 || !scale || (!q && !fq)) return FQ_E_INVALID;
    if (!fqh::aligned(x, 4) || !fqh::aligned(scale, 4) || !fqh::aligned(fq, 4)) return FQ_E_INVALID;
    const bool al = fqh::aligned(x, 16) && fqh::aligned(q, 4) && fqh::aligned(fq, 16);
    const unsigned G = fqh::grid_all(n / 4 + 1, kB);
    const Draws d = Draws::make(seed, offset);
    if (fmt == FQ_E4M3) {
        if (al) k_fp8_quant_sr<0, true><<<G, kB, 0, stream>>>(x, n, scale, d, q, fq);
        else k_fp8_quant_sr<0, false><<<G, kB, 0, stream>>>(x, n, scale, d, q, fq);
    } else {
        if (al) k_fp8_quant_sr<1, true><<<G, kB, 0, stream>>>(x, n, scale, d, q, fq);
        else k_fp8_quant_sr<1, false><<<G, kB, 0, stream>>>(x, n, scale, d, q, fq);
    }
    return fqh::launched();
}

}  // extern "C"
