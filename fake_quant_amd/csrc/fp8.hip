// fp8.hip -- saturating fp8 (E4M3 / E5M2) quantize, fake-quant and dequantize with
// a per-tensor scale.
//
// [QAT] optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
// Training (QAT) primitives": module docs "fp8 quantization" (format table,
// saturation, NaN propagation, unified ULP rounding), fake_quant_fp8.
// [MAR] ferrum-kernels 0.8.0 marlin_repack.rs, quantized_fp8_bits: a zero scale
// encodes every element as byte 0.
//
// Chunks of four elements: one 16-byte load of x, one 4-byte store of codes,
// one 16-byte store of the fake-quant values; one chunk per thread over a grid
// covering the tensor.  The quotient mode (zero scale / exact fast quotient /
// true division) is decided once per launch from the device-resident scale.
#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;
// Resident workgroups per compute unit (0: as many as the wave slots allow).
#ifndef FQ_OCC_FP8Q
#define FQ_OCC_FP8Q 0
#endif
#ifndef FQ_OCC_FP8DQ
#define FQ_OCC_FP8DQ 0
#endif

// Quotient modes, chosen once per launch from the (device-resident) scale:
// zero scale -> every byte 0; divisor in the exact-quotient window -> Markstein
// corrections; otherwise the compiler's correctly rounded division.
enum { kZero = 0, kQuick = 1, kTrue = 2 };

template <int FMT, int MODE>
__device__ __forceinline__ uint32_t fp8_code(float x, const ExactDiv& d) {
    if (MODE == kZero) return 0u;
    return fp8_encode<FMT>(MODE == kQuick ? d.quick(x) : x / d.s);
}
// fake-quant value of a code produced above (the NaN byte decodes to NaN)
template <int FMT>
__device__ __forceinline__ float fp8_value(uint32_t b, float scale) {
    float v = fp8_decode_finite<FMT>(b) * scale;
    return (b == 0x7Fu) ? __builtin_nanf("") : v;
}

template <int FMT, bool AL, int MODE>
__device__ __forceinline__ void fp8_quant_loop(const float* __restrict__ x, int64_t n, const ExactDiv& d,
                                               float scale, uint8_t* __restrict__ q, float* __restrict__ fq) {
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x;
    auto chunk = [&](int64_t cc, float4 v) {
        uint32_t w = 0;
        if (MODE != kZero) {
            const float y0 = MODE == kQuick ? d.quick(v.x) : v.x / d.s;
            const float y1 = MODE == kQuick ? d.quick(v.y) : v.y / d.s;
            const float y2 = MODE == kQuick ? d.quick(v.z) : v.z / d.s;
            const float y3 = MODE == kQuick ? d.quick(v.w) : v.w / d.s;
            w = fp8_encode4_hw<FMT>(y0, y1, y2, y3);
        }
        if (q) reinterpret_cast<uint32_t*>(q)[cc] = w;
        if (fq)
            store_nt(reinterpret_cast<float4*>(fq) + cc,
                make_float4(fp8_value<FMT>(w & 0xFFu, scale), fp8_value<FMT>((w >> 8) & 0xFFu, scale),
                            fp8_value<FMT>((w >> 16) & 0xFFu, scale), fp8_value<FMT>(w >> 24, scale)));
    };
    if (AL) {
        const float4* xv = reinterpret_cast<const float4*>(x);
        for (; c + 3 * stride < nfull; c += 4 * stride) {
            float4 v0 = xv[c], v1 = xv[c + stride], v2 = xv[c + 2 * stride], v3 = xv[c + 3 * stride];
            chunk(c, v0);
            chunk(c + stride, v1);
            chunk(c + 2 * stride, v2);
            chunk(c + 3 * stride, v3);
        }
        for (; c < nfull; c += stride) chunk(c, xv[c]);
    } else {
        for (; c < nfull; c += stride) {
            for (int e = 0; e < 4; ++e) {
                uint32_t b = fp8_code<FMT, MODE>(x[4 * c + e], d);
                if (q) q[4 * c + e] = (uint8_t)b;
                if (fq) fq[4 * c + e] = fp8_value<FMT>(b, scale);
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        int64_t i = 4 * nfull + threadIdx.x;
        uint32_t b = fp8_code<FMT, MODE>(x[i], d);
        if (q) q[i] = (uint8_t)b;
        if (fq) fq[i] = fp8_value<FMT>(b, scale);
    }
}

template <int FMT, bool AL>
__global__ __launch_bounds__(kB) void k_fp8_quant(const float* __restrict__ x, int64_t n,
                                                  const float* __restrict__ scale_p,
                                                  uint8_t* __restrict__ q, float* __restrict__ fq) {
    const float s = *scale_p;
    const ExactDiv d(s == 0.0f ? 1.0f : s);
    if (s == 0.0f)
        fp8_quant_loop<FMT, AL, kZero>(x, n, d, s, q, fq);
    else if (d.fast)
        fp8_quant_loop<FMT, AL, kQuick>(x, n, d, s, q, fq);
    else
        fp8_quant_loop<FMT, AL, kTrue>(x, n, d, s, q, fq);
}

template <int FMT, bool AL>
__global__ __launch_bounds__(kB) void k_fp8_dequant(const uint8_t* __restrict__ q, int64_t n,
                                                    const float* __restrict__ scale_p,
                                                    float* __restrict__ out) {
    const float s = *scale_p;
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x;
    if (AL) {
        const uint32_t* qw = reinterpret_cast<const uint32_t*>(q);
        float4* ov = reinterpret_cast<float4*>(out);
        auto dec4 = [&](uint32_t w) {
            return make_float4(fp8_decode<FMT>(w & 0xFFu) * s, fp8_decode<FMT>((w >> 8) & 0xFFu) * s,
                               fp8_decode<FMT>((w >> 16) & 0xFFu) * s, fp8_decode<FMT>(w >> 24) * s);
        };
        for (; c + 3 * stride < nfull; c += 4 * stride) {
            uint32_t w0 = qw[c], w1 = qw[c + stride], w2 = qw[c + 2 * stride], w3 = qw[c + 3 * stride];
            store_nt(ov + c, dec4(w0));
            store_nt(ov + c + stride, dec4(w1));
            store_nt(ov + c + 2 * stride, dec4(w2));
            store_nt(ov + c + 3 * stride, dec4(w3));
        }
    }
    for (; c < nfull; c += stride) {
        uint32_t w;
        if (AL) {
            w = reinterpret_cast<const uint32_t*>(q)[c];
        } else {
            w = (uint32_t)q[4 * c] | ((uint32_t)q[4 * c + 1] << 8) | ((uint32_t)q[4 * c + 2] << 16) |
                ((uint32_t)q[4 * c + 3] << 24);
        }
        float4 v = make_float4(fp8_decode<FMT>(w & 0xFFu) * s, fp8_decode<FMT>((w >> 8) & 0xFFu) * s,
                               fp8_decode<FMT>((w >> 16) & 0xFFu) * s, fp8_decode<FMT>(w >> 24) * s);
        if (AL) {
            store_nt(reinterpret_cast<float4*>(out) + c, v);
        } else {
            out[4 * c] = v.x;
            out[4 * c + 1] = v.y;
            out[4 * c + 2] = v.z;
            out[4 * c + 3] = v.w;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        int64_t i = 4 * nfull + threadIdx.x;
        out[i] = fp8_decode<FMT>(q[i]) * s;
    }
}

template <int FMT>
void launch_quant(const float* x, int64_t n, const float* scale, uint8_t* q, float* fq, hipStream_t st) {
    const bool al = fqh::aligned(x, 16) && fqh::aligned(q, 4) && fqh::aligned(fq, 16);
    const unsigned G = fqh::grid_all((n + 3) / 4, kB);
    const size_t lds = fqh::lds_cap(FQ_OCC_FP8Q, 0);
    if (al) k_fp8_quant<FMT, true><<<G, kB, lds, st>>>(x, n, scale, q, fq);
    else k_fp8_quant<FMT, false><<<G, kB, lds, st>>>(x, n, scale, q, fq);
}

template <int FMT>
void launch_dequant(const uint8_t* q, int64_t n, const float* scale, float* out, hipStream_t st) {
    const bool al = fqh::aligned(q, 4) && fqh::aligned(out, 16);
    const unsigned G = fqh::grid_all((n + 3) / 4, kB);
    const size_t lds = fqh::lds_cap(FQ_OCC_FP8DQ, 0);
    if (al) k_fp8_dequant<FMT, true><<<G, kB, lds, st>>>(q, n, scale, out);
    else k_fp8_dequant<FMT, false><<<G, kB, lds, st>>>(q, n, scale, out);
}

}  // namespace

extern "C" {

int fq_fp8_quantize(const float* x, int64_t n, int fmt, const float* scale, uint8_t* q, float* fq,
                    hipStream_t stream) {
    if (!fqh::valid_fmt(fmt)) return FQ_E_UNSUPPORTED;
    if (!x || n < 1 || !scale || (!q && !fq)) return FQ_E_INVALID;
    if (!fqh::aligned(x, 4) || !fqh::aligned(scale, 4) || !fqh::aligned(fq, 4)) return FQ_E_INVALID;
    if (fmt == FQ_E4M3) launch_quant<0>(x, n, scale, q, fq, stream);
    else launch_quant<1>(x, n, scale, q, fq, stream);
    return fqh::launched();
}

int fq_fp8_dequantize(const uint8_t* q, int64_t n, int fmt, const float* scale, float* out,
                      hipStream_t stream) {
    if (!fqh::valid_fmt(fmt)) return FQ_E_UNSUPPORTED;
    if (!q || n < 1 || !scale || !out) return FQ_E_INVALID;
    if (!fqh::aligned(scale, 4) || !fqh::aligned(out, 4)) return FQ_E_INVALID;
    if (fmt == FQ_E4M3) launch_dequant<0>(q, n, scale, out, stream);
    else launch_dequant<1>(q, n, scale, out, stream);
    return fqh::launched();
}

}  // extern "C"
