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
// Cache policy of the float outputs (fake-quant values, dequantized values):
// nontemporal device-scope buffer stores (nt sc1).  Measured over the bench step
// on one box, two runs each, against global nontemporal stores: quantize E4M3
// 98.6-98.7 -> 96.3-96.8 us, E5M2 98.0-98.1 -> 95.1-95.4 us, dequantize -0.5 to
// -1 us.  The same stores in the per-row kernels cost them 1-2 points cold, and
// the per-tensor and wide-layout kernels did not move, so those keep global
// nontemporal stores.  Plain stores: the dequantize 52.6-53.0 against 54.9-55.0
// us cold, but 57 against 48 us warm and the fp8 step 0.379-0.382 against
// 0.341-0.346 ms (the plain stores leave dirty lines to the ops after them).
#ifndef FQ_FP8_OUT_CP
#define FQ_FP8_OUT_CP 18
#endif
constexpr int kOutCp = FQ_FP8_OUT_CP;

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
        if (fq) {
            // the codes above are never Inf codes; their NaN code decodes to NaN
            float d[4];
            fp8_decode4_hw<FMT>(w, d);
            store_out<kOutCp>(reinterpret_cast<float4*>(fq), cc,
                     make_float4(d[0] * scale, d[1] * scale, d[2] * scale, d[3] * scale));
        }
    };
    if (AL) {
        const float4* xv = reinterpret_cast<const float4*>(x);
        for (; c + 3 * stride < nfull; c += 4 * stride) {
            float4 v0 = ld_f4<FQ_NT_LOADS_FP8 != 0>(xv + c), v1 = ld_f4<FQ_NT_LOADS_FP8 != 0>(xv + c + stride), v2 = ld_f4<FQ_NT_LOADS_FP8 != 0>(xv + c + 2 * stride),
                   v3 = ld_f4<FQ_NT_LOADS_FP8 != 0>(xv + c + 3 * stride);
            chunk(c, v0);
            chunk(c + stride, v1);
            chunk(c + 2 * stride, v2);
            chunk(c + 3 * stride, v3);
        }
        for (; c < nfull; c += stride) chunk(c, ld_f4<FQ_NT_LOADS_FP8 != 0>(xv + c));
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

// Dequantize, any alignment: one chunk of four codes per thread-iteration, byte
// loads and element stores.
template <int FMT>
__global__ __launch_bounds__(kB) void k_fp8_dequant_any(const uint8_t* __restrict__ q, int64_t n,
                                                        const float* __restrict__ scale_p,
                                                        float* __restrict__ out) {
    const float s = *scale_p;
    const int64_t stride = (int64_t)gridDim.x * kB;
    for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n; i += stride)
        out[i] = fp8_decode<FMT>(q[i]) * s;
}

// Aligned dequantize, U chunks of four codes per lane: wave w of the grid owns
// chunks [64 U w, 64 U (w + 1)); its lane l takes chunks 64 U w + 64 u + l, so
// every load and store instruction of the wave is one contiguous run and a wave
// has U loads in flight before its first store (U = 2 measured fastest with the
// codes cold in HBM: one 4-byte load per lane leaves too few reads in flight).
template <int FMT, int U>
__global__ __launch_bounds__(kB) void k_fp8_dequant_w(const uint32_t* __restrict__ qw, int64_t n,
                                                      const float* __restrict__ scale_p,
                                                      float4* __restrict__ out) {
    const float s = *scale_p;
    const int64_t nfull = n >> 2;
    const int64_t base = ((int64_t)blockIdx.x * (kB / kWave) + threadIdx.x / kWave) * (kWave * U) + threadIdx.x % kWave;
    uint32_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = base + u * kWave < nfull ? qw[base + u * kWave] : 0u;
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (base + u * kWave < nfull) {
            float d[4];
            fp8_decode4_hw<FMT>(w[u], d);
            store_out<kOutCp>(out, base + u * kWave, make_float4(d[0] * s, d[1] * s, d[2] * s, d[3] * s));
        }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        const int64_t i = 4 * nfull + threadIdx.x;
        reinterpret_cast<float*>(out)[i] = fp8_decode<FMT>(reinterpret_cast<const uint8_t*>(qw)[i]) * s;
    }
}

constexpr int kDqU = 2;

template <int FMT>
void launch_quant(const float* x, int64_t n, const float* scale, uint8_t* q, float* fq, hipStream_t st) {
    const bool al = fqh::aligned(x, 16) && fqh::aligned(q, 4) && fqh::aligned(fq, 16);
    const unsigned G = fqh::grid_all((n + 3) / 4, kB);
    if (al) k_fp8_quant<FMT, true><<<G, kB, 0, st>>>(x, n, scale, q, fq);
    else k_fp8_quant<FMT, false><<<G, kB, 0, st>>>(x, n, scale, q, fq);
}

template <int FMT>
void launch_dequant(const uint8_t* q, int64_t n, const float* scale, float* out, hipStream_t st) {
    const int64_t blocks = (n / 4 + 1 + (int64_t)kB * kDqU - 1) / ((int64_t)kB * kDqU);
    if (fqh::aligned(q, 4) && fqh::aligned(out, 16) && blocks <= 0x7FFFFFFF) {
        const unsigned G = fqh::grid_all(n / 4 + 1, (int64_t)kB * kDqU);
        k_fp8_dequant_w<FMT, kDqU><<<G, kB, 0, st>>>(reinterpret_cast<const uint32_t*>(q), n, scale,
                                                     reinterpret_cast<float4*>(out));
    } else {
        k_fp8_dequant_any<FMT><<<fqh::grid_for(n, kB, 8), kB, 0, st>>>(q, n, scale, out);
    }
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
