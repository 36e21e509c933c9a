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
// one 16-byte store of the fake-quant values; grid-stride, four chunks in flight.
#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;

template <int FMT>
struct Fp8QuantOp {
    ExactDiv div;
    float scale;
    bool zero;
    __device__ __forceinline__ explicit Fp8QuantOp(float s)
        : div(s == 0.0f ? 1.0f : s), scale(s), zero(s == 0.0f) {}
    __device__ __forceinline__ uint32_t code(float x) const {
        if (zero) return 0u;
        return fp8_encode<FMT>(div(x));
    }
    // fake-quant value of a code produced by code(): NaN byte -> NaN
    __device__ __forceinline__ float value(uint32_t b) const {
        float v = fp8_decode_finite<FMT>(b) * scale;
        return (b == 0x7Fu) ? __builtin_nanf("") : v;
    }
};

template <int FMT, bool AL>
__global__ __launch_bounds__(kB) void k_fp8_quant(const float* __restrict__ x, int64_t n,
                                                  const float* __restrict__ scale_p,
                                                  uint8_t* __restrict__ q, float* __restrict__ fq) {
    const Fp8QuantOp<FMT> op(*scale_p);
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x;
    auto chunk = [&](int64_t cc, float4 v) {
        uint32_t b0 = op.code(v.x), b1 = op.code(v.y), b2 = op.code(v.z), b3 = op.code(v.w);
        if (q) reinterpret_cast<uint32_t*>(q)[cc] = pack4(b0, b1, b2, b3);
        if (fq)
            reinterpret_cast<float4*>(fq)[cc] = make_float4(op.value(b0), op.value(b1), op.value(b2), op.value(b3));
    };
    if (AL) {
        for (; c + 3 * stride < nfull; c += 4 * stride) {
            const float4* xv = reinterpret_cast<const float4*>(x);
            float4 v0 = xv[c], v1 = xv[c + stride], v2 = xv[c + 2 * stride], v3 = xv[c + 3 * stride];
            chunk(c, v0);
            chunk(c + stride, v1);
            chunk(c + 2 * stride, v2);
            chunk(c + 3 * stride, v3);
        }
        for (; c < nfull; c += stride) chunk(c, reinterpret_cast<const float4*>(x)[c]);
    } else {
        for (; c < nfull; c += stride) {
            for (int e = 0; e < 4; ++e) {
                uint32_t b = op.code(x[4 * c + e]);
                if (q) q[4 * c + e] = (uint8_t)b;
                if (fq) fq[4 * c + e] = op.value(b);
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        int64_t i = 4 * nfull + threadIdx.x;
        uint32_t b = op.code(x[i]);
        if (q) q[i] = (uint8_t)b;
        if (fq) fq[i] = op.value(b);
    }
}

template <int FMT, bool AL>
__global__ __launch_bounds__(kB) void k_fp8_dequant(const uint8_t* __restrict__ q, int64_t n,
                                                    const float* __restrict__ scale_p,
                                                    float* __restrict__ out) {
    const float s = *scale_p;
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x;
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
            reinterpret_cast<float4*>(out)[c] = v;
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
    const unsigned G = fqh::grid_for((n + 3) / 4, 4 * kB, 8);
    if (al) k_fp8_quant<FMT, true><<<G, kB, 0, st>>>(x, n, scale, q, fq);
    else k_fp8_quant<FMT, false><<<G, kB, 0, st>>>(x, n, scale, q, fq);
}

template <int FMT>
void launch_dequant(const uint8_t* q, int64_t n, const float* scale, float* out, hipStream_t st) {
    const bool al = fqh::aligned(q, 4) && fqh::aligned(out, 16);
    const unsigned G = fqh::grid_for((n + 3) / 4, kB, 8);
    if (al) k_fp8_dequant<FMT, true><<<G, kB, 0, st>>>(q, n, scale, out);
    else k_fp8_dequant<FMT, false><<<G, kB, 0, st>>>(q, n, scale, out);
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
