// rows.hip -- fused per-row (per-channel along axis 0 / per-token) calibration and
// integer quantization, and the matching per-row dequantize.
//
// [QAT] optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
// Training (QAT) primitives": per_channel_params (axis 0), QuantParams::from_minmax,
// fake_quant_int_per_channel.  The page calibrates every channel in one pass and
// quantizes in a second; here one workgroup owns a row, keeps it in registers
// between the reduction and the quantize step, and reads it from HBM once.
//
// Three launch shapes, chosen by the row length in 16-byte vectors (4 fp32 or
// 8 bf16) and the buffers' alignment:
//   k_rows_wg    aligned rows of 257 .. 4 TW vectors: a workgroup of TW threads
//                per row (512 for fp32, 256 for bf16), up to four vectors per
//                thread;
//   k_rows_wave  other aligned rows: one wave per row, up to 16 vectors per lane
//                per slab, longer rows slab by slab;
//   k_quant_rows ragged or unaligned rows: 256-thread workgroup per row with
//                element loads.
// Every shape keeps a slab of the row in registers between the reduction and the
// quantize step.
#include <type_traits>

#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;
constexpr int kWaves = kB / kWave;
constexpr int kCache = 4;              // vectors per thread per slab
constexpr int kSlab = kCache * kB;     // vectors per slab

template <int DT>
struct Vec;
template <>
struct Vec<FQ_F32> {
    static constexpr int N = 4;
    float4 v;
    __device__ __forceinline__ float get(int e) const { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
};
template <>
struct Vec<FQ_BF16> {
    static constexpr int N = 8;
    uint4 v;
    __device__ __forceinline__ float get(int e) const {
        uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
        return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    }
};

// Load vector vi of a row: 16-byte load when aligned, else element loads with a
// bound check against cols (missing elements read as 0 and are marked invalid by
// the caller through the same bound).
template <int DT, bool AL>
__device__ __forceinline__ Vec<DT> load_vec(const void* row, int64_t vi, int64_t cols) {
    Vec<DT> r;
    constexpr int N = Vec<DT>::N;
    if constexpr (AL) {
        if constexpr (DT == FQ_F32) r.v = ld_f4<FQ_NT_LOADS_ROWS != 0>(reinterpret_cast<const float4*>(row) + vi);
        else r.v = ld_u4<FQ_NT_LOADS_ROWS != 0>(reinterpret_cast<const uint4*>(row) + vi);
    } else {
        uint32_t w[4] = {0, 0, 0, 0};
        for (int e = 0; e < N; ++e) {
            int64_t c = vi * N + e;
            if (c >= cols) break;
            if constexpr (DT == FQ_F32) {
                w[e] = as_u(reinterpret_cast<const float*>(row)[c]);
            } else {
                uint32_t h = reinterpret_cast<const uint16_t*>(row)[c];
                w[e >> 1] |= (e & 1) ? (h << 16) : h;
            }
        }
        *reinterpret_cast<uint4*>(&r.v) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return r;
}

template <int DT, int BITS, bool AL>
__global__ __launch_bounds__(kB) void k_quant_rows(const void* __restrict__ x, int64_t cols, int affine,
                                                   uint8_t* __restrict__ codes, float* __restrict__ fq,
                                                   float* __restrict__ scale_out,
                                                   int32_t* __restrict__ zp_out,
                                                   uint32_t* __restrict__ flags) {
    constexpr int N = Vec<DT>::N;
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const size_t esz = DT == FQ_F32 ? 4 : 2;
    const char* xr = reinterpret_cast<const char*>(x) + (size_t)row * (size_t)cols * esz;
    const int64_t nv = (cols + N - 1) / N;
    const int nslab = (int)((nv + kSlab - 1) / kSlab);

    // ---- reduction: finite min / max, non-finite marker ----
    MinMax m;
    Vec<DT> cache[kCache];
    for (int s = 0; s < nslab; ++s) {
#pragma unroll
        for (int k = 0; k < kCache; ++k) {
            int64_t vi = (int64_t)s * kSlab + k * kB + t;
            if (vi < nv) cache[k] = load_vec<DT, AL>(xr, vi, cols);
        }
#pragma unroll
        for (int k = 0; k < kCache; ++k) {
            int64_t vi = (int64_t)s * kSlab + k * kB + t;
            if (vi >= nv) continue;
#pragma unroll
            for (int e = 0; e < N; ++e)
                if (AL || vi * N + e < cols) m.add(cache[k].get(e));
        }
    }
    __shared__ float4 lds[kWaves];
    {
        float4 r = make_float4(wave_min_f(m.mn), wave_max_f(m.mx), as_f(wave_max_u(m.nf)), 0.f);
        if (t % kWave == 0) lds[t / kWave] = r;
        __syncthreads();
        MinMax all;
        for (int i = 0; i < kWaves; ++i) all.merge(lds[i].x, lds[i].y, as_u(lds[i].z));
        m = all;
    }
    const bool aff = affine != 0;
    const IntRange rg = int_range(BITS, aff);
    const IntCal cal = calibrate(m.mn, m.mx, rg, aff);
    if (t == 0) {
        scale_out[row] = cal.scale;
        zp_out[row] = cal.zp;
        uint32_t f = (m.nonfinite() ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
        if (flags && f) atomicOr(flags, f);
    }
    const IntQ q(cal.scale, cal.zp, rg);
    // all elements finite and the divisor admitted to the exact fast quotient:
    // no NaN / Inf / overflow can reach the rounding step
    const bool finite_fast = !m.nonfinite() && !q.zero && q.div.fast;
    const float sc = cal.scale;
    const int zp = cal.zp;

    // ---- quantize (last slab is still in registers) ----
    uint8_t* crow8 = codes ? codes + (size_t)row * (size_t)cols : nullptr;
    const int64_t pstride = (cols + 1) / 2;
    uint8_t* crow4 = codes ? codes + (size_t)row * (size_t)pstride : nullptr;
    float* frow = fq ? fq + (size_t)row * (size_t)cols : nullptr;
    for (int s = nslab - 1; s >= 0; --s) {
        if (s != nslab - 1) {
#pragma unroll
            for (int k = 0; k < kCache; ++k) {
                int64_t vi = (int64_t)s * kSlab + k * kB + t;
                if (vi < nv) cache[k] = load_vec<DT, AL>(xr, vi, cols);
            }
        }
#pragma unroll
        for (int k = 0; k < kCache; ++k) {
            int64_t vi = (int64_t)s * kSlab + k * kB + t;
            if (vi >= nv) continue;
            float o[N];
#pragma unroll
            for (int e = 0; e < N; ++e) {
                float xv = cache[k].get(e);
                o[e] = finite_fast ? q.offset_finite(xv) : q.offset(xv);
            }
            if (AL) {
                if (codes) {
                    if (BITS == 8) {
                        uint32_t w0 = pack4((int)o[0] + zp, (int)o[1] + zp, (int)o[2] + zp, (int)o[3] + zp);
                        if (N == 4) {
                            reinterpret_cast<uint32_t*>(crow8)[vi] = w0;
                        } else {
                            uint32_t w1 = pack4((int)o[4] + zp, (int)o[5] + zp, (int)o[6] + zp, (int)o[7] + zp);
                            reinterpret_cast<uint2*>(crow8)[vi] = make_uint2(w0, w1);
                        }
                    } else {
                        uint32_t b01 = nib2((int)o[0] + zp, (int)o[1] + zp);
                        uint32_t b23 = nib2((int)o[2] + zp, (int)o[3] + zp);
                        if (N == 4) {
                            reinterpret_cast<uint16_t*>(crow4)[vi] = (uint16_t)(b01 | (b23 << 8));
                        } else {
                            uint32_t b45 = nib2((int)o[4] + zp, (int)o[5] + zp);
                            uint32_t b67 = nib2((int)o[6] + zp, (int)o[7] + zp);
                            reinterpret_cast<uint32_t*>(crow4)[vi] = b01 | (b23 << 8) | (b45 << 16) | (b67 << 24);
                        }
                    }
                }
                if (fq) {
                    float4* fr = reinterpret_cast<float4*>(frow);
                    fr[vi * (N / 4)] = make_float4(o[0] * sc, o[1] * sc, o[2] * sc, o[3] * sc);
                    if (N == 8)
                        fr[vi * 2 + 1] = make_float4(o[4] * sc, o[5] * sc, o[6] * sc, o[7] * sc);
                }
            } else {
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    int64_t c = vi * N + e;
                    if (c >= cols) break;
                    int code = (int)o[e] + zp;
                    if (frow) frow[c] = o[e] * sc;
                    if (!codes) continue;
                    if (BITS == 8) {
                        crow8[c] = (uint8_t)code;
                    } else if ((e & 1) == 0) {
                        int next = (c + 1 < cols) ? (int)o[e + 1] + zp : 0;
                        crow4[c >> 1] = (uint8_t)nib2(code, next);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Aligned rows: one wave per row.  Lane l holds 16-byte vectors l + 64 k,
// k < KV, of a slab of 64 * KV vectors (a 4096-float / 8192-bf16 row is one slab
// at KV = 16: 64 registers of data per lane).  No barrier: the row reduction is
// DPP + lane shuffles, the parameters are wave-uniform.
// Fast path (row all finite, divisor in the exact-quotient window):
//   t = fl(x / s) (two Markstein corrections), tc = clamp(t, qmin - zp, qmax - zp),
//   f = tc + kMagic rounds tc half-even; code = low bits of (pattern(f) + zp);
//   fake-quant = (f - kMagic) * s.
// Rows holding Inf / NaN are calibrated on their finite elements and quantized
// with the general per-element rule (NaN -> 0, +-Inf clamp).
// ---------------------------------------------------------------------------
template <int DT, bool NEED>
__device__ __forceinline__ void minmax_vec(const Vec<DT>& v, float& mn, float& mx, bool& bad) {
    constexpr int N = Vec<DT>::N;
#pragma unroll
    for (int e = 0; e < N; e += 4) {
        float a = v.get(e), b = v.get(e + 1), c = v.get(e + 2), d = v.get(e + 3);
        mn = fminf(fminf(mn, a), fminf(b, fminf(c, d)));
        mx = fmaxf(fmaxf(mx, a), fmaxf(b, fmaxf(c, d)));
        if (NEED) bad = bad | (a != a) | (b != b) | (c != c) | (d != d);
    }
}

// min / max of a vector with NaN propagation (IEEE 754-2019 minimum / maximum,
// v_minimum3_f32 / v_maximum3_f32): a NaN anywhere makes both results NaN, an
// infinity shows as itself, so a finite result proves the vector finite.
template <int DT>
__device__ __forceinline__ void minmax_nan(const Vec<DT>& v, float& mn, float& mx) {
    constexpr int N = Vec<DT>::N;
#pragma unroll
    for (int e = 0; e < N; e += 2) {
        const float a = v.get(e), b = v.get(e + 1);
        mn = __builtin_elementwise_minimum(mn, __builtin_elementwise_minimum(a, b));
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(a, b));
    }
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// a code store: plain, or with the nontemporal hint
template <bool NT, class V>
__device__ __forceinline__ void st_code(V* p, V v) {
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Codes of one vector (N = 4 fp32 or 8 bf16 elements).  fp32 rows (N = 4)
// store them with the nontemporal hint: measured in the bench step, the fp8
// amax pass that follows the [4096, 4096] fp32 row ops then finds fewer dirty
// lines to write back (70.1 -> 64.9 us), while the row ops themselves lose
// about 1 us in the step.  bf16 rows keep plain stores: with the hint the
// per-token op itself slowed by more than the op after it gained.
template <int BITS, int N>
__device__ __forceinline__ void store_codes(uint8_t* crow, int64_t vi, const uint32_t (&cb)[N]) {
    constexpr bool NT = N == 4;
    if (BITS == 8) {
        uint32_t w0 = pack4(cb[0], cb[1], cb[2], cb[3]);
        if (N == 4) {
            st_code<NT>(reinterpret_cast<uint32_t*>(crow) + vi, w0);
        } else {
            uint32_t w1 = pack4(cb[4 % N], cb[5 % N], cb[6 % N], cb[7 % N]);
            st_code<NT>(reinterpret_cast<u32x2*>(crow) + vi, u32x2{w0, w1});
        }
    } else {
        uint32_t b01 = ((cb[0] & 0xFu) << 4) | (cb[1] & 0xFu);
        uint32_t b23 = ((cb[2] & 0xFu) << 4) | (cb[3] & 0xFu);
        if (N == 4) {
            st_code<NT>(reinterpret_cast<uint16_t*>(crow) + vi, (uint16_t)(b01 | (b23 << 8)));
        } else {
            uint32_t b45 = ((cb[4 % N] & 0xFu) << 4) | (cb[5 % N] & 0xFu);
            uint32_t b67 = ((cb[6 % N] & 0xFu) << 4) | (cb[7 % N] & 0xFu);
            st_code<NT>(reinterpret_cast<uint32_t*>(crow) + vi, b01 | (b23 << 8) | (b45 << 16) | (b67 << 24));
        }
    }
}

template <int DT, int BITS, int KV>
__global__ __launch_bounds__(kB) void k_rows_wave(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                  int affine, uint8_t* __restrict__ codes,
                                                  float* __restrict__ fq, float* __restrict__ scale_out,
                                                  int32_t* __restrict__ zp_out, uint32_t* __restrict__ flags) {
    constexpr int N = Vec<DT>::N;
    constexpr int kSlabW = kWave * KV;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole wave
    const size_t esz = DT == FQ_F32 ? 4 : 2;
    const char* xr = reinterpret_cast<const char*>(x) + (size_t)row * (size_t)cols * esz;
    const int64_t nv = cols / N;
    const int nslab = (int)((nv + kSlabW - 1) / kSlabW);

    Vec<DT> cache[KV];
    auto load_slab = [&](int s) {
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            const int64_t vi = (int64_t)s * kSlabW + k * kWave + lane;
            if (vi < nv) cache[k] = load_vec<DT, true>(xr, vi, cols);
        }
    };

    // ---- reduction (NaN is ignored by min / max; +-Inf and NaN are detected) ----
    float mn = __builtin_inff(), mx = -__builtin_inff();
    bool bad = false;
    for (int s = 0; s < nslab; ++s) {
        load_slab(s);
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            const int64_t vi = (int64_t)s * kSlabW + k * kWave + lane;
            if (vi < nv) minmax_vec<DT, true>(cache[k], mn, mx, bad);
        }
    }
    mn = wave_min_f(mn);
    mx = wave_max_f(mx);
    const bool nonfinite = __any(bad) || mn == -__builtin_inff() || mx == __builtin_inff();
    if (nonfinite) {
        MinMax m;
        for (int s = nslab - 1; s >= 0; --s) {
            if (s != nslab - 1) load_slab(s);
#pragma unroll
            for (int k = 0; k < KV; ++k) {
                const int64_t vi = (int64_t)s * kSlabW + k * kWave + lane;
                if (vi >= nv) continue;
#pragma unroll
                for (int e = 0; e < N; ++e) m.add(cache[k].get(e));
            }
        }
        mn = wave_min_f(m.mn);
        mx = wave_max_f(m.mx);
        if (nslab > 1) load_slab(nslab - 1);
    }
    const bool aff = affine != 0;
    const IntRange rg = int_range(BITS, aff);
    const IntCal cal = calibrate(mn, mx, rg, aff);
    if (lane == 0) {
        scale_out[row] = cal.scale;
        zp_out[row] = cal.zp;
        uint32_t f = (nonfinite ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
        if (flags && f) atomicOr(flags, f);
    }
    const float sc = cal.scale;
    const int zp = cal.zp;
    const bool fast = !nonfinite && !cal.degenerate && fast_divisor(sc);
    const IntQ q(sc, zp, rg);
    const float y = q.div.y;
    const float lo = q.lo, hi = q.hi;

    uint8_t* crow = codes ? codes + (size_t)row * (size_t)(BITS == 8 ? cols : cols / 2) : nullptr;
    float* frow = fq ? fq + (size_t)row * (size_t)cols : nullptr;
    for (int s = nslab - 1; s >= 0; --s) {
        if (s != nslab - 1) load_slab(s);
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            const int64_t vi = (int64_t)s * kSlabW + k * kWave + lane;
            if (vi >= nv) continue;
            uint32_t cb[N];
            float fv[N];
            if (fast) {
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    const float tc = fminf(fmaxf(quick_div(cache[k].get(e), sc, y), lo), hi);
                    const float f = tc + kMagic;
                    cb[e] = as_u(f) + (uint32_t)zp;
                    fv[e] = (f - kMagic) * sc;
                }
            } else {
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    const float o = q.offset(cache[k].get(e));
                    cb[e] = (uint32_t)((int)o + zp);
                    fv[e] = o * sc;
                }
            }
            if (crow) store_codes<BITS, N>(crow, vi, cb);
            if (frow) {
                float4* fr = reinterpret_cast<float4*>(frow);
                store_nt(fr + vi * (N / 4), make_float4(fv[0], fv[1], fv[2], fv[3]));
                if (N == 8) store_nt(fr + vi * 2 + 1, make_float4(fv[4 % N], fv[5 % N], fv[6 % N], fv[7 % N]));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Aligned rows that fit one workgroup: T threads, V vectors of 16 bytes per
// thread (vi = k * T + t).  The row min / max is NaN-propagating per thread
// (v_minimum3 / v_maximum3) and reduced as order-preserving integer keys (DPP
// within the wave, LDS across waves), so one test on the result tells a finite
// row from one that needs the finite-only recomputation.  Same fast and general
// quantize paths as k_rows_wave; the fast clamp is one v_med3_f32.
// ---------------------------------------------------------------------------
template <int DT, int BITS, int T, int V>
__global__ __launch_bounds__(T) void k_rows_wg(const void* __restrict__ x, int64_t cols, int affine,
                                               uint8_t* __restrict__ codes, float* __restrict__ fq,
                                               float* __restrict__ scale_out, int32_t* __restrict__ zp_out,
                                               uint32_t* __restrict__ flags) {
    constexpr int N = Vec<DT>::N;
    constexpr int NW = T / kWave;
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const size_t esz = DT == FQ_F32 ? 4 : 2;
    const char* xr = reinterpret_cast<const char*>(x) + (size_t)row * (size_t)cols * esz;
    const int64_t nv = cols / N;

    Vec<DT> cache[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int64_t vi = (int64_t)k * T + t;
        if (vi < nv) cache[k] = load_vec<DT, true>(xr, vi, cols);
    }
    // Row min / max: NaN-propagating per thread, then as order-preserving integer
    // keys across the wave (DPP) and the workgroup (LDS).  A thread that met a
    // NaN reports the extreme keys, which decode to NaN.
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < V; ++k)
        if ((int64_t)k * T + t < nv) minmax_nan<DT>(cache[k], mn, mx);
    const bool tnan = mn != mn;
    int32_t kmn = wave_min_i(tnan ? INT32_MIN : fkey(mn));
    int32_t kmx = wave_max_i(tnan ? INT32_MAX : fkey(mx));

    __shared__ int32_t s_key[2 * NW];
    __shared__ float s_mn[NW], s_mx[NW];
    const int w = t / kWave;
    if ((t & (kWave - 1)) == 0) {
        s_key[w] = kmn;
        s_key[NW + w] = kmx;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        kmn = min(kmn, s_key[i]);
        kmx = max(kmx, s_key[NW + i]);
    }
    mn = fkey_value(kmn);
    mx = fkey_value(kmx);
    const bool nonfinite = !(__builtin_fabsf(mn) < __builtin_inff()) || !(__builtin_fabsf(mx) < __builtin_inff());
    if (nonfinite) {
        // calibrate on the finite elements only
        MinMax m;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            if ((int64_t)k * T + t >= nv) continue;
#pragma unroll
            for (int e = 0; e < N; ++e) m.add(cache[k].get(e));
        }
        const float wmn = wave_min_f(m.mn), wmx = wave_max_f(m.mx);
        if ((t & (kWave - 1)) == 0) {
            s_mn[w] = wmn;
            s_mx[w] = wmx;
        }
        __syncthreads();
        mn = s_mn[0];
        mx = s_mx[0];
#pragma unroll
        for (int i = 1; i < NW; ++i) {
            mn = fminf(mn, s_mn[i]);
            mx = fmaxf(mx, s_mx[i]);
        }
    }
    const bool aff = affine != 0;
    const IntRange rg = int_range(BITS, aff);
    const IntCal cal = calibrate(mn, mx, rg, aff);
    if (t == 0) {
        scale_out[row] = cal.scale;
        zp_out[row] = cal.zp;
        uint32_t f = (nonfinite ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
        if (flags && f) atomicOr(flags, f);
    }
    const float sc = cal.scale;
    const int zp = cal.zp;
    const bool fast = !nonfinite && !cal.degenerate && fast_divisor(sc);
    const IntQ q(sc, zp, rg);
    const float y = q.div.y;
    const float lo = q.lo, hi = q.hi;
    uint8_t* crow = codes ? codes + (size_t)row * (size_t)(BITS == 8 ? cols : cols / 2) : nullptr;
    float* frow = fq ? fq + (size_t)row * (size_t)cols : nullptr;
    // the fast loop is instantiated with and without the fake-quant output, so a
    // codes-only call spends nothing on fake-quant values
    auto quantize = [&](auto want_fq) {
        constexpr bool WF = decltype(want_fq)::value;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int64_t vi = (int64_t)k * T + t;
            if (vi >= nv) continue;
            uint32_t cb[N];
            float fv[N];
            if (fast) {
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    // the row is finite here, so the clamp is one v_med3_f32
                    const float tc = __builtin_amdgcn_fmed3f(quick_div(cache[k].get(e), sc, y), lo, hi);
                    const float f = tc + kMagic;
                    cb[e] = as_u(f) + (uint32_t)zp;
                    if (WF) fv[e] = (f - kMagic) * sc;
                }
            } else {
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    const float o = q.offset(cache[k].get(e));
                    cb[e] = (uint32_t)((int)o + zp);
                    if (WF) fv[e] = o * sc;
                }
            }
            if (crow) store_codes<BITS, N>(crow, vi, cb);
            if (WF) {
                float4* fr = reinterpret_cast<float4*>(frow);
                store_nt(fr + vi * (N / 4), make_float4(fv[0], fv[1], fv[2], fv[3]));
                if (N == 8) store_nt(fr + vi * 2 + 1, make_float4(fv[4 % N], fv[5 % N], fv[6 % N], fv[7 % N]));
            }
        }
    };
    if (frow) quantize(std::true_type{});
    else quantize(std::false_type{});
}

// Per-row dequantize: out[r, c] = (code - zp[r]) * scale[r]
template <int BITS>
__global__ __launch_bounds__(kB) void k_dq_rows(const uint8_t* __restrict__ codes, int64_t cols,
                                                const float* __restrict__ scale,
                                                const int32_t* __restrict__ zp,
                                                float* __restrict__ out) {
    const int64_t row = blockIdx.y;
    const float s = scale[row];
    const int z = zp[row];
    const int64_t pstride = BITS == 8 ? cols : (cols + 1) / 2;
    const uint8_t* cr = codes + (size_t)row * (size_t)pstride;
    float* orow = out + (size_t)row * (size_t)cols;
    for (int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x; c < cols; c += (int64_t)gridDim.x * kB) {
        int q;
        if (BITS == 8) {
            q = (int)(int8_t)cr[c];
        } else {
            uint32_t b = cr[c >> 1];
            uint32_t nib = (c & 1) ? (b & 0xFu) : (b >> 4);
            q = ((int)(nib << 28)) >> 28;
        }
        orow[c] = (float)(q - z) * s;
    }
}

template <int DT, int BITS>
void launch_rows(const void* x, int64_t rows, int64_t cols, int affine, void* codes, float* fq,
                 float* scale, int32_t* zp, uint32_t* flags, hipStream_t st) {
    constexpr int N = Vec<DT>::N;
    const size_t code_align = BITS == 8 ? (N == 4 ? 4 : 8) : (N == 4 ? 2 : 4);
    const bool al = (cols % N == 0) && fqh::aligned(x, 16) && fqh::aligned(fq, 16) &&
                    fqh::aligned(codes, code_align) && (BITS == 8 || (cols / 2) % (N / 2) == 0);
    uint8_t* cd = (uint8_t*)codes;
    if (!al) {
        k_quant_rows<DT, BITS, false><<<dim3((unsigned)rows), kB, 0, st>>>(x, cols, affine, cd, fq, scale, zp, flags);
        return;
    }
    const int64_t nv = cols / N;
    // threads per row in the workgroup-per-row kernel: bf16 rows carry eight
    // elements per vector and are bound by arithmetic, so fewer threads with four
    // vectors each spread the per-row work thinner; fp32 rows stream faster with
    // 512 threads of two vectors (both measured on 8192-bf16 / 4096-fp32 rows).
    constexpr int TW = DT == FQ_BF16 ? 256 : 512;
    if (nv > 256 && nv <= 4 * TW) {
        const dim3 g((unsigned)rows);
        switch ((nv + TW - 1) / TW) {
            case 1: k_rows_wg<DT, BITS, TW, 1><<<g, TW, 0, st>>>(x, cols, affine, cd, fq, scale, zp, flags); break;
            case 2: k_rows_wg<DT, BITS, TW, 2><<<g, TW, 0, st>>>(x, cols, affine, cd, fq, scale, zp, flags); break;
            case 3: k_rows_wg<DT, BITS, TW, 3><<<g, TW, 0, st>>>(x, cols, affine, cd, fq, scale, zp, flags); break;
            default: k_rows_wg<DT, BITS, TW, 4><<<g, TW, 0, st>>>(x, cols, affine, cd, fq, scale, zp, flags); break;
        }
        return;
    }
    const dim3 grid((unsigned)((rows + kWaves - 1) / kWaves));
    if (nv <= 64)
        k_rows_wave<DT, BITS, 1><<<grid, kB, 0, st>>>(x, rows, cols, affine, cd, fq, scale, zp, flags);
    else if (nv <= 128)
        k_rows_wave<DT, BITS, 2><<<grid, kB, 0, st>>>(x, rows, cols, affine, cd, fq, scale, zp, flags);
    else if (nv <= 256)
        k_rows_wave<DT, BITS, 4><<<grid, kB, 0, st>>>(x, rows, cols, affine, cd, fq, scale, zp, flags);
    else if (nv <= 512)
        k_rows_wave<DT, BITS, 8><<<grid, kB, 0, st>>>(x, rows, cols, affine, cd, fq, scale, zp, flags);
    else
        k_rows_wave<DT, BITS, 16><<<grid, kB, 0, st>>>(x, rows, cols, affine, cd, fq, scale, zp, flags);
}

}  // namespace

extern "C" {

int fq_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols, int bits, int scheme,
                  void* codes, float* fq, float* scale, int32_t* zero_point, uint32_t* flags,
                  hipStream_t stream) {
    if (!fqh::valid_bits(bits) || !fqh::valid_scheme(scheme) || !fqh::valid_dtype(dtype))
        return FQ_E_UNSUPPORTED;
    if (!x || rows < 1 || cols < 1 || !scale || !zero_point) return FQ_E_INVALID;
    if (rows > 0x7FFFFFFF) return FQ_E_INVALID;
    if (!fqh::aligned(x, dtype == FQ_F32 ? 4 : 2) || !fqh::aligned(fq, 4) || !fqh::aligned(scale, 4) ||
        !fqh::aligned(zero_point, 4) || !fqh::aligned(flags, 4))
        return FQ_E_INVALID;
    const int aff = scheme == FQ_AFFINE;
    if (dtype == FQ_F32) {
        if (bits == 8) launch_rows<FQ_F32, 8>(x, rows, cols, aff, codes, fq, scale, zero_point, flags, stream);
        else launch_rows<FQ_F32, 4>(x, rows, cols, aff, codes, fq, scale, zero_point, flags, stream);
    } else {
        if (bits == 8) launch_rows<FQ_BF16, 8>(x, rows, cols, aff, codes, fq, scale, zero_point, flags, stream);
        else launch_rows<FQ_BF16, 4>(x, rows, cols, aff, codes, fq, scale, zero_point, flags, stream);
    }
    return fqh::launched();
}

int fq_dequantize_rows(const void* codes, int64_t rows, int64_t cols, int bits, const float* scale,
                       const int32_t* zero_point, float* out, hipStream_t stream) {
    if (!fqh::valid_bits(bits)) return FQ_E_UNSUPPORTED;
    if (!codes || rows < 1 || cols < 1 || !scale || !zero_point || !out) return FQ_E_INVALID;
    if (rows > 65535) {
        // grid.y limit: process in row batches
        for (int64_t r0 = 0; r0 < rows; r0 += 65535) {
            int64_t nr = rows - r0 < 65535 ? rows - r0 : 65535;
            const int64_t pstride = bits == 8 ? cols : (cols + 1) / 2;
            int st = fq_dequantize_rows((const uint8_t*)codes + r0 * pstride, nr, cols, bits, scale + r0,
                                        zero_point + r0, out + r0 * cols, stream);
            if (st != FQ_OK) return st;
        }
        return FQ_OK;
    }
    if (!fqh::aligned(scale, 4) || !fqh::aligned(zero_point, 4) || !fqh::aligned(out, 4))
        return FQ_E_INVALID;
    unsigned gx = (unsigned)((cols + kB - 1) / kB);
    if (gx > 64) gx = 64;
    dim3 grid(gx, (unsigned)rows);
    if (bits == 8) k_dq_rows<8><<<grid, kB, 0, stream>>>((const uint8_t*)codes, cols, scale, zero_point, out);
    else k_dq_rows<4><<<grid, kB, 0, stream>>>((const uint8_t*)codes, cols, scale, zero_point, out);
    return fqh::launched();
}

}  // extern "C"
