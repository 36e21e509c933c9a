// fq_device.h -- device-side building blocks shared by the gfx950 kernels:
// exact binary32 quotients with a fixed divisor, the saturating fp8 codec,
// bfloat16 widening, wave64 DPP reductions and the scale rules of the pages.
//
// Sources (page title, section):
//   [QAT] optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
//         Training (QAT) primitives": module docs (integer grid, fp8 table,
//         unified ULP rule), QuantParams::{from_minmax, from_absmax}.
//   [DQ]  aprender-train 0.32.0 entrenar/quant/double_quant.rs.
//   [CS]  CS349E 05_quantization_basics.py demo 4, `block_scaled` "e8m0".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fqk {

constexpr int kWave = 64;

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------------------
// Exact quotient fl(x / s) for a divisor fixed per group.
//
// Every code the method produces is a function of the binary32 quotient x/s, so
// the division must be correctly rounded; a multiply by a reciprocal is not.
// With y = RN(1/s) (one true division per group) the quotient is refined by two
// Markstein corrections (P. Markstein, IBM J. Res. Dev. 34(1), 1990):
//   q0 = RN(x y); r0 = x - s q0 (fma); q1 = RN(q0 + r0 y);
//   r1 = x - s q1 (fma);  q2 = RN(q1 + r1 y).
// q1 is within one ulp of x/s, r1 is exact and y is within half an ulp of 1/s, so
// q2 = RN(x/s) whenever no intermediate overflows or underflows.  The group is
// admitted to this path only for 2^-60 <= s <= 2^60; then
//   * |x/s| in the normal range: q2 == x / s bit for bit;
//   * tiny x: the residuals may round, but then |x/s| < 2^-17, below half the
//     smallest fp8 subnormal and below every integer rounding threshold, and q2
//     stays in that range -- every code taken from it is the same;
//   * x = +-Inf, NaN, or x*y overflowing: q2 is NaN, and x*y (+-Inf, NaN or a huge
//     finite value) carries the same code (saturation / NaN).
// The corrections add +0 to -0 when x is a zero, so the sign of x (the sign of
// x/s, as s > 0) is put back on the result.
// Other divisors take the compiler's correctly rounded division.
// ---------------------------------------------------------------------------
struct ExactDiv {
    float s, y;
    bool fast;
    __device__ __forceinline__ explicit ExactDiv(float s_) : s(s_) {
        y = 1.0f / s_;
        fast = (s_ >= 0x1p-60f) && (s_ <= 0x1p60f);
    }
    // from a divisor and its reciprocal RN(1 / s) computed earlier
    __device__ __forceinline__ ExactDiv(float s_, float y_) : s(s_), y(y_) {
        fast = (s_ >= 0x1p-60f) && (s_ <= 0x1p60f);
    }
    // Markstein path only; valid when `fast`.
    __device__ __forceinline__ float quick(float x) const {
        float q = x * y;
        float r = __builtin_fmaf(-s, q, x);
        q = __builtin_fmaf(r, y, q);
        r = __builtin_fmaf(-s, q, x);
        q = __builtin_fmaf(r, y, q);
        return (q != q) ? x * y : __builtin_copysignf(q, x);
    }
    __device__ __forceinline__ float operator()(float x) const { return fast ? quick(x) : x / s; }
};

// The two Markstein corrections alone, for callers that know x is finite and
// |x/s| is bounded by the group's own range (no overflow, no NaN): 5 operations.
// A zero x may come back as +0; callers that need the sign of zero use ExactDiv.
__device__ __forceinline__ float quick_div(float x, float s, float y) {
    float q = x * y;
    float r = __builtin_fmaf(-s, q, x);
    q = __builtin_fmaf(r, y, q);
    r = __builtin_fmaf(-s, q, x);
    return __builtin_fmaf(r, y, q);
}
__device__ __forceinline__ bool fast_divisor(float s) { return (s >= 0x1p-60f) && (s <= 0x1p60f); }

// Adding 1.5 * 2^23 to a binary32 v with |v| < 2^22 leaves round-half-even(v) in
// the low mantissa bits: the sum's ulp is 1 and the constant is even, so
// RNE(v + kMagic) = RNE(v) + kMagic exactly; (sum - kMagic) is RNE(v) as a float
// (+0 for a zero) and the low bits of the sum's pattern hold RNE(v) in two's
// complement.
constexpr float kMagic = 12582912.0f;
constexpr uint32_t kMagicBits = 0x4B400000u;

// compile-time loop: f(std::integral_constant<int, I>{}) for I in [0, N)
template <int I, int N>
struct StaticFor {
    template <class F>
    __device__ __forceinline__ static void run(F&& f) {
        f(std::integral_constant<int, I>{});
        StaticFor<I + 1, N>::run(f);
    }
};
template <int N>
struct StaticFor<N, N> {
    template <class F>
    __device__ __forceinline__ static void run(F&&) {}
};

// ---------------------------------------------------------------------------
// bfloat16 -> binary32 (exact: bf16 is the upper half of a binary32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return as_f(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return as_f(pair & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// wave64 reductions.  DPP row operations stay inside 16-lane rows; the two
// cross-row steps use lane shuffles.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return as_f(dpp_u<CTRL>(as_u(v)));
}
// lane J of each 16-lane row, broadcast to the whole row (DPP row_newbcast)
template <int J>
__device__ __forceinline__ float row_bcast_f(float v) {
    return dpp_f<0x150 + J>(v);
}
template <int J>
__device__ __forceinline__ uint32_t row_bcast_u(uint32_t v) {
    return dpp_u<0x150 + J>(v);
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kMirror = 0x140;      // lane i <-> 15-i within 16

// max over each 4-lane quad, result in every lane of the quad
__device__ __forceinline__ uint32_t quad_max_u(uint32_t v) {
    v = max(v, dpp_u<kQuadXor1>(v));
    v = max(v, dpp_u<kQuadXor2>(v));
    return v;
}
// max over each 16-lane row, result in every lane of the row
__device__ __forceinline__ uint32_t row16_max_u(uint32_t v) {
    v = quad_max_u(v);
    v = max(v, dpp_u<kHalfMirror>(v));
    v = max(v, dpp_u<kMirror>(v));
    return v;
}
__device__ __forceinline__ float row16_min_f(float v) {
    v = fminf(v, dpp_f<kQuadXor1>(v));
    v = fminf(v, dpp_f<kQuadXor2>(v));
    v = fminf(v, dpp_f<kHalfMirror>(v));
    v = fminf(v, dpp_f<kMirror>(v));
    return v;
}
__device__ __forceinline__ float row16_max_f(float v) {
    v = fmaxf(v, dpp_f<kQuadXor1>(v));
    v = fmaxf(v, dpp_f<kQuadXor2>(v));
    v = fmaxf(v, dpp_f<kHalfMirror>(v));
    v = fmaxf(v, dpp_f<kMirror>(v));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
    v = row16_max_u(v);
    v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}
__device__ __forceinline__ float wave_min_f(float v) {
    v = row16_min_f(v);
    v = fminf(v, __shfl_xor(v, 16));
    v = fminf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
    v = row16_max_f(v);
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Order-preserving signed key of a binary32 that is not NaN (-0 sorts just
// below +0); the map is its own inverse.  Integer min / max fold into DPP
// instructions (v_max_i32_dpp), float ones need separate moves.
__device__ __forceinline__ int32_t fkey(float f) {
    const int32_t i = (int32_t)as_u(f);
    return i ^ ((i >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float fkey_value(int32_t k) { return as_f((uint32_t)(k ^ ((k >> 31) & 0x7FFFFFFF))); }

// DPP move that leaves lanes of rows outside ROWS unchanged
template <int CTRL, int ROWS>
__device__ __forceinline__ int32_t dpp_keep_i(int32_t v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xF, false);
}
constexpr int kRowBcast15 = 0x142;  // lane 15 of each row into the next row
constexpr int kRowBcast31 = 0x143;  // lane 31 into rows 2 and 3

// max / min over the whole wave as a wave-uniform value: 16-lane rows by DPP,
// then rows folded with the row broadcasts into lane 63
__device__ __forceinline__ int32_t wave_max_i(int32_t v) {
    v = max(v, (int32_t)dpp_u<kQuadXor1>((uint32_t)v));
    v = max(v, (int32_t)dpp_u<kQuadXor2>((uint32_t)v));
    v = max(v, (int32_t)dpp_u<kHalfMirror>((uint32_t)v));
    v = max(v, (int32_t)dpp_u<kMirror>((uint32_t)v));
    v = max(v, dpp_keep_i<kRowBcast15, 0xA>(v));
    v = max(v, dpp_keep_i<kRowBcast31, 0xC>(v));
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int32_t wave_min_i(int32_t v) {
    v = min(v, (int32_t)dpp_u<kQuadXor1>((uint32_t)v));
    v = min(v, (int32_t)dpp_u<kQuadXor2>((uint32_t)v));
    v = min(v, (int32_t)dpp_u<kHalfMirror>((uint32_t)v));
    v = min(v, (int32_t)dpp_u<kMirror>((uint32_t)v));
    v = min(v, dpp_keep_i<kRowBcast15, 0xA>(v));
    v = min(v, dpp_keep_i<kRowBcast31, 0xC>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// ---------------------------------------------------------------------------
// Stores of outputs that no later step of the same kernel reads: with the
// nontemporal hint they stream to HBM instead of settling in the Infinity Cache
// as dirty lines that the next kernel's traffic would have to write back first.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(float4* p, float4 v) {
    f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
}

// ---------------------------------------------------------------------------
// Streaming 16-byte loads of kernel inputs: plain, or with the nontemporal hint
// (NT).  Which kernels take the hint is a measured choice: it changes what the
// Infinity Cache holds for the kernels after them.  Measured over the bench step
// on one box, two runs each (step ms): no hint 2.9602 / 2.9567; the hint on the
// tensor-scope reduction, the MX fp8 blocks and the fp8 quantize 2.9466 /
// 2.9483 (the fp8 amax pass 65 -> 47 us, the MX blocks 69 -> 64 us, the fp8
// quantize after the amax 94 -> 99 us, both fp8 dequantizes -2.5 us, the 4-bit
// dequantize +10 us); on the reduction alone 2.9554 / 2.9509 (the fp8 quantize,
// no longer finding x in the cache, 94 -> 104 us).  The per-row kernels keep
// plain loads: with the hint the three row ops after the first, which find the
// [4096, 4096] weight in the cache, lost 2.5 us each.  Of the wide-layout kernels
// only the MX fp8 blocks take it (load16's NT), on bf16 input: with the hint the
// fp32 wide kernels (NVFP4, group-wise) fetched 10-12 % more than they read (a
// lane's four consecutive 16-byte loads are four instructions whose lines the L2
// must keep between them), and the FP4 blocks ran 4 % slower cold.
// ---------------------------------------------------------------------------
#ifndef FQ_NT_LOADS_REDUCE
#define FQ_NT_LOADS_REDUCE 1
#endif
#ifndef FQ_NT_LOADS_FP8
#define FQ_NT_LOADS_FP8 1
#endif
#ifndef FQ_NT_LOADS_ROWS
#define FQ_NT_LOADS_ROWS 0
#endif
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ float4 ld_f4(const float4* p) {
    if constexpr (NT) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}
template <bool NT>
__device__ __forceinline__ uint4 ld_u4(const uint4* p) {
    if constexpr (NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

// ---------------------------------------------------------------------------
// Buffer loads and stores with explicit cache-policy bits (gfx950 CPol: sc0 = 1,
// nt = 2, sc1 = 16) from a wave-uniform base address and a per-lane byte offset
// below 2^31 (a raw buffer resource: offsets past num_records read 0 / are not
// written, never fault).
// ---------------------------------------------------------------------------
enum { kCpSc0 = 1, kCpNt = 2, kCpSc1 = 16 };
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
template <int CP>
__device__ __forceinline__ float4 buf_load16(const void* base, uint32_t off) {
    const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(wave_rsrc(base), off, 0, CP);
    return make_float4(as_f(r.x), as_f(r.y), as_f(r.z), as_f(r.w));
}
template <int CP>
__device__ __forceinline__ void buf_store16(void* base, uint32_t off, float4 v) {
    const u32x4 w = {as_u(v.x), as_u(v.y), as_u(v.z), as_u(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(w, wave_rsrc(base), off, 0, CP);
}

// Stream store of float4 number i of `out`, for indices whose distance from the
// wave's lane number is the same in every lane (i - lane wave-uniform, as in
// every covering-grid layout here): CP < 0 is the global nontemporal store,
// otherwise a buffer store with cache policy CP from the wave's base address.
template <int CP>
__device__ __forceinline__ void store_out(float4* out, int64_t i, float4 v) {
    if constexpr (CP < 0) {
        store_nt(out + i, v);
    } else {
        const int lane = (int)(threadIdx.x & (kWave - 1));
        const uint64_t a = (uint64_t)(out + (i - lane));
        // readfirstlane returns an int: both halves go back through uint32_t, so a
        // low word with bit 31 set is not sign-extended into the high word
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
        const uint64_t ua = ((uint64_t)hi << 32) | (uint64_t)lo;
        buf_store16<CP>(reinterpret_cast<void*>(ua), (uint32_t)lane * 16u, v);
    }
}

// ---------------------------------------------------------------------------
// Wide layout: sixteen consecutive elements per lane, so that per-block work
// (reductions, scales, reciprocals) is shared by four times as many elements as
// with one 16-byte vector per lane.  A lane's sixteen outputs are contiguous in
// memory; they leave through a per-wave LDS transpose so that every store
// instruction writes one contiguous run across the wave.
// ---------------------------------------------------------------------------
// bits of |v| when v is finite, else 0: the key of a finite-amax reduction
// (unsigned order of the bits is the order of the magnitudes)
__device__ __forceinline__ uint32_t finite_abs_bits(float v) {
    const uint32_t a = as_u(v) & 0x7FFFFFFFu;
    return a < 0x7F800000u ? a : 0u;
}

// element i of a float32 or (BF16) bfloat16 tensor as binary32 (bf16 widens exactly)
template <bool BF16>
__device__ __forceinline__ float load_elem(const void* __restrict__ x, int64_t i) {
    if constexpr (!BF16) return reinterpret_cast<const float*>(x)[i];
    else return as_f((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
}

constexpr int kWide = 16;
constexpr int kWidePad = kWide + 4;  // LDS floats per lane of the staging buffer (16-byte rows)

// elements 16 v .. 16 v + 15 of x (binary32, or bf16 widened exactly); NT: bf16
// loads with the nontemporal hint
template <bool BF16, bool NT = false>
__device__ __forceinline__ void load16(const void* __restrict__ x, int64_t v, float (&e)[kWide]) {
    if constexpr (!BF16) {
        const float4* p = reinterpret_cast<const float4*>(x) + 4 * v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 q = ld_f4<false>(p + j);
            e[4 * j] = q.x;
            e[4 * j + 1] = q.y;
            e[4 * j + 2] = q.z;
            e[4 * j + 3] = q.w;
        }
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(x) + 2 * v;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 q = ld_u4<NT>(p + j);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                e[8 * j + 2 * k] = bf16_lo(w[k]);
                e[8 * j + 2 * k + 1] = bf16_hi(w[k]);
            }
        }
    }
}

// Stores the lane's sixteen values o as elements 16 v .. 16 v + 15 of out
// (nontemporal) through sw, this wave's LDS staging buffer of kWave * kWidePad
// floats.  v must be blockIdx.x * blockDim.x + threadIdx.x.  Every thread of the
// workgroup calls it (it holds a barrier); float4s from index 4 nvec on are not
// stored.
__device__ __forceinline__ void store16_staged(float4* __restrict__ out, int64_t v, int64_t nvec,
                                               const float (&o)[kWide], float4* sw) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        sw[lane * (kWidePad / 4) + j] = make_float4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
    __syncthreads();
    // float4 number idx of the wave's 256 belongs to lane idx / 4, part idx % 4
    const int64_t wbase = (v - lane) * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = k * kWave + lane;
        const float4 val = sw[(idx / 4) * (kWidePad / 4) + (idx % 4)];
        if (wbase + idx < nvec * 4) store_nt(out + wbase + idx, val);
    }
}

// ---------------------------------------------------------------------------
// Finite min / max / non-finite accumulation over binary32 values.
// `nf` collects max(|x| bits): it reaches 0x7F800000 iff an Inf or NaN was seen.
// ---------------------------------------------------------------------------
struct MinMax {
    float mn = __builtin_inff();
    float mx = -__builtin_inff();
    uint32_t nf = 0;
    // a non-finite v becomes a quiet NaN, which fminf / fmaxf pass over
    __device__ __forceinline__ void add(float v) {
        const uint32_t a = as_u(v) & 0x7FFFFFFFu;
        const float vf = a < 0x7F800000u ? v : __builtin_nanf("");
        mn = fminf(mn, vf);
        mx = fmaxf(mx, vf);
        nf = max(nf, a);
    }
    __device__ __forceinline__ void merge(float omn, float omx, uint32_t onf) {
        mn = fminf(mn, omn);
        mx = fmaxf(mx, omx);
        nf = max(nf, onf);
    }
    __device__ __forceinline__ bool nonfinite() const { return nf >= 0x7F800000u; }
};

// ---------------------------------------------------------------------------
// Integer calibration ([QAT] QuantParams::from_minmax / from_absmax), binary32.
// ---------------------------------------------------------------------------
struct IntRange {
    int qmin, qmax;
};
__device__ __forceinline__ IntRange int_range(int bits, bool affine) {
    // [QAT] IntDtype::q_range: restricted symmetric, full-range affine
    if (bits == 8) return affine ? IntRange{-128, 127} : IntRange{-127, 127};
    return affine ? IntRange{-8, 7} : IntRange{-7, 7};
}

struct IntCal {
    float scale;
    int zp;
    bool degenerate;
};

// (min, max) over the finite elements; a group without finite elements arrives
// as (+inf, -inf) and is degenerate.
__device__ __forceinline__ IntCal calibrate(float mn, float mx, IntRange r, bool affine) {
    IntCal c{0.0f, 0, true};
    if (!(mn <= mx)) return c;  // no finite element
    if (!affine) {
        float absmax = fmaxf(fabsf(mn), fabsf(mx));
        if (!(absmax > 0.0f)) return c;
        float s = absmax / (float)r.qmax;
        if (!(s > 0.0f) || !(s < __builtin_inff())) return c;
        c.scale = s;
        c.degenerate = false;
        return c;
    }
    float rmin = fminf(mn, 0.0f);
    float rmax = fmaxf(mx, 0.0f);
    float range = rmax - rmin;
    if (!(range > 0.0f)) return c;
    float s = range / (float)(r.qmax - r.qmin);
    if (!(s > 0.0f) || !(s < __builtin_inff())) return c;
    float z = rintf((float)r.qmin - rmin / s);
    z = fminf(fmaxf(z, (float)r.qmin), (float)r.qmax);
    c.scale = s;
    c.zp = (int)z;
    c.degenerate = false;
    return c;
}

// Quantize helper for one group: offset = clamp(RNE(x/s), qmin - zp, qmax - zp),
// code = offset + zp.  NaN -> code 0 (offset -zp); scale 0 -> code 0.
struct IntQ {
    ExactDiv div;
    float lo, hi;   // qmin - zp, qmax - zp as floats
    float nan_off;  // -zp
    bool zero;      // scale == 0
    __device__ __forceinline__ IntQ(float scale, int zp, IntRange r)
        : div(scale == 0.0f ? 1.0f : scale),
          lo((float)(r.qmin - zp)),
          hi((float)(r.qmax - zp)),
          nan_off((float)(-zp)),
          zero(scale == 0.0f) {}
    // offset q - zp as an exact small integer in a float (a zero offset is +0,
    // as the integer difference q - zp converts to +0)
    __device__ __forceinline__ float offset(float x) const {
        if (zero) return nan_off;  // code 0 (zp is 0 for degenerate groups)
        float t = div(x);
        float r = fminf(fmaxf(rintf(t), lo), hi) + 0.0f;
        return (t != t) ? nan_off : r;
    }
    // offset with the quotient mode fixed at compile time: 0 = zero scale,
    // 1 = divisor in the exact-quotient window, 2 = true division
    template <int MODE>
    __device__ __forceinline__ float offset_m(float x) const {
        if (MODE == 0) return nan_off;
        float t = MODE == 1 ? div.quick(x) : x / div.s;
        float r = fminf(fmaxf(rintf(t), lo), hi) + 0.0f;
        return (t != t) ? nan_off : r;
    }
    // offset for a group whose divisor passed the fast test and whose inputs are
    // known finite with |x / s| bounded by the group's own range
    __device__ __forceinline__ float offset_finite(float x) const {
        float t = div.quick(x);
        return fminf(fmaxf(rintf(t), lo), hi) + 0.0f;
    }
};

// ---------------------------------------------------------------------------
// fp8 codec.  [QAT] module docs "fp8 quantization": E4M3 (3 mantissa bits, bias
// 7, max 448, no Inf, NaN S.1111.111) and E5M2 (2 mantissa bits, bias 15, max
// 57344, IEEE-like).  Rounding is the page's unified ULP rule: for a > 0 with
// e = floor(log2 a), step = 2^(max(e, emin) - mbits), ties to even, then a
// rounded magnitude above max saturates to max; +-Inf saturate; NaN -> 0x7F.
//
// Encoding arithmetic (bitwise emulation): with E the biased binary32 exponent
// of a, clamped below at emin, k = RNE(a * 2^(mbits - e)) is the rounded
// significand on the step grid (k in [2^mbits, 2^(mbits+1)] in a normal binade,
// [0, 2^mbits] below emin), and the fp8 code is k + ((e + bias - 1) << mbits):
// the carry k = 2^(mbits+1) moves into the next binade by itself, and the
// subnormal codes are k themselves.  Codes above the largest finite code are
// clamped to it.
// ---------------------------------------------------------------------------
template <int FMT>
struct Fp8Fmt;
template <>
struct Fp8Fmt<0> {  // E4M3
    static constexpr int mbits = 3, bias = 7;
    static constexpr uint32_t max_code = 0x7E;
    static constexpr float big = 0x1p10f;  // anything >= this saturates
    static constexpr float rebias = 0x1p120f;  // 2^(127 - bias)
};
template <>
struct Fp8Fmt<1> {  // E5M2
    static constexpr int mbits = 2, bias = 15;
    static constexpr uint32_t max_code = 0x7B;
    static constexpr float big = 0x1p17f;
    static constexpr float rebias = 0x1p112f;
};

// |y| -> 7-bit magnitude code (finite or Inf input; NaN handled by the caller)
template <int FMT>
__device__ __forceinline__ uint32_t fp8_mag_code(float y) {
    using F = Fp8Fmt<FMT>;
    constexpr uint32_t emin_biased = 127u + 1u - F::bias;  // binary32 field of 2^emin
    float a = fminf(fabsf(y), F::big);
    uint32_t E = max(as_u(a) >> 23, emin_biased);
    float k = rintf(__builtin_amdgcn_ldexpf(a, (int)(127u + F::mbits) - (int)E));
    uint32_t code = (uint32_t)k + ((E - emin_biased) << F::mbits);
    return min(code, F::max_code);
}

template <int FMT>
__device__ __forceinline__ uint32_t fp8_encode(float y) {
    uint32_t code = fp8_mag_code<FMT>(y) | ((as_u(y) >> 24) & 0x80u);
    return (y != y) ? 0x7Fu : code;
}

// The same cast on the CDNA4 conversion unit, four values per call, packed
// little-endian.  v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 round to nearest even on
// the E4M3 / E5M2 grid; an exhaustive comparison over all 2^32 binary32 inputs
// with fp8_encode above found them equal for every |y| <= max-normal (zeros and
// binary32 subnormals included), while larger magnitudes and infinities come
// out as NaN / Inf codes and a NaN comes out as a negative NaN byte.  So the
// input is clamped to [-max, max] first (saturation, sign of zero kept) and NaN
// inputs are patched to 0x7F afterwards.
template <int FMT>
__device__ __forceinline__ uint32_t fp8_encode4_hw(float y0, float y1, float y2, float y3) {
    constexpr float M = FMT == 0 ? 448.0f : 57344.0f;
    const float c0 = fminf(fmaxf(y0, -M), M), c1 = fminf(fmaxf(y1, -M), M);
    const float c2 = fminf(fmaxf(y2, -M), M), c3 = fminf(fmaxf(y3, -M), M);
    int w;
    if (FMT == 0) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(c0, c1, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(c2, c3, w, true);
    }
    uint32_t u = (uint32_t)w;
    if ((y0 != y0) | (y1 != y1) | (y2 != y2) | (y3 != y3)) {
        const uint32_t m = ((y0 != y0) ? 0xFFu : 0u) | ((y1 != y1) ? 0xFF00u : 0u) |
                           ((y2 != y2) ? 0xFF0000u : 0u) | ((y3 != y3) ? 0xFF000000u : 0u);
        u = (u & ~m) | (0x7F7F7F7Fu & m);
    }
    return u;
}

// Value of a code that is not NaN and not Inf: the 7 magnitude bits placed under
// the binary32 exponent field give 2^(E-127) (1 + M/2^mb) (or a binary32
// subnormal for E = 0); multiplying by 2^(127 - bias) rebiases exactly.
template <int FMT>
__device__ __forceinline__ float fp8_decode_finite(uint32_t b) {
    using F = Fp8Fmt<FMT>;
    float v = as_f((b & 0x7Fu) << (23 - F::mbits)) * F::rebias;
    return as_f(as_u(v) | ((b & 0x80u) << 24));
}

// Value of any code (NaN patterns -> NaN, E5M2 infinities -> +-Inf)
template <int FMT>
__device__ __forceinline__ float fp8_decode(uint32_t b) {
    float v = fp8_decode_finite<FMT>(b);
    uint32_t m = b & 0x7Fu;
    if (FMT == 0) return m == 0x7Fu ? __builtin_nanf("") : v;
    if (m >= 0x7Cu) {
        float inf = as_f(0x7F800000u | ((b & 0x80u) << 24));
        return m == 0x7Cu ? inf : __builtin_nanf("");
    }
    return v;
}

// The four codes of w (code e in byte e) decoded by gfx950's conversion unit
// (v_cvt_pk_f32_fp8 / v_cvt_pk_f32_bf8, two codes per instruction, OCP formats):
// exact, and for every one of the 256 codes of either format the value of
// fp8_decode (E4M3 S.1111.111 and E5M2 S.11111.xx with xx != 0 -> NaN, E5M2
// S.11111.00 -> +-Inf).
template <int FMT>
__device__ __forceinline__ void fp8_decode4_hw(uint32_t w, float (&d)[4]) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    v2f lo, hi;
    if constexpr (FMT == 0) {
        lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    } else {
        lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
    }
    d[0] = lo.x;
    d[1] = lo.y;
    d[2] = hi.x;
    d[3] = hi.y;
}

// ---------------------------------------------------------------------------
// Stochastic rounding ([QAT] module docs "Rounding modes", RoundingMode::
// Stochastic): the uniform variate of element index i is word i mod 4 of
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11) at counter (floor(i/4) low 32 bits, high 32 bits, 0, 0)
// under key (seed low, seed high), as a binary32 with 24 random bits:
// (word >> 8) 2^-24.  Rounding: up iff the draw is below fl(t - floor(t)).
// ---------------------------------------------------------------------------
// multipliers and Weyl key increments of the published generator
constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;

__device__ __forceinline__ uint4 philox4x32_10(uint64_t block, uint32_t k0, uint32_t k1) {
    uint32_t c0 = (uint32_t)block, c1 = (uint32_t)(block >> 32), c2 = 0u, c3 = 0u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += kW0;
            k1 += kW1;
        }
        const uint64_t p0 = (uint64_t)kM0 * c0;
        const uint64_t p1 = (uint64_t)kM1 * c2;
        // three-input xors in one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ uint32_t word(const uint4& w, int i) {
    return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

// The four 24-bit draws of chunk c (elements offset + 4c .. offset + 4c + 3), as
// integers j (the variate is j 2^-24).
struct Draws {
    uint32_t k0, k1;
    uint64_t base;  // offset >> 2
    int shift;      // offset & 3
    static Draws make(uint64_t seed, uint64_t offset) {
        return Draws{(uint32_t)seed, (uint32_t)(seed >> 32), offset >> 2, (int)(offset & 3)};
    }
    __device__ __forceinline__ void get(int64_t c, uint32_t (&j)[4]) const {
        const uint64_t b = base + (uint64_t)c;
        const uint4 w0 = philox4x32_10(b, k0, k1);
        if (shift == 0) {
            j[0] = w0.x >> 8;
            j[1] = w0.y >> 8;
            j[2] = w0.z >> 8;
            j[3] = w0.w >> 8;
        } else {
            const uint4 w1 = philox4x32_10(b + 1, k0, k1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = e + shift;
                j[e] = (s < 4 ? word(w0, s) : word(w1, s - 4)) >> 8;
            }
        }
    }
};

// round t stochastically with the draw j 2^-24: floor(t) + (j 2^-24 < frac);
// +-Inf stay themselves (their frac is NaN, which compares false), NaN stays NaN
__device__ __forceinline__ float round_sr(float t, uint32_t j) {
    const float lower = floorf(t);
    const float frac = t - lower;
    return ((float)j * 0x1p-24f < frac) ? lower + 1.0f : lower;
}

// fp8 cast with stochastic rounding: the unified-ULP step of |y|, ratio = |y| /
// step exact, rounded stochastically, code = k + binade, saturated; NaN -> 0x7F
template <int FMT>
__device__ __forceinline__ uint32_t fp8_encode_sr(float y, uint32_t j) {
    using F = Fp8Fmt<FMT>;
    constexpr uint32_t emin_biased = 127u + 1u - F::bias;  // binary32 field of 2^emin
    const float a = fminf(fabsf(y), F::big);                // anything >= big saturates
    const uint32_t E = max(as_u(a) >> 23, emin_biased);
    const float k = round_sr(__builtin_amdgcn_ldexpf(a, (int)(127u + F::mbits) - (int)E), j);
    const uint32_t code = min((uint32_t)k + ((E - emin_biased) << F::mbits), F::max_code);
    return (y != y) ? 0x7Fu : (code | ((as_u(y) >> 24) & 0x80u));
}


// pack the low bytes of four words into one word (little-endian order)
__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
    uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
    return lo | hi;
}
// two 4-bit codes (as ints) -> one byte, first one in the high nibble
__device__ __forceinline__ uint32_t nib2(int c0, int c1) {
    return (((uint32_t)c0 & 0xFu) << 4) | ((uint32_t)c1 & 0xFu);
}

}  // namespace fqk
