// q4dq.hip -- 64-element 4-bit absmax blocks with 8-bit double quantization of
// the block scales over groups of 256 blocks, and its dequantization.
//
// [DQ] aprender-train 0.32.0 entrenar/quant/double_quant.rs, "Double
// quantization for QLoRA": quantize_4bit_double (super-scale = max of 256 block
// scales with a 1e-8 floor, u8 = round(scale / super * 255)), dequantize_4bit_double
// and reconstruct_scales (scale = u8 / 255 * super; nibble order: element i in byte
// i/2, even i in the high nibble, two's complement).  The first-level quantizer
// (imported by the page): blocks of 64, scale = absmax / 7, ties to even.
//
// A 1024-thread workgroup owns super-blocks of 256 blocks = 16384 elements =
// 64 KiB of input, two consecutive ones in turn (four for the dequantize).
// Thread t loads float4 number j*1024 + t for j = 0..3, so each 64-element block
// is one 16-lane DPP row of a wave; the block absmax is a 4-step row reduction.
// The super-block stays in registers: codes are written at once, the
// super-scale comes from a wave + LDS maximum, and the reconstruction is written
// from the codes kept in registers -- the input is read once.  The next
// super-block's loads are issued before the current reconstruction is stored,
// and an LDS reservation keeps one workgroup per compute unit (both measured
// fastest on MI355X).
#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;
constexpr int kWaves = kB / kWave;
constexpr int kBlockElems = 64;
constexpr int kGroup = 256;                         // block scales per super-scale
constexpr int kSuperElems = kBlockElems * kGroup;   // 16384
constexpr int kJ = kSuperElems / (4 * kB);          // 16 float4 per thread (generic kernels)
#ifndef FQ_Q4_THREADS
#define FQ_Q4_THREADS 1024
#endif
constexpr int kQ4Threads = FQ_Q4_THREADS;            // threads per super-block (full kernels)
// Resident workgroups per compute unit for the full-super-block kernels (one:
// measured fastest on MI355X for both directions), and an upper bound of their
// static LDS.
#ifndef FQ_OCC_Q4
#define FQ_OCC_Q4 1
#endif
#ifndef FQ_OCC_Q4DQ
#define FQ_OCC_Q4DQ 1
#endif
#ifndef FQ_Q4_NSB
#define FQ_Q4_NSB 4
#endif
constexpr int kQuantNsb = FQ_Q4_NSB;  // super-blocks per workgroup of the quantize kernel
#ifndef FQ_Q4DQ_NSB
#define FQ_Q4DQ_NSB 4
#endif
constexpr int kDequantNsb = FQ_Q4DQ_NSB;  // super-blocks per workgroup of the dequantize kernel
constexpr int kOccQuant = FQ_OCC_Q4;
constexpr int kOccDequant = FQ_OCC_Q4DQ;
// Cache policy of the full-super-block kernels, measured over the whole bench step
// on one box (quantize + reconstruct / dequantize, us): plain loads and global
// nontemporal stores 1561 / 827; nontemporal loads (CPol nt) of x, nontemporal
// device-scope stores (nt sc1) of the reconstruction and nontemporal code stores
// 1494 / 830; the same with plain code stores 1467 / 859 (the dequantize then
// writes back the codes the quantize left dirty in the cache: the same total);
// nt sc1 stores in the dequantize too 1496 / 864; the codes through buffer
// stores (nt, or nt sc1) no faster than global nontemporal ones.  Staging a
// super-block's codes in LDS so that each lane stores 16 bytes (8 store
// instructions per super-block instead of 64): 1487-1488 against 1498-1499 us
// (three runs each, one box).  The dequantize with one super-block per workgroup
// and plain stores ran 811-815 against 825-828 us cold on its own, but the
// quantize + dequantize step took 2.328-2.340 against 2.321-2.333 ms (the plain
// stores leave dirty lines for the next operation), and plain stores with four
// super-blocks 848-853 us; two, four or any number of resident workgroups per CU
// instead of one 876-886 us.
#ifndef FQ_Q4_LD_CP
#define FQ_Q4_LD_CP 2
#endif
#ifndef FQ_Q4_ST_CP
#define FQ_Q4_ST_CP 18
#endif
#ifndef FQ_Q4DQ_ST_CP
#define FQ_Q4DQ_ST_CP -1
#endif
#ifndef FQ_Q4_CODES_NT
#define FQ_Q4_CODES_NT 1
#endif
constexpr int kLdCp = FQ_Q4_LD_CP;      // cache policy of the x loads (-1: plain global loads)
constexpr int kStCp = FQ_Q4_ST_CP;      // cache policy of the reconstruction stores (-1: global nontemporal)
constexpr int kDqStCp = FQ_Q4DQ_ST_CP;  // cache policy of the dequantize stores (-1: global nontemporal)
constexpr bool kCodesNt = FQ_Q4_CODES_NT != 0;  // packed codes and u8 scales with the nontemporal hint
#ifndef FQ_Q4_CODES_LDS
#define FQ_Q4_CODES_LDS 1
#endif
constexpr bool kCodesLds = FQ_Q4_CODES_LDS != 0;  // codes staged in LDS, stored 16 bytes per lane
constexpr int kQuantLds = 2048 + (kCodesLds ? kSuperElems / 2 : 0);
constexpr int kDequantLds = 1024;

// code of x in a block with scale s (s > 0): clamp(RNE(x / s), -7, 7), NaN -> 0
__device__ __forceinline__ float q4_code(const ExactDiv& d, float x) {
    float t = d(x);
    float r = fminf(fmaxf(rintf(t), -7.0f), 7.0f) + 0.0f;  // code 0 is +0
    return (t != t) ? 0.0f : r;
}

// code and scale-code stores, with the nontemporal hint when kCodesNt
__device__ __forceinline__ void st_u16(uint16_t* p, uint16_t v) {
    if constexpr (kCodesNt) __builtin_nontemporal_store(v, p);
    else *p = v;
}
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
    if constexpr (kCodesNt) __builtin_nontemporal_store(v, p);
    else *p = v;
}
// [DQ] u8 scale code: clamp(round_half_away(s / S * 255), 0, 255)
__device__ __forceinline__ uint32_t u8_scale(float s, float S) {
    float v = (s / S) * 255.0f;
    v = roundf(v);
    v = fminf(fmaxf(v, 0.0f), 255.0f);
    return (uint32_t)v;
}
// [DQ] reconstruct_scales: q / 255 * super, left to right
__device__ __forceinline__ float recon_scale(uint32_t u, float S) { return (float)u / 255.0f * S; }

// Full super-block, 16-byte aligned buffers.
//
// Per thread: 16 float4 (elements of 16 different blocks).  Per 64-element
// block (a 16-lane row at step j): the absmax is a DPP row maximum; the block's
// scale s = absmax / 7 and its reciprocal are computed once, by the row's lane j,
// and broadcast back to the row with DPP row_newbcast -- one pair of true
// divisions per lane per super-block instead of one per float4.  Codes are
// RNE(fl(x / s)) clamped to +-7 (kMagic rounding); the packed nibbles stay in
// registers for the reconstruction written after the super-scale is known.
// A wave holding Inf / NaN takes the general per-element rule (finite absmax,
// NaN -> 0, +-Inf -> +-7).
__device__ __forceinline__ uint32_t abs_bits(float v) { return as_u(v) & 0x7FFFFFFFu; }
// two nibbles from two magic-rounded floats (low 4 bits of their patterns)
__device__ __forceinline__ uint32_t nib_pair(float f0, float f1) {
    return __builtin_amdgcn_ubfe(as_u(f0), 0, 4) << 4 | __builtin_amdgcn_ubfe(as_u(f1), 0, 4);
}
// general code of one element, as an int in [-7, 7]
__device__ __forceinline__ int q4_general(float x, float s, float y, bool fast) {
    if (s == 0.0f) return 0;
    ExactDiv d(s);
    d.y = y;
    d.fast = fast;
    return (int)q4_code(d, x);
}

template <int TPB, int NSB>
__global__ __launch_bounds__(TPB) void k_q4dq_full(const float* __restrict__ x, uint8_t* __restrict__ packed,
                                                   uint8_t* __restrict__ qscale, float* __restrict__ super_scale,
                                                   float* __restrict__ block_scale, float* __restrict__ recon,
                                                   uint32_t* __restrict__ flags) {
    constexpr int J = kSuperElems / (4 * TPB);  // float4 per thread
    constexpr int RW = TPB / 16;                // 16-lane rows per workgroup
    constexpr int NW = TPB / kWave;             // waves per workgroup
    const int t = threadIdx.x;
    const int lrow = t & 15;  // position inside the 16-lane row
    float4 v[J];
    auto load_sb = [&](const float* base) {
        if constexpr (kLdCp < 0) {
            const float4* xv = reinterpret_cast<const float4*>(base);
#pragma unroll
            for (int j = 0; j < J; ++j) v[j] = xv[j * TPB + t];
        } else {
#pragma unroll
            for (int j = 0; j < J; ++j) v[j] = buf_load16<kLdCp>(base, (uint32_t)(j * TPB + t) * 16u);
        }
    };
    load_sb(x + (int64_t)blockIdx.x * NSB * kSuperElems);

    __shared__ float s_scale[kGroup];
    __shared__ uint32_t s_u8[kGroup / 4];
    __shared__ float s_max[NW];
    __shared__ uint4 s_codes[kCodesLds ? kSuperElems / 32 : 1];  // the super-block's packed codes
    uint16_t* const s_pk = reinterpret_cast<uint16_t*>(s_codes);

    // NSB consecutive super-blocks per workgroup: the loads of the next one are
    // issued before the reconstruction of the current one is stored.  (The LDS
    // arrays are rewritten only after the next iteration's first barrier, which
    // every reader of the current values has passed.)
#pragma unroll
    for (int isb = 0; isb < NSB; ++isb) {
    const int64_t sb = (int64_t)blockIdx.x * NSB + isb;

    // Block absmax bits (raw: Inf / NaN included); lane lrow (< J) of each row
    // keeps the maximum of block j = lrow of that row.  The wave's non-finite
    // marker picks the finite-only recomputation.
    uint32_t nf = 0, my_am = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        uint32_t m = max(max(abs_bits(v[j].x), abs_bits(v[j].y)), max(abs_bits(v[j].z), abs_bits(v[j].w)));
        nf = max(nf, m);
        m = row16_max_u(m);
        my_am = (lrow == j) ? m : my_am;
    }
    const bool wave_nf = __any(nf >= 0x7F800000u);
    if (wave_nf) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            uint32_t m = max(max(finite_abs_bits(v[j].x), finite_abs_bits(v[j].y)),
                             max(finite_abs_bits(v[j].z), finite_abs_bits(v[j].w)));
            m = row16_max_u(m);
            my_am = (lrow == j) ? m : my_am;
        }
    }
    const float my_s = as_f(my_am) / 7.0f;  // lanes lrow >= J hold 0 (neutral below)
    const float my_y = 1.0f / (my_s == 0.0f ? 1.0f : my_s);
    const bool all_fast = __all(lrow >= J || fast_divisor(my_s)) && !wave_nf;

    uint32_t pc[J];  // packed codes of each float4 (16 bits)
    uint16_t* pk = reinterpret_cast<uint16_t*>(packed + sb * (kSuperElems / 2));
    if (all_fast) {
        StaticFor<0, J>::run([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const float s = row_bcast_f<j>(my_s);
            const float y = row_bcast_f<j>(my_y);
            const float f0 = __builtin_amdgcn_fmed3f(quick_div(v[j].x, s, y), -7.0f, 7.0f) + kMagic;
            const float f1 = __builtin_amdgcn_fmed3f(quick_div(v[j].y, s, y), -7.0f, 7.0f) + kMagic;
            const float f2 = __builtin_amdgcn_fmed3f(quick_div(v[j].z, s, y), -7.0f, 7.0f) + kMagic;
            const float f3 = __builtin_amdgcn_fmed3f(quick_div(v[j].w, s, y), -7.0f, 7.0f) + kMagic;
            const uint32_t w = nib_pair(f0, f1) | (nib_pair(f2, f3) << 8);
            if constexpr (kCodesLds) s_pk[j * TPB + t] = (uint16_t)w;
            else st_u16(pk + j * TPB + t, (uint16_t)w);
            pc[j] = w;
        });
    } else {
        StaticFor<0, J>::run([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const float s = row_bcast_f<j>(my_s);
            const float y = row_bcast_f<j>(my_y);
            const bool fast = fast_divisor(s);
            const uint32_t w = nib2(q4_general(v[j].x, s, y, fast), q4_general(v[j].y, s, y, fast)) |
                               (nib2(q4_general(v[j].z, s, y, fast), q4_general(v[j].w, s, y, fast)) << 8);
            if constexpr (kCodesLds) s_pk[j * TPB + t] = (uint16_t)w;
            else st_u16(pk + j * TPB + t, (uint16_t)w);
            pc[j] = w;
        });
    }

    // super-scale: max over the 256 block scales, floored at 1e-8
    const float wmax = wave_max_f(my_s);
    if ((t & 63) == 0) s_max[t >> 6] = wmax;
    if (flags && (t & 63) == 0 && wave_nf) atomicOr(flags, FQ_FLAG_NONFINITE);
    if (lrow < J) s_scale[lrow * RW + (t >> 4)] = my_s;  // block (j = lrow, this row)
    __syncthreads();
    float S = s_max[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) S = fmaxf(S, s_max[i]);
    S = fmaxf(S, 1e-8f);
    if (t == 0) super_scale[sb] = S;
    if (t < kGroup) {
        if (block_scale) block_scale[sb * kGroup + t] = s_scale[t];
        // u8 scale codes: thread t encodes block t, four per word
        uint32_t u = u8_scale(s_scale[t], S);
        uint32_t u1 = __shfl_down(u, 1), u2 = __shfl_down(u, 2), u3 = __shfl_down(u, 3);
        if ((t & 3) == 0) s_u8[t >> 2] = u | (u1 << 8) | (u2 << 16) | (u3 << 24);
    }
    const float my_sh = recon_scale(u8_scale(my_s, S), S);
    if constexpr (kCodesLds) {
        // the LDS codes were written before the barrier above; the next
        // super-block's codes are written only after the barrier below
        if (t < kSuperElems / 32) {
            const uint4 c = s_codes[t];
            typedef uint32_t u4v __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(u4v{c.x, c.y, c.z, c.w}, reinterpret_cast<u4v*>(pk) + t);
        }
    }
    __syncthreads();
    if (t < kGroup / 4) st_u32(reinterpret_cast<uint32_t*>(qscale + sb * kGroup) + t, s_u8[t]);
    if (isb + 1 < NSB) load_sb(x + (sb + 1) * kSuperElems);
    if (recon) {
        float4* rv = reinterpret_cast<float4*>(recon + sb * kSuperElems);
        StaticFor<0, J>::run([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const float sh = row_bcast_f<j>(my_sh);
            const uint32_t w = pc[j];
            const float c0 = (float)(int)__builtin_amdgcn_sbfe((int)w, 4, 4);
            const float c1 = (float)(int)__builtin_amdgcn_sbfe((int)w, 0, 4);
            const float c2 = (float)(int)__builtin_amdgcn_sbfe((int)w, 12, 4);
            const float c3 = (float)(int)__builtin_amdgcn_sbfe((int)w, 8, 4);
            const float4 o = make_float4(c0 * sh, c1 * sh, c2 * sh, c3 * sh);
            if constexpr (kStCp < 0) store_nt(rv + j * TPB + t, o);
            else buf_store16<kStCp>(rv, (uint32_t)(j * TPB + t) * 16u, o);
        });
    }
    }  // super-blocks of this workgroup
}

// Any super-block (partial, unaligned): element-wise, one thread per element
// slot, same block structure (4 elements per lane, 16 lanes per block).
__global__ __launch_bounds__(kB) void k_q4dq_any(const float* __restrict__ x, int64_t n, int64_t sb0,
                                                 uint8_t* __restrict__ packed, uint8_t* __restrict__ qscale,
                                                 float* __restrict__ super_scale,
                                                 float* __restrict__ block_scale,
                                                 float* __restrict__ recon, uint32_t* __restrict__ flags) {
    const int64_t sb = sb0 + blockIdx.x;
    const int t = threadIdx.x;
    const int64_t base = sb * kSuperElems;
    __shared__ float s_scale[kGroup];
    __shared__ float s_max[kWaves];
    float smax = 0.0f;
    uint32_t nf = 0;
    float code[kJ][4];
    float sblk[kJ];
    for (int j = 0; j < kJ; ++j) {
        const int64_t e0 = base + 4 * ((int64_t)j * kB + t);
        float xe[4];
        uint32_t am = 0;
        for (int e = 0; e < 4; ++e) {
            xe[e] = (e0 + e < n) ? x[e0 + e] : 0.0f;
            uint32_t a = as_u(xe[e]) & 0x7FFFFFFFu;
            nf = max(nf, a);
            am = max(am, a < 0x7F800000u ? a : 0u);
        }
        am = row16_max_u(am);
        float s = as_f(am) / 7.0f;
        sblk[j] = s;
        smax = fmaxf(smax, s);
        ExactDiv d(s == 0.0f ? 1.0f : s);
        for (int e = 0; e < 4; ++e) code[j][e] = (s != 0.0f) ? q4_code(d, xe[e]) : 0.0f;
        for (int e = 0; e < 4; e += 2) {
            int64_t i = e0 + e;
            if (i < n) packed[i >> 1] = (uint8_t)nib2((int)code[j][e], (i + 1 < n) ? (int)code[j][e + 1] : 0);
        }
        if ((t & 15) == 0) s_scale[j * 16 + (t >> 4)] = s;
    }
    smax = fmaxf(smax, __shfl_xor(smax, 16));
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    nf = wave_max_u(nf);
    if ((t & 63) == 0) s_max[t >> 6] = smax;
    if (flags && (t & 63) == 0 && nf >= 0x7F800000u) atomicOr(flags, FQ_FLAG_NONFINITE);
    __syncthreads();
    float S = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    S = fmaxf(S, 1e-8f);
    const int64_t nb = (n + kBlockElems - 1) / kBlockElems;
    if (t == 0) super_scale[sb] = S;
    const int64_t b = sb * kGroup + t;
    if (b < nb) {
        qscale[b] = (uint8_t)u8_scale(s_scale[t], S);
        if (block_scale) block_scale[b] = s_scale[t];
    }
    if (!recon) return;
    for (int j = 0; j < kJ; ++j) {
        const int64_t e0 = base + 4 * ((int64_t)j * kB + t);
        float sh = recon_scale(u8_scale(sblk[j], S), S);
        for (int e = 0; e < 4; ++e)
            if (e0 + e < n) recon[e0 + e] = code[j][e] * sh;
    }
}

// [DQ] dequantize_4bit_double, full super-block: thread t reconstructs block t's
// scale into LDS, every packed word is loaded up front, then each float4 is
// decoded with its block's scale.
template <int TPB, int NSB>
__global__ __launch_bounds__(TPB) void k_q4dq_dequant_full(const uint8_t* __restrict__ packed,
                                                           const uint8_t* __restrict__ qscale,
                                                           const float* __restrict__ super_scale,
                                                           float* __restrict__ out) {
    constexpr int J = kSuperElems / (4 * TPB);
    constexpr int RW = TPB / 16;
    const int t = threadIdx.x;
    __shared__ float s_sh[kGroup];
    uint32_t w[J];
    {
        const uint16_t* pk = reinterpret_cast<const uint16_t*>(packed + (int64_t)blockIdx.x * NSB * (kSuperElems / 2));
#pragma unroll
        for (int j = 0; j < J; ++j) w[j] = pk[j * TPB + t];
    }
    // NSB consecutive super-blocks per workgroup; the codes of the next one are
    // loaded before the current one is stored.
#pragma unroll
    for (int isb = 0; isb < NSB; ++isb) {
        const int64_t sb = (int64_t)blockIdx.x * NSB + isb;
        if (isb > 0) __syncthreads();  // every thread is done reading s_sh of the previous super-block
        if (t < kGroup) s_sh[t] = recon_scale(qscale[sb * kGroup + t], super_scale[sb]);
        __syncthreads();
        uint32_t wc[J];
#pragma unroll
        for (int j = 0; j < J; ++j) wc[j] = w[j];
        if (isb + 1 < NSB) {
            const uint16_t* pn = reinterpret_cast<const uint16_t*>(packed + (sb + 1) * (kSuperElems / 2));
#pragma unroll
            for (int j = 0; j < J; ++j) w[j] = pn[j * TPB + t];
        }
        float4* o = reinterpret_cast<float4*>(out + sb * kSuperElems);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const float sh = s_sh[j * RW + (t >> 4)];
            const float c0 = (float)(int)__builtin_amdgcn_sbfe((int)wc[j], 4, 4);
            const float c1 = (float)(int)__builtin_amdgcn_sbfe((int)wc[j], 0, 4);
            const float c2 = (float)(int)__builtin_amdgcn_sbfe((int)wc[j], 12, 4);
            const float c3 = (float)(int)__builtin_amdgcn_sbfe((int)wc[j], 8, 4);
            const float4 r = make_float4(c0 * sh, c1 * sh, c2 * sh, c3 * sh);
            if constexpr (kDqStCp < 0) store_nt(o + j * TPB + t, r);
            else buf_store16<kDqStCp>(o, (uint32_t)(j * TPB + t) * 16u, r);
        }
    }
}

// [DQ] dequantize_4bit_double, any super-block (partial or unaligned).
__global__ __launch_bounds__(kB) void k_q4dq_dequant_any(const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ qscale,
                                                         const float* __restrict__ super_scale, int64_t n,
                                                         int64_t sb0, float* __restrict__ out) {
    const int64_t sb = sb0 + blockIdx.x;
    const int t = threadIdx.x;
    const float S = super_scale[sb];
    const int64_t base = sb * kSuperElems;
    const int64_t nb = (n + kBlockElems - 1) / kBlockElems;
    for (int j = 0; j < kJ; ++j) {
        const int64_t b = sb * kGroup + j * 16 + (t >> 4);
        if (b >= nb) continue;
        const float sh = recon_scale(qscale[b], S);
        const int64_t e0 = base + 4 * ((int64_t)j * kB + t);
        for (int e = 0; e < 4; ++e) {
            int64_t i = e0 + e;
            if (i >= n) break;
            uint32_t byte = packed[i >> 1];
            uint32_t nib = (i & 1) ? (byte & 0xFu) : (byte >> 4);
            out[i] = (float)(((int)(nib << 28)) >> 28) * sh;
        }
    }
}

}  // namespace

extern "C" {

int fq_q4dq_quantize(const float* x, int64_t n, uint8_t* packed, uint8_t* qscale,
                     float* super_scale, float* block_scale, float* recon, uint32_t* flags,
                     hipStream_t stream) {
    if (!x || n < 1 || !packed || !qscale || !super_scale) return FQ_E_INVALID;
    if (!fqh::aligned(x, 4) || !fqh::aligned(super_scale, 4) || !fqh::aligned(block_scale, 4) ||
        !fqh::aligned(recon, 4) || !fqh::aligned(flags, 4))
        return FQ_E_INVALID;
    const int64_t nsb = (n + kSuperElems - 1) / kSuperElems;
    const int64_t nfull = n / kSuperElems;
    if (nsb > 0x7FFFFFFF) return FQ_E_INVALID;
    const bool al = fqh::aligned(x, 16) && fqh::aligned(packed, kCodesLds ? 16 : 2) && fqh::aligned(qscale, 4) &&
                    fqh::aligned(recon, 16);
    int64_t done = 0;
    if (al && nfull > 0) {
        const size_t lds = fqh::lds_cap(kOccQuant, kQuantLds);
        const int64_t pairs = kQuantNsb > 1 ? nfull / kQuantNsb : 0;
        if (pairs > 0)
            k_q4dq_full<kQ4Threads, kQuantNsb><<<(unsigned)pairs, kQ4Threads, lds, stream>>>(
                x, packed, qscale, super_scale, block_scale, recon, flags);
        done = pairs * kQuantNsb;
        if (done < nfull)
            k_q4dq_full<kQ4Threads, 1><<<(unsigned)(nfull - done), kQ4Threads, lds, stream>>>(
                x + done * kSuperElems, packed + done * (kSuperElems / 2), qscale + done * kGroup,
                super_scale + done, block_scale ? block_scale + done * kGroup : nullptr,
                recon ? recon + done * kSuperElems : nullptr, flags);
        done = nfull;
    }
    if (done < nsb)
        k_q4dq_any<<<(unsigned)(nsb - done), kB, 0, stream>>>(x, n, done, packed, qscale, super_scale,
                                                             block_scale, recon, flags);
    return fqh::launched();
}

int fq_q4dq_dequantize(const uint8_t* packed, const uint8_t* qscale, const float* super_scale,
                       int64_t n, float* out, hipStream_t stream) {
    if (!packed || !qscale || !super_scale || n < 1 || !out) return FQ_E_INVALID;
    if (!fqh::aligned(super_scale, 4) || !fqh::aligned(out, 4)) return FQ_E_INVALID;
    const int64_t nsb = (n + kSuperElems - 1) / kSuperElems;
    const int64_t nfull = n / kSuperElems;
    if (nsb > 0x7FFFFFFF) return FQ_E_INVALID;
    const bool al = fqh::aligned(packed, 2) && fqh::aligned(out, 16);
    int64_t done = 0;
    if (al && nfull > 0) {
        const size_t lds = fqh::lds_cap(kOccDequant, kDequantLds);
        const int64_t groups = kDequantNsb > 1 ? nfull / kDequantNsb : 0;
        if (groups > 0)
            k_q4dq_dequant_full<kQ4Threads, kDequantNsb><<<(unsigned)groups, kQ4Threads, lds, stream>>>(
                packed, qscale, super_scale, out);
        done = groups * kDequantNsb;
        if (done < nfull)
            k_q4dq_dequant_full<kQ4Threads, 1><<<(unsigned)(nfull - done), kQ4Threads, lds, stream>>>(
                packed + done * (kSuperElems / 2), qscale + done * kGroup, super_scale + done,
                out + done * kSuperElems);
        done = nfull;
    }
    if (done < nsb)
        k_q4dq_dequant_any<<<(unsigned)(nsb - done), kB, 0, stream>>>(packed, qscale, super_scale, n, done, out);
    return fqh::launched();
}

}  // extern "C"
