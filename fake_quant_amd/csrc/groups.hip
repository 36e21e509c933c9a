// groups.hip -- group-wise calibration and integer quantization along rows.
//
// [CS] CS349E 05_quantization_basics.py, demo 3 "granularity": groups of
// `group` consecutive elements along the last dimension of each row, one scale
// per group.  Each group is calibrated and quantized as a channel of [QAT]
// optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware Training
// (QAT) primitives" (per_channel_params: finite min / max, from_minmax; then
// quantize / dequantize).  A row's last group keeps the elements left when
// `group` does not divide the row (the page's quantize_int body is not shown).
//
// Three paths, chosen on the host:
//   * group divides the row, is 1..64 vectors of four elements (a power of two;
//     a vector is one 16-byte fp32 load or one 8-byte bf16 load, so each lane's
//     fake-quant output is one contiguous 16-byte store) and the buffers are
//     aligned: k_groups, one vector per lane over the flattened tensor, a group
//     = a run of L lanes reduced with DPP (and cross-row shuffles for L >= 32);
//     every lane of the group derives the same parameters and quantizes its own
//     vector;
//   * group divides the row otherwise (and the 4-bit codes of a group fill whole
//     bytes): the groups are the rows of the [rows * cols / group, group]
//     reshape, so the per-row path quantizes them, bit for bit the same;
//   * anything else (a ragged last group, an odd group with 4-bit codes):
//     k_groups_any, one thread per group (or per row when two groups share a
//     code byte), two passes over the group.
#include <type_traits>

#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;

constexpr int kN = 4;  // elements per lane on the register path

// min / max / max |x| bits over the L lanes of each group (L a power of two, a
// group a run of L lanes starting at a multiple of L), the result in every lane
template <int L>
__device__ __forceinline__ void group_reduce(MinMax& m) {
    auto step_dpp = [&](auto ctrl) {
        constexpr int C = decltype(ctrl)::value;
        m.mn = fminf(m.mn, dpp_f<C>(m.mn));
        m.mx = fmaxf(m.mx, dpp_f<C>(m.mx));
        m.nf = max(m.nf, dpp_u<C>(m.nf));
    };
    auto step_xor = [&](int mask) {
        m.mn = fminf(m.mn, __shfl_xor(m.mn, mask));
        m.mx = fmaxf(m.mx, __shfl_xor(m.mx, mask));
        m.nf = max(m.nf, (uint32_t)__shfl_xor((int)m.nf, mask));
    };
    if constexpr (L >= 2) step_dpp(std::integral_constant<int, kQuadXor1>{});
    if constexpr (L >= 4) step_dpp(std::integral_constant<int, kQuadXor2>{});
    if constexpr (L >= 8) step_dpp(std::integral_constant<int, kHalfMirror>{});
    if constexpr (L >= 16) step_dpp(std::integral_constant<int, kMirror>{});
    if constexpr (L >= 32) step_xor(16);
    if constexpr (L >= 64) step_xor(32);
}

template <int DT>
__device__ __forceinline__ void load_vec(const void* __restrict__ x, int64_t v, float (&e)[kN]) {
    if constexpr (DT == FQ_F32) {
        const float4 q = reinterpret_cast<const float4*>(x)[v];
        e[0] = q.x;
        e[1] = q.y;
        e[2] = q.z;
        e[3] = q.w;
    } else {
        const uint2 q = reinterpret_cast<const uint2*>(x)[v];
        e[0] = bf16_lo(q.x);
        e[1] = bf16_hi(q.x);
        e[2] = bf16_lo(q.y);
        e[3] = bf16_hi(q.y);
    }
}

// Every lane of the grid takes part in the group reductions (lanes past the end
// hold no element), so no lane returns before them.
template <int DT, int BITS, int L>
__global__ __launch_bounds__(kB) void k_groups(const void* __restrict__ x, int64_t nvec, int affine,
                                               uint8_t* __restrict__ codes, float* __restrict__ fq,
                                               float* __restrict__ scale, int32_t* __restrict__ zp,
                                               uint32_t* __restrict__ flags) {
    constexpr int N = kN;
    const int64_t v = (int64_t)blockIdx.x * kB + threadIdx.x;
    const bool in = v < nvec;
    float e[N];
    MinMax m;
    if (in) {
        load_vec<DT>(x, v, e);
#pragma unroll
        for (int i = 0; i < N; ++i) m.add(e[i]);
    }
    group_reduce<L>(m);
    const IntRange rg = int_range(BITS, affine != 0);
    const IntCal cal = calibrate(m.mn, m.mx, rg, affine != 0);
    const bool first = in && (v % L) == 0;
    if (first) {
        scale[v / L] = cal.scale;
        zp[v / L] = cal.zp;
    }
    // one flag update per wave at most
    const uint32_t f = first ? ((m.nonfinite() ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u))
                             : 0u;
    const uint32_t fw = (__ballot(f & FQ_FLAG_NONFINITE) ? FQ_FLAG_NONFINITE : 0u) |
                        (__ballot(f & FQ_FLAG_DEGENERATE) ? FQ_FLAG_DEGENERATE : 0u);
    if (flags && fw && (threadIdx.x % kWave) == 0) atomicOr(flags, fw);
    if (!in) return;
    const IntQ q(cal.scale, cal.zp, rg);
    float o[N];
    int code[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        o[i] = q.offset(e[i]);
        code[i] = (int)o[i] + cal.zp;
    }
    if (codes) {
        if (BITS == 8) reinterpret_cast<uint32_t*>(codes)[v] = pack4(code[0], code[1], code[2], code[3]);
        else reinterpret_cast<uint16_t*>(codes)[v] = (uint16_t)(nib2(code[0], code[1]) | (nib2(code[2], code[3]) << 8));
    }
    if (fq)
        store_nt(reinterpret_cast<float4*>(fq) + v,
                 make_float4(o[0] * cal.scale, o[1] * cal.scale, o[2] * cal.scale, o[3] * cal.scale));
}

// Wide path: sixteen consecutive elements per lane (the wide layout), so the
// per-group work (reduction, calibration, reciprocal) is shared by four times as
// many elements.
constexpr int kW = kWide;

template <int DT, int BITS, int L>
__global__ __launch_bounds__(kB) void k_groups_wide(const void* __restrict__ x, int64_t nvec, int affine,
                                                    uint8_t* __restrict__ codes, float* __restrict__ fq,
                                                    float* __restrict__ scale, int32_t* __restrict__ zp,
                                                    uint32_t* __restrict__ flags) {
    __shared__ float4 s_out[kB / kWave][kWave * kWidePad / 4];
    const int64_t v = (int64_t)blockIdx.x * kB + threadIdx.x;
    const bool in = v < nvec;
    float e[kW];
    MinMax m;
    if (in) {
        load16<DT == FQ_BF16>(x, v, e);
#pragma unroll
        for (int i = 0; i < kW; ++i) m.add(e[i]);
    } else {
#pragma unroll
        for (int i = 0; i < kW; ++i) e[i] = 0.0f;
    }
    group_reduce<L>(m);
    const IntRange rg = int_range(BITS, affine != 0);
    const IntCal cal = calibrate(m.mn, m.mx, rg, affine != 0);
    const bool first = in && (v % L) == 0;
    if (first) {
        scale[v / L] = cal.scale;
        zp[v / L] = cal.zp;
    }
    const uint32_t f = first ? ((m.nonfinite() ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u))
                             : 0u;
    const uint32_t fw = (__ballot(f & FQ_FLAG_NONFINITE) ? FQ_FLAG_NONFINITE : 0u) |
                        (__ballot(f & FQ_FLAG_DEGENERATE) ? FQ_FLAG_DEGENERATE : 0u);
    if (flags && fw && (threadIdx.x % kWave) == 0) atomicOr(flags, fw);
    const IntQ q(cal.scale, cal.zp, rg);
    float o[kW];
    int code[kW];
#pragma unroll
    for (int i = 0; i < kW; ++i) {
        o[i] = q.offset(e[i]);
        code[i] = (int)o[i] + cal.zp;
    }
    if (in && codes) {
        if (BITS == 8) {
            reinterpret_cast<uint4*>(codes)[v] =
                make_uint4(pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7]),
                           pack4(code[8], code[9], code[10], code[11]), pack4(code[12], code[13], code[14], code[15]));
        } else {
            uint32_t w[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                w[h] = nib2(code[8 * h], code[8 * h + 1]) | (nib2(code[8 * h + 2], code[8 * h + 3]) << 8) |
                       (nib2(code[8 * h + 4], code[8 * h + 5]) << 16) | (nib2(code[8 * h + 6], code[8 * h + 7]) << 24);
            reinterpret_cast<uint2*>(codes)[v] = make_uint2(w[0], w[1]);
        }
    }
    if (fq) {  // uniform: every thread of the block reaches the barrier
#pragma unroll
        for (int i = 0; i < kW; ++i) o[i] *= cal.scale;
        store16_staged(reinterpret_cast<float4*>(fq), v, nvec, o, s_out[threadIdx.x / kWave]);
    }
}

// Groups [g0, g1) of row r, in order: calibrate, store the parameters, quantize.
// 4-bit codes go out a byte at a time (the high nibble held until its partner),
// so a caller that owns whole bytes owns every nibble it writes.
template <int DT, int BITS>
__device__ void quant_groups_of_row(const void* __restrict__ x, int64_t r, int64_t cols, int64_t group, int64_t g0,
                                    int64_t g1, bool affine, uint8_t* __restrict__ codes, float* __restrict__ fq,
                                    float* __restrict__ scale, int32_t* __restrict__ zp, uint32_t& fl) {
    const IntRange rg = int_range(BITS, affine);
    const int64_t ng = (cols + group - 1) / group;
    const int64_t pstride = (cols + 1) / 2;
    uint32_t hold = 0;
    for (int64_t g = g0; g < g1; ++g) {
        const int64_t c0 = g * group;
        const int64_t c1 = c0 + group < cols ? c0 + group : cols;
        MinMax m;
        for (int64_t c = c0; c < c1; ++c) m.add(load_elem<DT == FQ_BF16>(x, r * cols + c));
        const IntCal cal = calibrate(m.mn, m.mx, rg, affine);
        scale[r * ng + g] = cal.scale;
        zp[r * ng + g] = cal.zp;
        fl |= (m.nonfinite() ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
        const IntQ q(cal.scale, cal.zp, rg);
        for (int64_t c = c0; c < c1; ++c) {
            const float o = q.offset(load_elem<DT == FQ_BF16>(x, r * cols + c));
            const int code = (int)o + cal.zp;
            if (fq) fq[r * cols + c] = o * cal.scale;
            if (!codes) continue;
            if (BITS == 8) {
                codes[r * cols + c] = (uint8_t)code;
            } else if ((c & 1) == 0) {
                hold = ((uint32_t)code & 0xFu) << 4;
                if (c == cols - 1) codes[r * pstride + c / 2] = (uint8_t)hold;
            } else {
                codes[r * pstride + c / 2] = (uint8_t)(hold | ((uint32_t)code & 0xFu));
            }
        }
    }
}

// per_row = false: thread i takes group i of the [rows, ceil(cols / group)]
// grid (each group starts on a byte of the codes); per_row = true: thread i takes
// row i.  One flag update per wave at most.
template <int DT, int BITS>
__global__ __launch_bounds__(kB) void k_groups_any(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                   int64_t group, int affine, bool per_row,
                                                   uint8_t* __restrict__ codes, float* __restrict__ fq,
                                                   float* __restrict__ scale, int32_t* __restrict__ zp,
                                                   uint32_t* __restrict__ flags) {
    const int64_t ng = (cols + group - 1) / group;
    const int64_t items = per_row ? rows : rows * ng;
    uint32_t fl = 0;
    for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < items; i += (int64_t)gridDim.x * kB) {
        if (per_row) quant_groups_of_row<DT, BITS>(x, i, cols, group, 0, ng, affine != 0, codes, fq, scale, zp, fl);
        else quant_groups_of_row<DT, BITS>(x, i / ng, cols, group, i % ng, i % ng + 1, affine != 0, codes, fq, scale,
                                           zp, fl);
    }
    const uint32_t fw = (__ballot(fl & FQ_FLAG_NONFINITE) ? FQ_FLAG_NONFINITE : 0u) |
                        (__ballot(fl & FQ_FLAG_DEGENERATE) ? FQ_FLAG_DEGENERATE : 0u);
    if (flags && fw && (threadIdx.x % kWave) == 0) atomicOr(flags, fw);
}

template <int DT, int BITS, int L>
void launch_fast(const void* x, int64_t nvec, int affine, uint8_t* codes, float* fq, float* scale, int32_t* zp,
                 uint32_t* flags, hipStream_t st) {
    const unsigned G = (unsigned)((nvec + kB - 1) / kB);
    k_groups<DT, BITS, L><<<G, kB, 0, st>>>(x, nvec, affine, codes, fq, scale, zp, flags);
}

template <int DT, int BITS>
bool try_fast(const void* x, int64_t nvec, int64_t lanes, int affine, uint8_t* codes, float* fq, float* scale,
              int32_t* zp, uint32_t* flags, hipStream_t st) {
    switch (lanes) {
        case 1: launch_fast<DT, BITS, 1>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 2: launch_fast<DT, BITS, 2>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 4: launch_fast<DT, BITS, 4>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 8: launch_fast<DT, BITS, 8>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 16: launch_fast<DT, BITS, 16>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 32: launch_fast<DT, BITS, 32>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 64: launch_fast<DT, BITS, 64>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        default: return false;
    }
}

template <int DT, int BITS, int L>
void launch_wide(const void* x, int64_t nvec, int affine, uint8_t* codes, float* fq, float* scale, int32_t* zp,
                 uint32_t* flags, hipStream_t st) {
    const unsigned G = (unsigned)((nvec + kB - 1) / kB);
    k_groups_wide<DT, BITS, L><<<G, kB, 0, st>>>(x, nvec, affine, codes, fq, scale, zp, flags);
}

template <int DT, int BITS>
bool try_wide(const void* x, int64_t nvec, int64_t lanes, int affine, uint8_t* codes, float* fq, float* scale,
              int32_t* zp, uint32_t* flags, hipStream_t st) {
    switch (lanes) {
        case 1: launch_wide<DT, BITS, 1>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 2: launch_wide<DT, BITS, 2>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 4: launch_wide<DT, BITS, 4>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 8: launch_wide<DT, BITS, 8>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 16: launch_wide<DT, BITS, 16>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 32: launch_wide<DT, BITS, 32>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        case 64: launch_wide<DT, BITS, 64>(x, nvec, affine, codes, fq, scale, zp, flags, st); return true;
        default: return false;
    }
}

template <int DT, int BITS>
int launch_groups(const void* x, int64_t rows, int64_t cols, int64_t group, int scheme, uint8_t* codes, float* fq,
                  float* scale, int32_t* zp, uint32_t* flags, hipStream_t st) {
    constexpr int N = kN;
    const int affine = scheme == FQ_AFFINE ? 1 : 0;
    if (cols % group == 0) {
        const bool al_wide = fqh::aligned(x, 16) && fqh::aligned(fq, 16) && fqh::aligned(codes, BITS == 8 ? 16 : 8);
        if (group % kW == 0 && al_wide) {
            const int64_t nvec = rows * (cols / kW);
            if (nvec / 0x7FFFFFFFLL < kB && try_wide<DT, BITS>(x, nvec, group / kW, affine, codes, fq, scale, zp,
                                                                 flags, st))
                return fqh::launched();
        }
        const bool al = fqh::aligned(x, DT == FQ_F32 ? 16 : 8) && fqh::aligned(fq, 16) &&
                        fqh::aligned(codes, BITS == 8 ? 4 : 2);
        if (group % N == 0 && al) {
            const int64_t nvec = rows * (cols / N);
            if (nvec / 0x7FFFFFFFLL < kB && try_fast<DT, BITS>(x, nvec, group / N, affine, codes, fq, scale, zp,
                                                                 flags, st))
                return fqh::launched();
        }
        // the groups are the rows of the [rows * cols / group, group] reshape
        if (BITS == 8 || group % 2 == 0)
            return fq_quant_rows(x, DT, rows * (cols / group), group, BITS, scheme, codes, fq, scale, zp, flags, st);
    }
    // two groups share a code byte only for 4-bit codes and an odd group
    const bool per_row = BITS == 4 && (group % 2) == 1;
    const int64_t items = per_row ? rows : rows * ((cols + group - 1) / group);
    const unsigned G = fqh::grid_for(items, kB, 4);
    k_groups_any<DT, BITS><<<G, kB, 0, st>>>(x, rows, cols, group, affine, per_row, codes, fq, scale, zp, flags);
    return fqh::launched();
}

}  // namespace

extern "C" {

int fq_quant_groups(const void* x, int dtype, int64_t rows, int64_t cols, int64_t group, int bits, int scheme,
                    void* codes, float* fq, float* scale, int32_t* zero_point, uint32_t* flags, hipStream_t stream) {
    if (!fqh::valid_dtype(dtype) || !fqh::valid_bits(bits) || !fqh::valid_scheme(scheme)) return FQ_E_UNSUPPORTED;
    if (!x || rows < 1 || cols < 1 || group < 1 || !scale || !zero_point) return FQ_E_INVALID;
    if (!fqh::aligned(x, dtype == FQ_F32 ? 4 : 2) || !fqh::aligned(fq, 4) || !fqh::aligned(scale, 4) ||
        !fqh::aligned(zero_point, 4) || !fqh::aligned(flags, 4))
        return FQ_E_INVALID;
    uint8_t* cd = (uint8_t*)codes;
    if (dtype == FQ_F32) {
        if (bits == 8) return launch_groups<FQ_F32, 8>(x, rows, cols, group, scheme, cd, fq, scale, zero_point, flags, stream);
        return launch_groups<FQ_F32, 4>(x, rows, cols, group, scheme, cd, fq, scale, zero_point, flags, stream);
    }
    if (bits == 8) return launch_groups<FQ_BF16, 8>(x, rows, cols, group, scheme, cd, fq, scale, zero_point, flags, stream);
    return launch_groups<FQ_BF16, 4>(x, rows, cols, group, scheme, cd, fq, scale, zero_point, flags, stream);
}

}  // extern "C"
