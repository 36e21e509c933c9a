// cols.hip -- per-column (axis 1) calibration and integer quantization of a
// row-major [rows, cols] tensor.
//
// [QAT] optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
// Training (QAT) primitives": per_channel_params and fake_quant_int_per_channel
// with axis = 1 (each column is a channel, calibrated on that column only).
//
// A column's elements are cols apart, so the work is three launches:
//   1. k_cols_partial: thread (column vector, row chunk) folds the finite min /
//      max / max |x| bits of N consecutive columns (N = 4 fp32 or 8 bf16: one
//      16-byte load per row) over its chunk of rows -- every load instruction of
//      a wave reads one contiguous run of a row;
//   2. k_cols_params: one thread per column folds the chunk partials, derives the
//      column's parameters ([QAT] from_minmax) and the reciprocal for the exact
//      quotient;
//   3. k_cols_quant: element-wise quantize with the parameters of each element's
//      column, one vector of N columns of one row per thread (so one thread owns
//      every packed nibble byte it writes).
// Workspace: nrc chunk partials per column (16 bytes each), then one 16-byte
// record per column (scale, reciprocal, zero-point, quotient mode).
#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;
constexpr int64_t kMaxChunks = 64;  // row chunks (partials per column)

int64_t row_chunks(int64_t rows) { return rows < kMaxChunks ? rows : kMaxChunks; }

template <int DT>
struct ColVec {
    static constexpr int N = DT == FQ_F32 ? 4 : 8;
};

// element e of the vector of N columns starting at column c0 of row r
// (aligned: one 16-byte load; otherwise element loads, out-of-range as 0)
template <int DT, bool AL>
__device__ __forceinline__ void load_cols(const void* __restrict__ x, int64_t r, int64_t cols, int64_t c0,
                                          float (&v)[ColVec<DT>::N]) {
    constexpr int N = ColVec<DT>::N;
    if constexpr (AL) {
        if constexpr (DT == FQ_F32) {
            const float4 q = reinterpret_cast<const float4*>(x)[(r * cols + c0) / 4];
            v[0] = q.x;
            v[1] = q.y;
            v[2] = q.z;
            v[3] = q.w;
        } else {
            const uint4 q = reinterpret_cast<const uint4*>(x)[(r * cols + c0) / 8];
            v[0] = bf16_lo(q.x);
            v[1] = bf16_hi(q.x);
            v[2] = bf16_lo(q.y);
            v[3] = bf16_hi(q.y);
            v[4] = bf16_lo(q.z);
            v[5] = bf16_hi(q.z);
            v[6] = bf16_lo(q.w);
            v[7] = bf16_hi(q.w);
        }
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const int64_t c = c0 + e;
            if (c >= cols) {
                v[e] = 0.0f;
            } else if constexpr (DT == FQ_F32) {
                v[e] = reinterpret_cast<const float*>(x)[r * cols + c];
            } else {
                v[e] = as_f((uint32_t)reinterpret_cast<const uint16_t*>(x)[r * cols + c] << 16);
            }
        }
    }
}

template <int DT, bool AL>
__global__ __launch_bounds__(kB) void k_cols_partial(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                     int64_t rows_per_chunk, float4* __restrict__ part) {
    constexpr int N = ColVec<DT>::N;
    const int64_t cv = (int64_t)blockIdx.x * kB + threadIdx.x;
    const int64_t c0 = cv * N;
    if (c0 >= cols) return;
    const int64_t chunk = blockIdx.y;
    const int64_t r0 = chunk * rows_per_chunk;
    const int64_t r1 = r0 + rows_per_chunk < rows ? r0 + rows_per_chunk : rows;
    MinMax m[N];
    for (int64_t r = r0; r < r1; ++r) {
        float v[N];
        load_cols<DT, AL>(x, r, cols, c0, v);
#pragma unroll
        for (int e = 0; e < N; ++e) m[e].add(v[e]);
    }
#pragma unroll
    for (int e = 0; e < N; ++e)
        if (c0 + e < cols) part[chunk * cols + c0 + e] = make_float4(m[e].mn, m[e].mx, as_f(m[e].nf), 0.0f);
}

template <int BITS>
__global__ __launch_bounds__(kB) void k_cols_params(const float4* __restrict__ part, int64_t nchunks, int64_t cols,
                                                    int affine, float4* __restrict__ cpar, float* __restrict__ scale,
                                                    int32_t* __restrict__ zp, uint32_t* __restrict__ flags) {
    const int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x;
    if (c >= cols) return;
    MinMax m;
    for (int64_t k = 0; k < nchunks; ++k) {
        const float4 p = part[k * cols + c];
        m.merge(p.x, p.y, as_u(p.z));
    }
    const IntRange rg = int_range(BITS, affine != 0);
    const IntCal cal = calibrate(m.mn, m.mx, rg, affine != 0);
    scale[c] = cal.scale;
    zp[c] = cal.zp;
    const float s = cal.scale == 0.0f ? 1.0f : cal.scale;
    const ExactDiv d(s);
    // (scale, reciprocal, zero-point bits, quotient mode: 0 zero scale, 1 exact fast, 2 true division)
    const uint32_t mode = cal.scale == 0.0f ? 0u : (d.fast ? 1u : 2u);
    cpar[c] = make_float4(cal.scale, d.y, as_f((uint32_t)cal.zp), as_f(mode));
    const uint32_t f = (m.nonfinite() ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
    if (flags && f) atomicOr(flags, f);
}

// code offset q - zp of x for one column's record (the per-element rule of
// IntQ::offset: zero scale -> code 0, NaN -> code 0, +-Inf clamp, -0 -> +0)
__device__ __forceinline__ float col_offset(float x, const float4& cp, float lo, float hi) {
    const uint32_t mode = as_u(cp.w);
    const float zpf = (float)(-(int32_t)as_u(cp.z));
    if (mode == 0u) return zpf;
    const float t = mode == 1u ? ExactDiv(cp.x, cp.y).quick(x) : x / cp.x;  // +-Inf / NaN safe
    const float r = fminf(fmaxf(rintf(t), lo), hi) + 0.0f;
    return (t != t) ? zpf : r;
}

template <int DT, int BITS, bool AL>
__global__ __launch_bounds__(kB) void k_cols_quant(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                   int affine, const float4* __restrict__ cpar,
                                                   uint8_t* __restrict__ codes, float* __restrict__ fq) {
    constexpr int N = ColVec<DT>::N;
    const int64_t ncv = (cols + N - 1) / N;
    const int64_t total = rows * ncv;
    const IntRange rg = int_range(BITS, affine != 0);
    const int64_t pstride = BITS == 8 ? cols : (cols + 1) / 2;
    for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < total; i += (int64_t)gridDim.x * kB) {
        const int64_t r = i / ncv, c0 = (i % ncv) * N;
        float v[N];
        load_cols<DT, AL>(x, r, cols, c0, v);
        int code[N];
        float o[N];
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const int64_t c = c0 + e < cols ? c0 + e : cols - 1;
            const float4 cp = cpar[c];
            const int zpv = (int)as_u(cp.z);
            o[e] = col_offset(v[e], cp, (float)(rg.qmin - zpv), (float)(rg.qmax - zpv));
            code[e] = (int)o[e] + zpv;
            o[e] *= cp.x;
        }
        if (AL) {
            if (codes) {
                uint8_t* crow = codes + r * pstride;
                if (BITS == 8) {
                    const uint32_t w0 = pack4(code[0], code[1], code[2], code[3]);
                    if (N == 4) reinterpret_cast<uint32_t*>(crow)[c0 / 4] = w0;
                    else reinterpret_cast<uint2*>(crow)[c0 / 8] = make_uint2(w0, pack4(code[4 % N], code[5 % N], code[6 % N], code[7 % N]));
                } else {
                    const uint32_t b01 = nib2(code[0], code[1]), b23 = nib2(code[2], code[3]);
                    if (N == 4) {
                        reinterpret_cast<uint16_t*>(crow)[c0 / 4] = (uint16_t)(b01 | (b23 << 8));
                    } else {
                        const uint32_t b45 = nib2(code[4 % N], code[5 % N]), b67 = nib2(code[6 % N], code[7 % N]);
                        reinterpret_cast<uint32_t*>(crow)[c0 / 8] = b01 | (b23 << 8) | (b45 << 16) | (b67 << 24);
                    }
                }
            }
            if (fq) {
                float4* fr = reinterpret_cast<float4*>(fq + r * cols + c0);
                store_nt(fr, make_float4(o[0], o[1], o[2], o[3]));
                if (N == 8) store_nt(fr + 1, make_float4(o[4 % N], o[5 % N], o[6 % N], o[7 % N]));
            }
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e) {
                const int64_t c = c0 + e;
                if (c >= cols) break;
                if (fq) fq[r * cols + c] = o[e];
                if (codes && BITS == 8) codes[r * pstride + c] = (uint8_t)code[e];
            }
            if (codes && BITS == 4) {
#pragma unroll
                for (int e = 0; e < N; e += 2) {
                    const int64_t c = c0 + e;
                    if (c >= cols) break;
                    codes[r * pstride + c / 2] = (uint8_t)nib2(code[e], c + 1 < cols ? code[e + 1] : 0);
                }
            }
        }
    }
}

template <int DT, int BITS>
int launch_cols(const void* x, int64_t rows, int64_t cols, int affine, void* ws, uint8_t* codes, float* fq,
                float* scale, int32_t* zp, uint32_t* flags, hipStream_t st) {
    constexpr int N = ColVec<DT>::N;
    const int64_t nrc = row_chunks(rows);
    const int64_t rpc = (rows + nrc - 1) / nrc;
    float4* part = reinterpret_cast<float4*>(ws);
    float4* cpar = part + nrc * cols;
    const size_t code_align = BITS == 8 ? (N == 4 ? 4 : 8) : (N == 4 ? 2 : 4);
    const bool al = (cols % N == 0) && fqh::aligned(x, 16) && fqh::aligned(fq, 16) && fqh::aligned(codes, code_align);
    const int64_t ncv = (cols + N - 1) / N;
    const dim3 g1((unsigned)((ncv + kB - 1) / kB), (unsigned)nrc);
    if (al) k_cols_partial<DT, true><<<g1, kB, 0, st>>>(x, rows, cols, rpc, part);
    else k_cols_partial<DT, false><<<g1, kB, 0, st>>>(x, rows, cols, rpc, part);
    k_cols_params<BITS><<<(unsigned)((cols + kB - 1) / kB), kB, 0, st>>>(part, nrc, cols, affine, cpar, scale, zp,
                                                                        flags);
    const unsigned g3 = fqh::grid_all(rows * ncv, kB);
    if (al) k_cols_quant<DT, BITS, true><<<g3, kB, 0, st>>>(x, rows, cols, affine, cpar, codes, fq);
    else k_cols_quant<DT, BITS, false><<<g3, kB, 0, st>>>(x, rows, cols, affine, cpar, codes, fq);
    return fqh::launched();
}

}  // namespace

extern "C" {

size_t fq_cols_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows < 1 || cols < 1) return 0;
    return (size_t)((row_chunks(rows) + 1) * cols * 16);
}

int fq_quant_cols(const void* x, int dtype, int64_t rows, int64_t cols, int bits, int scheme, void* workspace,
                  size_t workspace_bytes, void* codes, float* fq, float* scale, int32_t* zero_point, uint32_t* flags,
                  hipStream_t stream) {
    if (!fqh::valid_dtype(dtype) || !fqh::valid_bits(bits) || !fqh::valid_scheme(scheme)) return FQ_E_UNSUPPORTED;
    if (!x || rows < 1 || cols < 1 || !workspace || !scale || !zero_point) return FQ_E_INVALID;
    if (workspace_bytes < fq_cols_workspace_bytes(rows, cols) || !fqh::aligned(workspace, 16)) return FQ_E_INVALID;
    if (!fqh::aligned(x, dtype == FQ_F32 ? 4 : 2) || !fqh::aligned(fq, 4) || !fqh::aligned(scale, 4) ||
        !fqh::aligned(zero_point, 4) || !fqh::aligned(flags, 4))
        return FQ_E_INVALID;
    const int aff = scheme == FQ_AFFINE;
    uint8_t* cd = (uint8_t*)codes;
    if (dtype == FQ_F32) {
        if (bits == 8) return launch_cols<FQ_F32, 8>(x, rows, cols, aff, workspace, cd, fq, scale, zero_point, flags, stream);
        return launch_cols<FQ_F32, 4>(x, rows, cols, aff, workspace, cd, fq, scale, zero_point, flags, stream);
    }
    if (bits == 8) return launch_cols<FQ_BF16, 8>(x, rows, cols, aff, workspace, cd, fq, scale, zero_point, flags, stream);
    return launch_cols<FQ_BF16, 4>(x, rows, cols, aff, workspace, cd, fq, scale, zero_point, flags, stream);
}

}  // extern "C"
