// tensor.hip -- per-tensor kernels: the tensor-scope min / max / amax reduction
// with parameter derivation on the device, integer quantize / fake-quant /
// dequantize with one parameter set, and the straight-through-estimator backward.
//
// [QAT] = optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
// Training (QAT) primitives": QuantParams::per_tensor_minmax, fake_quant_int,
// real_min / real_max, fake_quant_backward.
//
// Layout: the element-wise kernels walk the tensor in chunks of four consecutive
// elements (one 16-byte load of x), one chunk per thread over a grid that covers
// the whole tensor (many short workgroups sweeping memory in order stream best on
// MI355X).  The last n % 4 elements (and every chunk when a buffer is not
// vector-aligned) go through the scalar form of the same chunk code.
#include <atomic>

#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;

__device__ __forceinline__ float4 ld4(const float* p, int64_t c) {
    return *reinterpret_cast<const float4*>(p + 4 * c);
}
// the tensor-scope reduction's loads (nontemporal when FQ_NT_LOADS_REDUCE)
__device__ __forceinline__ float4 ld4_reduce(const float* p, int64_t c) {
    return ld_f4<FQ_NT_LOADS_REDUCE != 0>(reinterpret_cast<const float4*>(p + 4 * c));
}
__device__ __forceinline__ void st4(float* p, int64_t c, float4 v) {
    store_nt(reinterpret_cast<float4*>(p + 4 * c), v);
}

// ---------------------------------------------------------------------------
// Tensor-scope reduction, pass 1: one partial per block.
//   MINMAX: (finite min, finite max, max |x| bits) -- int calibration
//   AMAX:   (-, finite amax, -)                     -- fp8 calibration
// A block of kRT threads reduces tiles of 4 * kRT consecutive 16-byte chunks
// (thread t takes chunks t, t + kRT, t + 2 kRT, t + 3 kRT of a tile: four loads in
// flight, each load instruction covering 1 KiB per wave), tiles b, b + G, ... for
// block b of G.
// MINMAX runs unfiltered min / max first (NaN is ignored by them); a thread that
// met a NaN or an infinity redoes its own chunks with the finite filter.
// ---------------------------------------------------------------------------
enum { kMinMax = 0, kAmax = 1 };
constexpr int kRU = fqh::kReduceChunks;
constexpr int kRT = fqh::kReduceThreads;

template <int MODE, bool AL>
__global__ __launch_bounds__(kRT) void k_reduce_partial(const float* __restrict__ x, int64_t n,
                                                       float4* __restrict__ part) {
    const int64_t nfull = n >> 2;
    const int64_t ntiles = (nfull + fqh::kReduceTile - 1) / fqh::kReduceTile;
    const bool tail = blockIdx.x == 0 && threadIdx.x < (n & 3);
    auto ld = [&](int64_t c) -> float4 {
        if (AL) return ld4_reduce(x, c);
        return make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
    };
    float4 r;
    if (MODE == kAmax) {
        uint32_t acc[kRU];
#pragma unroll
        for (int u = 0; u < kRU; ++u) acc[u] = 0;
        for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
            const int64_t c0 = tile * fqh::kReduceTile + threadIdx.x;
            float4 v[kRU];
#pragma unroll
            for (int u = 0; u < kRU; ++u)
                v[u] = (c0 + u * kRT < nfull) ? ld(c0 + u * kRT) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < kRU; ++u)
                acc[u] = max(acc[u], max(max(finite_abs_bits(v[u].x), finite_abs_bits(v[u].y)),
                                         max(finite_abs_bits(v[u].z), finite_abs_bits(v[u].w))));
        }
        if (tail) acc[0] = max(acc[0], finite_abs_bits(x[4 * nfull + threadIdx.x]));
#pragma unroll
        for (int u = 1; u < kRU; ++u) acc[0] = max(acc[0], acc[u]);
        r = make_float4(0.f, as_f(wave_max_u(acc[0])), 0.f, 0.f);
    } else {
        float mn[kRU], mx[kRU];
        bool bad = false;
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
            mn[u] = __builtin_inff();
            mx[u] = -__builtin_inff();
        }
        for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
            const int64_t c0 = tile * fqh::kReduceTile + threadIdx.x;
            float4 v[kRU];
#pragma unroll
            for (int u = 0; u < kRU; ++u)
                v[u] = (c0 + u * kRT < nfull) ? ld(c0 + u * kRT) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < kRU; ++u) {
                if (c0 + u * kRT >= nfull) continue;
                mn[u] = fminf(fminf(mn[u], v[u].x), fminf(v[u].y, fminf(v[u].z, v[u].w)));
                mx[u] = fmaxf(fmaxf(mx[u], v[u].x), fmaxf(v[u].y, fmaxf(v[u].z, v[u].w)));
                bad = bad | (v[u].x != v[u].x) | (v[u].y != v[u].y) | (v[u].z != v[u].z) | (v[u].w != v[u].w);
            }
        }
        MinMax m;
        if (tail) m.add(x[4 * nfull + threadIdx.x]);
#pragma unroll
        for (int u = 0; u < kRU; ++u) m.merge(mn[u], mx[u], 0u);
        if (bad || m.mn == -__builtin_inff() || m.mx == __builtin_inff()) {
            // this thread saw a non-finite value: redo its chunks with the filter
            MinMax f;
            for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
                const int64_t c0 = tile * fqh::kReduceTile + threadIdx.x;
                for (int u = 0; u < kRU; ++u) {
                    if (c0 + u * kRT >= nfull) continue;
                    float4 v = ld(c0 + u * kRT);
                    f.add(v.x);
                    f.add(v.y);
                    f.add(v.z);
                    f.add(v.w);
                }
            }
            if (tail) f.add(x[4 * nfull + threadIdx.x]);
            m = f;
        }
        r = make_float4(wave_min_f(m.mn), wave_max_f(m.mx), as_f(wave_max_u(m.nf)), 0.f);
    }

    __shared__ float4 lds[kRT / kWave];
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    if (lane == 0) lds[w] = r;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kRT / kWave; ++i) {
            float4 o = lds[i];
            if (MODE == kMinMax) {
                r.x = fminf(r.x, o.x);
                r.y = fmaxf(r.y, o.y);
                r.z = as_f(max(as_u(r.z), as_u(o.z)));
            } else {
                r.y = as_f(max(as_u(r.y), as_u(o.y)));
            }
        }
        // amax partials are packed as 4-byte words (pass 2 then reads a quarter of
        // the bytes); min / max partials stay 16-byte records
        if (MODE == kAmax) reinterpret_cast<uint32_t*>(part)[blockIdx.x] = as_u(r.y);
        else part[blockIdx.x] = r;
    }
}

// Pass 2 (one block): fold the partials and derive the integer parameters
// ([QAT] from_minmax, real_min / real_max).
constexpr int kFT = fqh::kFinalThreads;
constexpr int kFW = kFT / kWave;
constexpr int kFinalLoads = (int)(fqh::kMaxReduceBlocks / kFT);  // partials per thread of pass 2
static_assert(fqh::kMaxReduceBlocks % kFT == 0, "pass 2 covers every partial");

__global__ __launch_bounds__(kFT) void k_params_int_final(const float4* __restrict__ part, int nparts,
                                                         int bits, int affine,
                                                         fq_int_params* __restrict__ params,
                                                         uint32_t* __restrict__ flags) {
    // every partial this thread folds is loaded at once (one memory round trip)
    MinMax m;
    float4 p[kFinalLoads];
#pragma unroll
    for (int u = 0; u < kFinalLoads; ++u) {
        const int i = threadIdx.x + u * kFT;
        p[u] = i < nparts ? part[i] : make_float4(__builtin_inff(), -__builtin_inff(), 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kFinalLoads; ++u) m.merge(p[u].x, p[u].y, as_u(p[u].z));
    __shared__ float4 lds[kFW];
    float4 r = make_float4(wave_min_f(m.mn), wave_max_f(m.mx), as_f(wave_max_u(m.nf)), 0.f);
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = r;
    __syncthreads();
    if (threadIdx.x != 0) return;
    for (int i = 1; i < kFW; ++i) m.merge(lds[i].x, lds[i].y, as_u(lds[i].z));
    m.merge(r.x, r.y, as_u(r.z));
    IntRange rg = int_range(bits, affine != 0);
    IntCal cal = calibrate(m.mn, m.mx, rg, affine != 0);
    fq_int_params out;
    out.scale = cal.scale;
    out.zero_point = cal.zp;
    out.real_min = (float)(rg.qmin - cal.zp) * cal.scale;
    out.real_max = (float)(rg.qmax - cal.zp) * cal.scale;
    *params = out;
    uint32_t f = (m.nonfinite() ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
    if (flags && f) atomicOr(flags, f);
}

// Pass 2 for fp8: amax over the finite elements -> scale = amax / max-normal.
__global__ __launch_bounds__(kFT) void k_fp8_scale_final(const uint32_t* __restrict__ part, int nparts,
                                                        float* __restrict__ s_e4m3,
                                                        float* __restrict__ s_e5m2,
                                                        uint32_t* __restrict__ flags) {
    uint32_t p[kFinalLoads];
#pragma unroll
    for (int u = 0; u < kFinalLoads; ++u) {
        const int i = threadIdx.x + u * kFT;
        p[u] = i < nparts ? part[i] : 0u;
    }
    uint32_t a = 0;
#pragma unroll
    for (int u = 0; u < kFinalLoads; ++u) a = max(a, p[u]);
    __shared__ uint32_t lds[kFW];
    a = wave_max_u(a);
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = a;
    __syncthreads();
    if (threadIdx.x != 0) return;
    for (int i = 1; i < kFW; ++i) a = max(a, lds[i]);
    float amax = as_f(a);
    bool zero = false;
    if (s_e4m3) {
        float s = amax / 448.0f;
        *s_e4m3 = s;
        zero |= (s == 0.0f);
    }
    if (s_e5m2) {
        float s = amax / 57344.0f;
        *s_e5m2 = s;
        zero |= (s == 0.0f);
    }
    if (flags && zero) atomicOr(flags, FQ_FLAG_DEGENERATE);
}

// Pass 2 that keeps the finite amax itself: its bits go to word 0 of the
// workspace (every partial has been read by then; this block is their only
// reader).
__global__ __launch_bounds__(kFT) void k_amax_final(uint32_t* __restrict__ part, int nparts) {
    uint32_t p[kFinalLoads];
#pragma unroll
    for (int u = 0; u < kFinalLoads; ++u) {
        const int i = threadIdx.x + u * kFT;
        p[u] = i < nparts ? part[i] : 0u;
    }
    uint32_t a = 0;
#pragma unroll
    for (int u = 0; u < kFinalLoads; ++u) a = max(a, p[u]);
    __shared__ uint32_t lds[kFW];
    a = wave_max_u(a);
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = a;
    __syncthreads();
    if (threadIdx.x != 0) return;
    for (int i = 1; i < kFW; ++i) a = max(a, lds[i]);
    part[0] = a;
}

// ---------------------------------------------------------------------------
// Integer quantize / fake-quant with one parameter set ([QAT] fake_quant_int)
// ---------------------------------------------------------------------------
template <int BITS, int MODE>
struct IntTensorOp {
    IntQ q;
    float scale;
    int zp;
    uint8_t* codes;
    float* fq;

    // scalar form for `cnt` (1..4) elements starting at chunk c
    __device__ void scalar_chunk(const float* x, int64_t c, int cnt) const {
        int code[4] = {0, 0, 0, 0};
        for (int e = 0; e < cnt; ++e) {
            float o = q.template offset_m<MODE>(x[4 * c + e]);
            code[e] = (int)o + zp;
            if (fq) fq[4 * c + e] = o * scale;
            if (codes && BITS == 8) codes[4 * c + e] = (uint8_t)code[e];
        }
        if (codes && BITS == 4) {
            codes[2 * c] = (uint8_t)nib2(code[0], code[1]);
            if (cnt > 2) codes[2 * c + 1] = (uint8_t)nib2(code[2], code[3]);
        }
    }
    __device__ __forceinline__ void vector_chunk(int64_t c, float4 v) const {
        float o0 = q.template offset_m<MODE>(v.x), o1 = q.template offset_m<MODE>(v.y);
        float o2 = q.template offset_m<MODE>(v.z), o3 = q.template offset_m<MODE>(v.w);
        if (codes) {
            int c0 = (int)o0 + zp, c1 = (int)o1 + zp, c2 = (int)o2 + zp, c3 = (int)o3 + zp;
            if (BITS == 8) {
                reinterpret_cast<uint32_t*>(codes)[c] = pack4(c0, c1, c2, c3);
            } else {
                reinterpret_cast<uint16_t*>(codes)[c] = (uint16_t)(nib2(c0, c1) | (nib2(c2, c3) << 8));
            }
        }
        if (fq) st4(fq, c, make_float4(o0 * scale, o1 * scale, o2 * scale, o3 * scale));
    }
};

template <int BITS, int MODE, bool AL>
__device__ __forceinline__ void fq_int_loop(const IntTensorOp<BITS, MODE>& op, const float* __restrict__ x,
                                            int64_t n) {
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x;
    if (AL) {
        for (; c + 3 * stride < nfull; c += 4 * stride) {
            float4 v0 = ld4(x, c), v1 = ld4(x, c + stride);
            float4 v2 = ld4(x, c + 2 * stride), v3 = ld4(x, c + 3 * stride);
            op.vector_chunk(c, v0);
            op.vector_chunk(c + stride, v1);
            op.vector_chunk(c + 2 * stride, v2);
            op.vector_chunk(c + 3 * stride, v3);
        }
        for (; c < nfull; c += stride) op.vector_chunk(c, ld4(x, c));
    } else {
        for (; c < nfull; c += stride) op.scalar_chunk(x, c, 4);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && (n & 3)) op.scalar_chunk(x, nfull, (int)(n & 3));
}

template <int BITS, bool AL>
__global__ __launch_bounds__(kB) void k_fq_int_tensor(const float* __restrict__ x, int64_t n, int affine,
                                                      const fq_int_params* __restrict__ p,
                                                      uint8_t* __restrict__ codes,
                                                      float* __restrict__ fq) {
    const fq_int_params P = *p;
    const IntRange rg = int_range(BITS, affine != 0);
    const IntQ q(P.scale, P.zero_point, rg);
    // one uniform decision per launch: the per-element code then carries no branch
    if (q.zero) {
        fq_int_loop<BITS, 0, AL>(IntTensorOp<BITS, 0>{q, P.scale, P.zero_point, codes, fq}, x, n);
    } else if (q.div.fast) {
        fq_int_loop<BITS, 1, AL>(IntTensorOp<BITS, 1>{q, P.scale, P.zero_point, codes, fq}, x, n);
    } else {
        fq_int_loop<BITS, 2, AL>(IntTensorOp<BITS, 2>{q, P.scale, P.zero_point, codes, fq}, x, n);
    }
}

// ---------------------------------------------------------------------------
// Per-tensor calibration + fake-quant in two launches for small tensors: after
// the reduction's first pass, every block of this kernel folds the (at most
// kFoldMaxParts) partials itself and derives the parameters ([QAT] from_minmax),
// so the one-block parameter pass and its launch drop out.  The fold is
// order-free, so every block derives the same parameters; block 0 stores them.
// Each thread's chunk of x is loaded before the partials, so the two loads
// overlap.  One 16-byte chunk per thread over a grid covering the tensor; the
// n % 4 elements after the last whole chunk go to thread 0 of block 0.
// ---------------------------------------------------------------------------
constexpr int kFoldMaxParts = (int)fqh::kFoldMaxParts;
static_assert(kFoldMaxParts % kB == 0, "whole loads of partials per thread");

template <int BITS>
__global__ __launch_bounds__(kB) void k_fq_int_tensor_fold(const float* __restrict__ x, int64_t n, int affine,
                                                           const float4* __restrict__ part, int nparts,
                                                           fq_int_params* __restrict__ params,
                                                           uint8_t* __restrict__ codes, float* __restrict__ fq,
                                                           uint32_t* __restrict__ flags) {
    const int64_t nfull = n >> 2;
    const int t = threadIdx.x;
    const int64_t c = (int64_t)blockIdx.x * kB + t;
    const float4 v = c < nfull ? ld4(x, c) : make_float4(0.f, 0.f, 0.f, 0.f);
    MinMax m;
#pragma unroll
    for (int k = 0; k < kFoldMaxParts / kB; ++k) {
        const int i = t + k * kB;
        if (i < nparts) {
            const float4 p = part[i];
            m.merge(p.x, p.y, as_u(p.z));
        }
    }
    __shared__ float4 lds[kB / kWave];
    const float4 r = make_float4(wave_min_f(m.mn), wave_max_f(m.mx), as_f(wave_max_u(m.nf)), 0.f);
    if (t % kWave == 0) lds[t / kWave] = r;
    __syncthreads();
    MinMax g;
#pragma unroll
    for (int i = 0; i < kB / kWave; ++i) g.merge(lds[i].x, lds[i].y, as_u(lds[i].z));
    const IntRange rg = int_range(BITS, affine != 0);
    const IntCal cal = calibrate(g.mn, g.mx, rg, affine != 0);
    if (blockIdx.x == 0 && t == 0) {
        fq_int_params out;
        out.scale = cal.scale;
        out.zero_point = cal.zp;
        out.real_min = (float)(rg.qmin - cal.zp) * cal.scale;
        out.real_max = (float)(rg.qmax - cal.zp) * cal.scale;
        *params = out;
        const uint32_t f = (g.nonfinite() ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
        if (flags && f) atomicOr(flags, f);
    }
    const IntQ q(cal.scale, cal.zp, rg);
    auto run = [&](auto op) {
        if (c < nfull) op.vector_chunk(c, v);
        if (blockIdx.x == 0 && t == 0 && (n & 3)) op.scalar_chunk(x, nfull, (int)(n & 3));
    };
    // one uniform decision per launch, as in k_fq_int_tensor
    if (q.zero) run(IntTensorOp<BITS, 0>{q, cal.scale, cal.zp, codes, fq});
    else if (q.div.fast) run(IntTensorOp<BITS, 1>{q, cal.scale, cal.zp, codes, fq});
    else run(IntTensorOp<BITS, 2>{q, cal.scale, cal.zp, codes, fq});
}

// ---------------------------------------------------------------------------
// The same fold ahead of a grid-stride fake-quant: every block first loads its
// first four chunks of x, then folds up to MAXP partials (all of a thread's
// partials loaded in one round, so the two loads overlap), derives the
// parameters (block 0 stores them), then quantizes its share of the tensor four
// chunks at a time.  The grid is capped at a few resident blocks per compute
// unit, so the partials are read from L2 a few thousand times at most.  Serves
// the integer QAT step: its update pass leaves the partials, so the step takes
// two launches instead of three.
// ---------------------------------------------------------------------------
template <int BITS, int MODE>
__device__ __forceinline__ void fq_int_gs_loop(const IntTensorOp<BITS, MODE>& op, const float* __restrict__ x,
                                               int64_t n, int64_t c, int64_t stride, float4 (&v)[4]) {
    const int64_t nfull = n >> 2;
    for (;;) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (c + u * stride < nfull) op.vector_chunk(c + u * stride, v[u]);
        c += 4 * stride;
        if (c >= nfull) break;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (c + u * stride < nfull) v[u] = ld4(x, c + u * stride);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && (n & 3)) op.scalar_chunk(x, nfull, (int)(n & 3));
}

template <int BITS, int MAXP>
__global__ __launch_bounds__(kB) void k_fq_int_tensor_fold_gs(const float* __restrict__ x, int64_t n, int affine,
                                                              const float4* __restrict__ part, int nparts,
                                                              fq_int_params* __restrict__ params,
                                                              uint8_t* __restrict__ codes, float* __restrict__ fq,
                                                              uint32_t* __restrict__ flags) {
    static_assert(MAXP % kB == 0, "whole loads of partials per thread");
    const int t = threadIdx.x;
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    const int64_t c = (int64_t)blockIdx.x * kB + t;
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = c + u * stride < nfull ? ld4(x, c + u * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 p[MAXP / kB];
#pragma unroll
    for (int k = 0; k < MAXP / kB; ++k) {
        const int i = t + k * kB;
        p[k] = i < nparts ? part[i] : make_float4(__builtin_inff(), -__builtin_inff(), 0.f, 0.f);
    }
    MinMax m;
#pragma unroll
    for (int k = 0; k < MAXP / kB; ++k) m.merge(p[k].x, p[k].y, as_u(p[k].z));
    __shared__ float4 lds[kB / kWave];
    const float4 r = make_float4(wave_min_f(m.mn), wave_max_f(m.mx), as_f(wave_max_u(m.nf)), 0.f);
    if (t % kWave == 0) lds[t / kWave] = r;
    __syncthreads();
    MinMax g;
#pragma unroll
    for (int i = 0; i < kB / kWave; ++i) g.merge(lds[i].x, lds[i].y, as_u(lds[i].z));
    const IntRange rg = int_range(BITS, affine != 0);
    const IntCal cal = calibrate(g.mn, g.mx, rg, affine != 0);
    if (blockIdx.x == 0 && t == 0) {
        fq_int_params out;
        out.scale = cal.scale;
        out.zero_point = cal.zp;
        out.real_min = (float)(rg.qmin - cal.zp) * cal.scale;
        out.real_max = (float)(rg.qmax - cal.zp) * cal.scale;
        *params = out;
        const uint32_t f = (g.nonfinite() ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
        if (flags && f) atomicOr(flags, f);
    }
    const IntQ q(cal.scale, cal.zp, rg);
    if (q.zero) fq_int_gs_loop<BITS, 0>(IntTensorOp<BITS, 0>{q, cal.scale, cal.zp, codes, fq}, x, n, c, stride, v);
    else if (q.div.fast) fq_int_gs_loop<BITS, 1>(IntTensorOp<BITS, 1>{q, cal.scale, cal.zp, codes, fq}, x, n, c, stride, v);
    else fq_int_gs_loop<BITS, 2>(IntTensorOp<BITS, 2>{q, cal.scale, cal.zp, codes, fq}, x, n, c, stride, v);
}

// ---------------------------------------------------------------------------
// Integer dequantize ([QAT] dequant(q) = (q - zero_point) * scale)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int sext4(uint32_t nib) { return ((int)(nib << 28)) >> 28; }
__device__ __forceinline__ int sext8(uint32_t b) { return ((int)(b << 24)) >> 24; }

template <int BITS, bool AL>
__global__ __launch_bounds__(kB) void k_dq_int_tensor(const uint8_t* __restrict__ codes, int64_t n,
                                                      const fq_int_params* __restrict__ p,
                                                      float* __restrict__ out) {
    const float s = p->scale;
    const int zp = p->zero_point;
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x;
    auto code_at = [&](int64_t i) -> int {
        if (BITS == 8) return sext8(codes[i]);
        uint32_t byte = codes[i >> 1];
        return sext4((i & 1) ? (byte & 0xFu) : (byte >> 4));
    };
    for (; c < nfull; c += stride) {
        int q0, q1, q2, q3;
        if (AL && BITS == 8) {
            uint32_t w = reinterpret_cast<const uint32_t*>(codes)[c];
            q0 = sext8(w);
            q1 = sext8(w >> 8);
            q2 = sext8(w >> 16);
            q3 = sext8(w >> 24);
        } else if (AL) {
            uint32_t w = reinterpret_cast<const uint16_t*>(codes)[c];
            q0 = sext4((w >> 4) & 0xFu);
            q1 = sext4(w & 0xFu);
            q2 = sext4((w >> 12) & 0xFu);
            q3 = sext4((w >> 8) & 0xFu);
        } else {
            q0 = code_at(4 * c);
            q1 = code_at(4 * c + 1);
            q2 = code_at(4 * c + 2);
            q3 = code_at(4 * c + 3);
        }
        float4 v = make_float4((float)(q0 - zp) * s, (float)(q1 - zp) * s, (float)(q2 - zp) * s,
                               (float)(q3 - zp) * s);
        if (AL) {
            st4(out, c, v);
        } else {
            out[4 * c] = v.x;
            out[4 * c + 1] = v.y;
            out[4 * c + 2] = v.z;
            out[4 * c + 3] = v.w;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        int64_t i = 4 * nfull + threadIdx.x;
        out[i] = (float)(code_at(i) - zp) * s;
    }
}

// ---------------------------------------------------------------------------
// STE backward ([QAT] fake_quant_backward): pass g where lo <= x <= hi.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ste1(float g, float x, float lo, float hi) {
    return (x >= lo && x <= hi) ? g : 0.0f;
}

template <bool AL>
__global__ __launch_bounds__(kB) void k_ste(const float* __restrict__ g, const float* __restrict__ x,
                                            int64_t n, const float* __restrict__ bounds,
                                            float* __restrict__ out) {
    const float b0 = bounds[0], b1 = bounds[1];
    const float lo = b0 <= b1 ? b0 : b1;
    const float hi = b0 <= b1 ? b1 : b0;
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x;
    if (AL) {
        for (; c + 1 * stride < nfull; c += 2 * stride) {
            float4 g0 = ld4(g, c), x0 = ld4(x, c), g1 = ld4(g, c + stride), x1 = ld4(x, c + stride);
            st4(out, c, make_float4(ste1(g0.x, x0.x, lo, hi), ste1(g0.y, x0.y, lo, hi),
                                    ste1(g0.z, x0.z, lo, hi), ste1(g0.w, x0.w, lo, hi)));
            st4(out, c + stride,
                make_float4(ste1(g1.x, x1.x, lo, hi), ste1(g1.y, x1.y, lo, hi),
                            ste1(g1.z, x1.z, lo, hi), ste1(g1.w, x1.w, lo, hi)));
        }
        for (; c < nfull; c += stride) {
            float4 g0 = ld4(g, c), x0 = ld4(x, c);
            st4(out, c, make_float4(ste1(g0.x, x0.x, lo, hi), ste1(g0.y, x0.y, lo, hi),
                                    ste1(g0.z, x0.z, lo, hi), ste1(g0.w, x0.w, lo, hi)));
        }
    } else {
        for (; c < nfull; c += stride)
            for (int e = 0; e < 4; ++e) out[4 * c + e] = ste1(g[4 * c + e], x[4 * c + e], lo, hi);
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        int64_t i = 4 * nfull + threadIdx.x;
        out[i] = ste1(g[i], x[i], lo, hi);
    }
}

// launch the reduction's first pass; returns the number of partials
template <int MODE>
unsigned launch_partial(const float* x, int64_t n, void* ws, hipStream_t st) {
    unsigned G = fqh::reduce_blocks(n);
    // amax: at most one workgroup per CU, each looping over its tiles.  Measured
    // on the 2^26 fp8 scale, cold, interleaved on one box: 44.5-44.6 us with 256
    // workgroups against 45.2-45.6 with 512, 46.1-46.2 with 384, 45.2-46.6 with
    // 1024 and 47.2-47.4 with one workgroup per tile (8192); on another box 44.6-
    // 44.9 against 46.7-47.5 us.  The NVFP4 amax pass gains 2-3 us the same way.
    if (MODE == kAmax) {
        const unsigned cap = (unsigned)fqh::num_cus();
        if (G > cap) G = cap;
    }
    if (fqh::aligned(x, 16))
        k_reduce_partial<MODE, true><<<G, kRT, 0, st>>>(x, n, (float4*)ws);
    else
        k_reduce_partial<MODE, false><<<G, kRT, 0, st>>>(x, n, (float4*)ws);
    return G;
}

}  // namespace

namespace fqh {

int params_from_partials(const void* workspace, unsigned nparts, int bits, int scheme, fq_int_params* params,
                         uint32_t* flags, hipStream_t stream) {
    k_params_int_final<<<1, kFT, 0, stream>>>((const float4*)workspace, (int)nparts, bits,
                                              scheme == FQ_AFFINE ? 1 : 0, params, flags);
    return launched();
}

int fake_quant_from_partials(const float* x, int64_t n, int bits, int scheme, const void* workspace, unsigned nparts,
                             fq_int_params* params, void* codes, float* fq, uint32_t* flags, hipStream_t stream) {
    const bool al = aligned(x, 16) && aligned(fq, 16) && aligned(codes, bits == 8 ? 4 : 2);
    if (!al || nparts > (unsigned)kFoldGsMaxParts) {
        int st = params_from_partials(workspace, nparts, bits, scheme, params, flags, stream);
        if (st != FQ_OK) return st;
        return fq_fake_quant_int_tensor(x, n, bits, scheme, params, codes, fq, stream);
    }
    const unsigned G = grid_for((n + 3) / 4, kBlock, kFoldGsBlocksPerCu);
    const int aff = scheme == FQ_AFFINE;
    const float4* part = (const float4*)workspace;
    uint8_t* cd = (uint8_t*)codes;
    if (bits == 8)
        k_fq_int_tensor_fold_gs<8, kFoldGsMaxParts><<<G, kBlock, 0, stream>>>(x, n, aff, part, (int)nparts, params,
                                                                             cd, fq, flags);
    else
        k_fq_int_tensor_fold_gs<4, kFoldGsMaxParts><<<G, kBlock, 0, stream>>>(x, n, aff, part, (int)nparts, params,
                                                                             cd, fq, flags);
    return launched();
}

int tensor_amax(const float* x, int64_t n, void* workspace, hipStream_t stream) {
    const unsigned G = launch_partial<kAmax>(x, n, workspace, stream);
    k_amax_final<<<1, kFT, 0, stream>>>((uint32_t*)workspace, (int)G);
    return launched();
}

}  // namespace fqh

// ---------------------------------------------------------------------------
// Static device scratch of fq_calibrate_fake_quant_int_tensor_noalloc: the
// reduction partials of one call (one 16-byte record per first-pass block, at
// most kMaxReduceBlocks of them for any n, so every n >= 1 fits).  Each GPU holds
// its own copy of the array from module load until the process ends.  Host code
// never names the array itself: its device address is looked up once per device
// and kept in scratch_addr.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)fqh::kMaxReduceBlocks * sizeof(float4);
static_assert(kScratchBytes == FQ_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
static __device__ __align__(256) float4 scratch[fqh::kMaxReduceBlocks];

namespace {
std::atomic<void*> scratch_addr[fqh::kMaxDevices];

// Device address of `scratch` on the current device, or nullptr when it cannot
// be had (device id beyond the cache, lookup failed).  The lookup is idempotent,
// so threads racing on a device's first call store the same address.
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= fqh::kMaxDevices) return nullptr;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    scratch_addr[dev].store(p, std::memory_order_release);
    return p;
}
}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

int fq_tensor_params_int(const float* x, int64_t n, int bits, int scheme, void* workspace,
                         size_t workspace_bytes, fq_int_params* params, uint32_t* flags,
                         hipStream_t stream) {
    if (!fqh::valid_bits(bits) || !fqh::valid_scheme(scheme)) return FQ_E_UNSUPPORTED;
    if (!x || n < 1 || !workspace || !params) return FQ_E_INVALID;
    if (workspace_bytes < fq_workspace_bytes(n) || !fqh::aligned(workspace, 16)) return FQ_E_INVALID;
    if (!fqh::aligned(params, 4) || !fqh::aligned(flags, 4) || !fqh::aligned(x, 4)) return FQ_E_INVALID;
    unsigned G = launch_partial<kMinMax>(x, n, workspace, stream);
    k_params_int_final<<<1, kFT, 0, stream>>>((const float4*)workspace, (int)G, bits,
                                             scheme == FQ_AFFINE, params, flags);
    return fqh::launched();
}

int fq_fake_quant_int_tensor(const float* x, int64_t n, int bits, int scheme,
                             const fq_int_params* params, void* codes, float* fq,
                             hipStream_t stream) {
    if (!fqh::valid_bits(bits) || !fqh::valid_scheme(scheme)) return FQ_E_UNSUPPORTED;
    if (!x || n < 1 || !params || (!codes && !fq)) return FQ_E_INVALID;
    if (!fqh::aligned(params, 4) || !fqh::aligned(x, 4) || !fqh::aligned(fq, 4)) return FQ_E_INVALID;
    const bool al = fqh::aligned(x, 16) && fqh::aligned(fq, 16) && fqh::aligned(codes, bits == 8 ? 4 : 2);
    const unsigned G = fqh::grid_all((n + 3) / 4, kB);
    uint8_t* cd = (uint8_t*)codes;
    const int aff = scheme == FQ_AFFINE;
    if (bits == 8) {
        if (al) k_fq_int_tensor<8, true><<<G, kB, 0, stream>>>(x, n, aff, params, cd, fq);
        else k_fq_int_tensor<8, false><<<G, kB, 0, stream>>>(x, n, aff, params, cd, fq);
    } else {
        if (al) k_fq_int_tensor<4, true><<<G, kB, 0, stream>>>(x, n, aff, params, cd, fq);
        else k_fq_int_tensor<4, false><<<G, kB, 0, stream>>>(x, n, aff, params, cd, fq);
    }
    return fqh::launched();
}

int fq_calibrate_fake_quant_int_tensor(const float* x, int64_t n, int bits, int scheme, void* workspace,
                                      size_t workspace_bytes, fq_int_params* params, void* codes, float* fq,
                                      uint32_t* flags, hipStream_t stream) {
    if (!fqh::valid_bits(bits) || !fqh::valid_scheme(scheme)) return FQ_E_UNSUPPORTED;
    if (!x || n < 1 || !workspace || !params || (!codes && !fq)) return FQ_E_INVALID;
    if (workspace_bytes < fq_workspace_bytes(n) || !fqh::aligned(workspace, 16)) return FQ_E_INVALID;
    if (!fqh::aligned(params, 4) || !fqh::aligned(flags, 4) || !fqh::aligned(x, 4) || !fqh::aligned(fq, 4))
        return FQ_E_INVALID;
    const bool al = fqh::aligned(x, 16) && fqh::aligned(fq, 16) && fqh::aligned(codes, bits == 8 ? 4 : 2);
    if (!al || fqh::reduce_blocks(n) > fqh::kFoldMaxParts) {
        // larger or unaligned tensors: the two calls (three launches)
        int st = fq_tensor_params_int(x, n, bits, scheme, workspace, workspace_bytes, params, flags, stream);
        if (st != FQ_OK) return st;
        return fq_fake_quant_int_tensor(x, n, bits, scheme, params, codes, fq, stream);
    }
    const unsigned G = launch_partial<kMinMax>(x, n, workspace, stream);
    int st = fqh::launched();
    if (st != FQ_OK) return st;
    const unsigned Q = fqh::grid_all((n + 3) / 4, kB);
    const int aff = scheme == FQ_AFFINE;
    uint8_t* cd = (uint8_t*)codes;
    if (bits == 8)
        k_fq_int_tensor_fold<8><<<Q, kB, 0, stream>>>(x, n, aff, (const float4*)workspace, (int)G, params, cd, fq, flags);
    else
        k_fq_int_tensor_fold<4><<<Q, kB, 0, stream>>>(x, n, aff, (const float4*)workspace, (int)G, params, cd, fq, flags);
    return fqh::launched();
}

int fq_calibrate_fake_quant_int_tensor_noalloc(const float* x, int64_t n, int bits, int scheme,
                                               fq_int_params* params, void* codes, float* fq, uint32_t* flags,
                                               hipStream_t stream) {
    // every argument check of the call below, before the first HIP call
    if (!fqh::valid_bits(bits) || !fqh::valid_scheme(scheme)) return FQ_E_UNSUPPORTED;
    if (!x || n < 1 || !params || (!codes && !fq)) return FQ_E_INVALID;
    if (!fqh::aligned(params, 4) || !fqh::aligned(flags, 4) || !fqh::aligned(x, 4) || !fqh::aligned(fq, 4))
        return FQ_E_INVALID;
    if (fq_workspace_bytes(n) > kScratchBytes) return FQ_E_INVALID;  // beyond the static scratch
    void* ws = scratch_ptr();
    if (!ws) return FQ_E_HIP;
    return fq_calibrate_fake_quant_int_tensor(x, n, bits, scheme, ws, kScratchBytes, params, codes, fq, flags,
                                              stream);
}

int fq_dequantize_int_tensor(const void* codes, int64_t n, int bits, const fq_int_params* params,
                             float* out, hipStream_t stream) {
    if (!fqh::valid_bits(bits)) return FQ_E_UNSUPPORTED;
    if (!codes || n < 1 || !params || !out) return FQ_E_INVALID;
    if (!fqh::aligned(params, 4) || !fqh::aligned(out, 4)) return FQ_E_INVALID;
    const bool al = fqh::aligned(out, 16) && fqh::aligned(codes, bits == 8 ? 4 : 2);
    const unsigned G = fqh::grid_all((n + 3) / 4, kB);
    const uint8_t* cd = (const uint8_t*)codes;
    if (bits == 8) {
        if (al) k_dq_int_tensor<8, true><<<G, kB, 0, stream>>>(cd, n, params, out);
        else k_dq_int_tensor<8, false><<<G, kB, 0, stream>>>(cd, n, params, out);
    } else {
        if (al) k_dq_int_tensor<4, true><<<G, kB, 0, stream>>>(cd, n, params, out);
        else k_dq_int_tensor<4, false><<<G, kB, 0, stream>>>(cd, n, params, out);
    }
    return fqh::launched();
}

int fq_ste_backward(const float* grad, int64_t n_grad, const float* x, int64_t n_x,
                    const float* bounds, float* grad_in, hipStream_t stream) {
    if (!grad || !x || !bounds || !grad_in || n_x < 1 || n_grad < 1) return FQ_E_INVALID;
    if (n_grad != n_x) return FQ_E_DIM;
    if (!fqh::aligned(grad, 4) || !fqh::aligned(x, 4) || !fqh::aligned(bounds, 4) ||
        !fqh::aligned(grad_in, 4))
        return FQ_E_INVALID;
    const bool al = fqh::aligned(grad, 16) && fqh::aligned(x, 16) && fqh::aligned(grad_in, 16);
    const unsigned G = fqh::grid_all((n_x + 3) / 4, kB);
    if (al) k_ste<true><<<G, kB, 0, stream>>>(grad, x, n_x, bounds, grad_in);
    else k_ste<false><<<G, kB, 0, stream>>>(grad, x, n_x, bounds, grad_in);
    return fqh::launched();
}

int fq_fp8_tensor_scale(const float* x, int64_t n, void* workspace, size_t workspace_bytes,
                        float* scale_e4m3, float* scale_e5m2, uint32_t* flags, hipStream_t stream) {
    if (!x || n < 1 || !workspace || (!scale_e4m3 && !scale_e5m2)) return FQ_E_INVALID;
    if (workspace_bytes < fq_workspace_bytes(n) || !fqh::aligned(workspace, 16)) return FQ_E_INVALID;
    if (!fqh::aligned(x, 4) || !fqh::aligned(scale_e4m3, 4) || !fqh::aligned(scale_e5m2, 4) ||
        !fqh::aligned(flags, 4))
        return FQ_E_INVALID;
    unsigned G = launch_partial<kAmax>(x, n, workspace, stream);
    k_fp8_scale_final<<<1, kFT, 0, stream>>>((const uint32_t*)workspace, (int)G, scale_e4m3, scale_e5m2,
                                            flags);
    return fqh::launched();
}

}  // extern "C"
