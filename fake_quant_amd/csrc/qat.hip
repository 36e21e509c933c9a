// qat.hip -- one QAT optimizer step: AdamW update of the fp32 master weights,
// then the quantized view re-derived from the updated master.
//
// [QAT] optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
// Training (QAT) primitives": QatConfig (lr, beta1, beta2, eps, weight_decay),
// QatOptimizer::step (per element m = beta1 m + (1 - beta1) g,
// v = beta2 v + (1 - beta2) g g, m_hat = m / (1 - beta1^t), v_hat = v /
// (1 - beta2^t), decoupled decay w -= lr wd w, then w -= lr m_hat /
// (sqrt(v_hat) + eps)) and requantize (integer target: per_tensor_minmax of the
// updated master + fake_quant_int; fp8 target: fake_quant_fp8 of the master).
// Arithmetic is binary32 with one rounding per operation, in the page's order
// and association; the bias corrections are formed in double on the host and
// rounded once.
//
// Integer target: one pass updates w, m, v and leaves one finite min / max
// partial per workgroup (the tiling of the tensor-scope reduction); with nearest
// rounding every block of the requantize pass folds those partials itself and
// re-reads the updated master (two launches), with stochastic rounding a
// one-block pass derives the parameters first.  fp8 target: the view needs no
// tensor-wide value, so update and cast are one pass.
#include <cmath>

#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;
constexpr int kRT = fqh::kReduceThreads;
constexpr int kRU = fqh::kReduceChunks;

// binary32 constants of one step (formed on the host)
struct AdamStep {
    float lr, b1, b2, eps, wd;
    float c1, c2;    // 1 - beta1, 1 - beta2
    float lrwd;      // lr * wd
    float bc1, bc2;  // 1 - beta^t
};

// one element of the update; m_hat and v_hat divide by the uniform bias
// corrections through the exact-quotient helper when they allow it
__device__ __forceinline__ void adam1(float& w, float g, float& m, float& v, const AdamStep& a, const ExactDiv& d1,
                                      const ExactDiv& d2) {
    const float mi = a.b1 * m + a.c1 * g;
    const float vi = a.b2 * v + a.c2 * g * g;
    m = mi;
    v = vi;
    const float m_hat = d1.fast ? d1.quick(mi) : mi / d1.s;
    const float v_hat = d2.fast ? d2.quick(vi) : vi / d2.s;
    float wi = w;
    if (a.wd != 0.0f) wi = wi - a.lrwd * wi;
    w = wi - a.lr * m_hat / (sqrtf(v_hat) + a.eps);
}

__device__ __forceinline__ void adam4(float4& w, float4 g, float4& m, float4& v, const AdamStep& a,
                                      const ExactDiv& d1, const ExactDiv& d2) {
    adam1(w.x, g.x, m.x, v.x, a, d1, d2);
    adam1(w.y, g.y, m.y, v.y, a, d1, d2);
    adam1(w.z, g.z, m.z, v.z, a, d1, d2);
    adam1(w.w, g.w, m.w, v.w, a, d1, d2);
}

// Integer target, pass 1: the update of every element, and per workgroup the
// finite min / max / max |w| bits of the updated master (same partial records and
// tiling as the tensor-scope reduction, so pass 2 is shared).
template <bool AL>
__global__ __launch_bounds__(kRT) void k_adamw_minmax(float* __restrict__ w, const float* __restrict__ g,
                                                      float* __restrict__ m, float* __restrict__ v, int64_t n,
                                                      AdamStep a, float4* __restrict__ part) {
    const ExactDiv d1(a.bc1), d2(a.bc2);
    const int64_t nfull = n >> 2;
    const int64_t ntiles = (nfull + fqh::kReduceTile - 1) / fqh::kReduceTile;
    MinMax mm;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t c0 = tile * fqh::kReduceTile + threadIdx.x;
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
            const int64_t c = c0 + u * kRT;
            if (c >= nfull) continue;
            if (AL) {
                float4 wv = reinterpret_cast<float4*>(w)[c];
                const float4 gv = reinterpret_cast<const float4*>(g)[c];
                float4 mv = reinterpret_cast<float4*>(m)[c];
                float4 vv = reinterpret_cast<float4*>(v)[c];
                adam4(wv, gv, mv, vv, a, d1, d2);
                reinterpret_cast<float4*>(w)[c] = wv;  // re-read by the requantize pass
                store_nt(reinterpret_cast<float4*>(m) + c, mv);
                store_nt(reinterpret_cast<float4*>(v) + c, vv);
                mm.add(wv.x);
                mm.add(wv.y);
                mm.add(wv.z);
                mm.add(wv.w);
            } else {
                for (int e = 0; e < 4; ++e) {
                    const int64_t i = 4 * c + e;
                    float wi = w[i], mi = m[i], vi = v[i];
                    adam1(wi, g[i], mi, vi, a, d1, d2);
                    w[i] = wi;
                    m[i] = mi;
                    v[i] = vi;
                    mm.add(wi);
                }
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        const int64_t i = 4 * nfull + threadIdx.x;
        float wi = w[i], mi = m[i], vi = v[i];
        adam1(wi, g[i], mi, vi, a, d1, d2);
        w[i] = wi;
        m[i] = mi;
        v[i] = vi;
        mm.add(wi);
    }
    float4 r = make_float4(wave_min_f(mm.mn), wave_max_f(mm.mx), as_f(wave_max_u(mm.nf)), 0.f);
    __shared__ float4 lds[kRT / kWave];
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = r;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kRT / kWave; ++i) {
            r.x = fminf(r.x, lds[i].x);
            r.y = fmaxf(r.y, lds[i].y);
            r.z = as_f(max(as_u(r.z), as_u(lds[i].z)));
        }
        part[blockIdx.x] = r;
    }
}

// fp8 target: update, then the fp8 cast of the updated master itself (no scale;
// nearest through the conversion unit, stochastic through the Philox draws) and
// its decoded view; one chunk of four elements per thread.
template <int FMT, bool SR, bool AL>
__global__ __launch_bounds__(kB) void k_adamw_fp8(float* __restrict__ w, const float* __restrict__ g,
                                                  float* __restrict__ m, float* __restrict__ v, int64_t n, AdamStep a,
                                                  Draws dr, uint8_t* __restrict__ q, float* __restrict__ view) {
    const ExactDiv d1(a.bc1), d2(a.bc2);
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    for (int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x; c <= nfull; c += stride) {
        const int cnt = c < nfull ? 4 : (int)(n & 3);
        if (cnt == 0) break;
        float we[4], ge[4] = {0.f, 0.f, 0.f, 0.f}, me[4], ve[4];
        const bool vec = AL && cnt == 4;
        if (vec) {
            const float4 wv = reinterpret_cast<const float4*>(w)[c], gv = reinterpret_cast<const float4*>(g)[c];
            const float4 mv = reinterpret_cast<const float4*>(m)[c], vv = reinterpret_cast<const float4*>(v)[c];
            we[0] = wv.x; we[1] = wv.y; we[2] = wv.z; we[3] = wv.w;
            ge[0] = gv.x; ge[1] = gv.y; ge[2] = gv.z; ge[3] = gv.w;
            me[0] = mv.x; me[1] = mv.y; me[2] = mv.z; me[3] = mv.w;
            ve[0] = vv.x; ve[1] = vv.y; ve[2] = vv.z; ve[3] = vv.w;
        } else {
            for (int e = 0; e < 4; ++e) {
                const bool in = e < cnt;
                we[e] = in ? w[4 * c + e] : 0.f;
                ge[e] = in ? g[4 * c + e] : 0.f;
                me[e] = in ? m[4 * c + e] : 0.f;
                ve[e] = in ? v[4 * c + e] : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) adam1(we[e], ge[e], me[e], ve[e], a, d1, d2);
        uint32_t b[4];
        if (SR) {
            uint32_t j[4];
            dr.get(c, j);
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = fp8_encode_sr<FMT>(we[e], j[e]);
        } else {
            const uint32_t wd = fp8_encode4_hw<FMT>(we[0], we[1], we[2], we[3]);
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = (wd >> (8 * e)) & 0xFFu;
        }
        float vw[4];
        fp8_decode4_hw<FMT>(pack4(b[0], b[1], b[2], b[3]), vw);  // never an Inf code; NaN decodes to NaN
        if (vec) {
            store_nt(reinterpret_cast<float4*>(w) + c, make_float4(we[0], we[1], we[2], we[3]));
            store_nt(reinterpret_cast<float4*>(m) + c, make_float4(me[0], me[1], me[2], me[3]));
            store_nt(reinterpret_cast<float4*>(v) + c, make_float4(ve[0], ve[1], ve[2], ve[3]));
            if (q) reinterpret_cast<uint32_t*>(q)[c] = pack4(b[0], b[1], b[2], b[3]);
            if (view) store_nt(reinterpret_cast<float4*>(view) + c, make_float4(vw[0], vw[1], vw[2], vw[3]));
        } else {
            for (int e = 0; e < cnt; ++e) {
                const int64_t i = 4 * c + e;
                w[i] = we[e];
                m[i] = me[e];
                v[i] = ve[e];
                if (q) q[i] = (uint8_t)b[e];
                if (view) view[i] = vw[e];
            }
        }
    }
}

// validate the configuration and form the step's binary32 constants
int make_step(const fq_adamw_config* cfg, int64_t t, AdamStep* a) {
    if (!cfg || t < 1) return FQ_E_INVALID;
    const float b1 = cfg->beta1, b2 = cfg->beta2;
    if (!(b1 >= 0.0f && b1 < 1.0f) || !(b2 >= 0.0f && b2 < 1.0f)) return FQ_E_INVALID;
    a->lr = cfg->lr;
    a->b1 = b1;
    a->b2 = b2;
    a->eps = cfg->eps;
    a->wd = cfg->weight_decay;
    a->c1 = 1.0f - b1;
    a->c2 = 1.0f - b2;
    a->lrwd = cfg->lr * cfg->weight_decay;
    a->bc1 = (float)(1.0 - pow((double)b1, (double)t));
    a->bc2 = (float)(1.0 - pow((double)b2, (double)t));
    if (!(a->bc1 > 0.0f) || !(a->bc2 > 0.0f)) return FQ_E_INVALID;
    return FQ_OK;
}

bool valid_rounding(int r) { return r == FQ_ROUND_NEAREST || r == FQ_ROUND_STOCHASTIC; }

}  // namespace

extern "C" {

int fq_qat_step_int(float* master, const float* grad, float* m, float* v, int64_t n, const fq_adamw_config* cfg,
                    int64_t t, int bits, int scheme, int rounding, uint64_t seed, uint64_t offset, void* workspace,
                    size_t workspace_bytes, fq_int_params* params, void* codes, float* view, uint32_t* flags,
                    hipStream_t stream) {
    if (!fqh::valid_bits(bits) || !fqh::valid_scheme(scheme) || !valid_rounding(rounding)) return FQ_E_UNSUPPORTED;
    if (!master || !grad || !m || !v || n < 1 || !workspace || !params || (!codes && !view)) return FQ_E_INVALID;
    if (workspace_bytes < fq_workspace_bytes(n) || !fqh::aligned(workspace, 16)) return FQ_E_INVALID;
    if (!fqh::aligned(master, 4) || !fqh::aligned(grad, 4) || !fqh::aligned(m, 4) || !fqh::aligned(v, 4) ||
        !fqh::aligned(params, 4) || !fqh::aligned(view, 4) || !fqh::aligned(flags, 4))
        return FQ_E_INVALID;
    AdamStep a;
    int st = make_step(cfg, t, &a);
    if (st != FQ_OK) return st;
    unsigned G = fqh::reduce_blocks(n);
    const bool al = fqh::aligned(master, 16) && fqh::aligned(grad, 16) && fqh::aligned(m, 16) && fqh::aligned(v, 16);
    // nearest rounding: the requantize blocks fold the update pass's partials
    // themselves (two launches), so the update grid is capped at the number of
    // partials they take (its blocks loop over further tiles)
    const bool fold = rounding == FQ_ROUND_NEAREST;
    if (fold && G > (unsigned)fqh::kFoldGsMaxParts) G = (unsigned)fqh::kFoldGsMaxParts;
    if (al) k_adamw_minmax<true><<<G, kRT, 0, stream>>>(master, grad, m, v, n, a, (float4*)workspace);
    else k_adamw_minmax<false><<<G, kRT, 0, stream>>>(master, grad, m, v, n, a, (float4*)workspace);
    if ((st = fqh::launched()) != FQ_OK) return st;
    if (fold) return fqh::fake_quant_from_partials(master, n, bits, scheme, workspace, G, params, codes, view, flags, stream);
    if ((st = fqh::params_from_partials(workspace, G, bits, scheme, params, flags, stream)) != FQ_OK) return st;
    if (rounding == FQ_ROUND_NEAREST) return fq_fake_quant_int_tensor(master, n, bits, scheme, params, codes, view, stream);
    return fq_fake_quant_int_tensor_sr(master, n, bits, scheme, params, seed, offset, codes, view, stream);
}

int fq_qat_step_fp8(float* master, const float* grad, float* m, float* v, int64_t n, const fq_adamw_config* cfg,
                    int64_t t, int fmt, int rounding, uint64_t seed, uint64_t offset, uint8_t* q, float* view,
                    hipStream_t stream) {
    if (!fqh::valid_fmt(fmt) || !valid_rounding(rounding)) return FQ_E_UNSUPPORTED;
    if (!master || !grad || !m || !v || n < 1 || (!q && !view)) return FQ_E_INVALID;
    if (!fqh::aligned(master, 4) || !fqh::aligned(grad, 4) || !fqh::aligned(m, 4) || !fqh::aligned(v, 4) ||
        !fqh::aligned(view, 4))
        return FQ_E_INVALID;
    AdamStep a;
    int st = make_step(cfg, t, &a);
    if (st != FQ_OK) return st;
    const bool al = fqh::aligned(master, 16) && fqh::aligned(grad, 16) && fqh::aligned(m, 16) &&
                    fqh::aligned(v, 16) && fqh::aligned(q, 4) && fqh::aligned(view, 16);
    const unsigned G = fqh::grid_all(n / 4 + 1, kB);
    const Draws dr = Draws::make(seed, offset);
    const bool sr = rounding == FQ_ROUND_STOCHASTIC;
#define FQ_ADAMW_FP8(FMT, SR)                                                                                \
    do {                                                                                                     \
        if (al) k_adamw_fp8<FMT, SR, true><<<G, kB, 0, stream>>>(master, grad, m, v, n, a, dr, q, view);     \
        else k_adamw_fp8<FMT, SR, false><<<G, kB, 0, stream>>>(master, grad, m, v, n, a, dr, q, view);       \
    } while (0)
    if (fmt == FQ_E4M3) {
        if (sr) FQ_ADAMW_FP8(0, true);
        else FQ_ADAMW_FP8(0, false);
    } else {
        if (sr) FQ_ADAMW_FP8(1, true);
        else FQ_ADAMW_FP8(1, false);
    }
#undef FQ_ADAMW_FP8
    return fqh::launched();
}

}  // extern "C"
