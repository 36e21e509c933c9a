// percentile.hip -- per-tensor calibration on clipped tails: the nearest-rank
// quantiles of the finite values, found by radix selection on the device.
//
// [QAT] optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
// Training (QAT) primitives": QuantParams::per_tensor_percentile (sort the
// values; lo = floor(cf * last), hi = ceil((1 - cf) * last) with f64
// arithmetic, last = count - 1; from_minmax(sorted[lo], sorted[hi])).  Non-finite
// values are left out and flagged NONFINITE (the page rejects them).
//
// Selection instead of a sort: each finite value maps to a 32-bit key whose
// unsigned order is the total order of the values (-0 before +0); three digit
// passes, most significant first (11, 11 and 10 bits), find the keys of rank lo
// and rank hi at once.
//
// A pass counts the digit of every key that shares the prefix fixed so far (one
// histogram per order statistic, one shared while the two prefixes agree) in
// LDS -- in the first pass every finite key counts and each wave keeps its own
// copy against contention -- and flushes the non-zero bins to that pass's
// histogram in the workspace with 64-bit atomic adds (integer counts: the result
// does not depend on their order).  The grid is capped (grid-stride loop): the
// flush atomics of all workgroups on a busy bin serialise.  The last workgroup
// to finish a pass (a counter taken after its flushes returned) scans the bins,
// narrows prefix and rank of both statistics, and after the last pass derives
// the parameters -- no separate select launches.
//
// The second pass also copies the keys that share either 11-bit prefix into a
// per-workgroup slice of the workspace (sized for one key in 16 of the
// workgroup's share; typically a few percent match); the third pass then reads
// only those slices, or x again if any slice overflowed.  Four launches; x is
// read twice (three times on overflow).
#include <cmath>

#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;
constexpr int kWaves = kB / kWave;
constexpr int kPasses = 3;
constexpr int kMaxBins = 2048;
constexpr int kU = 4;  // 16-byte loads in flight per thread

// Histogram workgroups: each flushes its non-zero bins with global atomics, and
// atomics on one address serialise, so the grid is capped (grid-stride loop).
#ifndef FQ_PCT_MAX_BLOCKS
#define FQ_PCT_MAX_BLOCKS 512
#endif
constexpr int64_t kMaxHistBlocks = FQ_PCT_MAX_BLOCKS;
constexpr int kCandShare = 16;  // candidate slots: one per 16 elements of a workgroup's share

// digit of pass p: bits [shift, shift + log2(bins)) of the key
__host__ __device__ constexpr int digit_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__host__ __device__ constexpr int digit_bins(int p) { return p == 2 ? 1024 : 2048; }

struct PctState {
    uint64_t hist[kPasses][2][kMaxBins];  // zeroed by k_pct_init
    uint64_t rank[2];
    uint64_t nfin;
    uint32_t prefix[2];
    uint32_t mask;
    uint32_t shared;  // the two prefixes agree: one histogram serves both
    uint32_t done[kPasses];
    uint32_t overflow;  // a candidate slice overflowed: the third pass reads x
    uint32_t cnt[kMaxHistBlocks];  // candidates kept by each workgroup
};

int64_t hist_blocks(int64_t n) {
    int64_t g = ((n >> 2) + (int64_t)kB * kU - 1) / ((int64_t)kB * kU);
    return g < 1 ? 1 : (g > kMaxHistBlocks ? kMaxHistBlocks : g);
}
// candidate slots per workgroup (a multiple of 4)
int64_t cand_per_block(int64_t n) {
    const int64_t g = hist_blocks(n);
    const int64_t chunks = ((n >> 2) + g - 1) / g;  // 16-byte chunks of one workgroup, at most
    return (4 * chunks / kCandShare + 64 + 3) / 4 * 4;
}
size_t state_bytes() { return (sizeof(PctState) + 255) / 256 * 256; }

__device__ __forceinline__ uint32_t sort_key(float v) {
    const uint32_t u = as_u(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return as_f((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ bool finite(float v) { return fabsf(v) < __builtin_inff(); }

__global__ __launch_bounds__(kB) void k_pct_init(PctState* __restrict__ st) {
    uint64_t* h = &st->hist[0][0][0];
    for (int i = blockIdx.x * kB + threadIdx.x; i < kPasses * 2 * kMaxBins; i += gridDim.x * kB) h[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->rank[0] = st->rank[1] = 0;
        st->nfin = 0;
        st->prefix[0] = st->prefix[1] = 0;
        st->mask = 0;
        st->shared = 1;
        for (int p = 0; p < kPasses; ++p) st->done[p] = 0;
        st->overflow = 0;
    }
}

// f(v) for every element of x, four per 16-byte chunk, kU chunks of a thread
// loaded before any is counted (past the end: NaN, which no pass counts)
template <bool AL, typename F>
__device__ __forceinline__ void for_each(const float* __restrict__ x, int64_t n, F&& f) {
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kB;
    for (int64_t c = (int64_t)blockIdx.x * kB + threadIdx.x; c < nfull; c += stride * kU) {
        float4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t cu = c + u * stride;
            if (cu < nfull) {
                if (AL) v[u] = reinterpret_cast<const float4*>(x)[cu];
                else v[u] = make_float4(x[4 * cu], x[4 * cu + 1], x[4 * cu + 2], x[4 * cu + 3]);
            } else {
                const float q = __builtin_nanf("");
                v[u] = make_float4(q, q, q, q);
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            f(v[u].x);
            f(v[u].y);
            f(v[u].z);
            f(v[u].w);
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) f(x[4 * nfull + threadIdx.x]);
}

// Adds c to a histogram count in the workspace and waits for the sum to come
// back: a count whose add has returned is in device memory, visible to the
// device-scope loads of the workgroup that selects.
__device__ __forceinline__ void flush_add(uint64_t* bin, uint32_t c) {
    const uint64_t old = __hip_atomic_fetch_add(bin, (uint64_t)c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(old));
}

// Taken by every workgroup after its flushes: the one that finishes a pass last
// gets true.  Each wave's flushes have returned before the barrier and the
// counter is taken after it, so the last workgroup's later device-scope loads
// see every count.  (No device-scope fence: on a multi-die part it would write
// back and invalidate the die's L2, and nothing here is a plain store.)
__device__ __forceinline__ bool last_to_finish(uint32_t* done) {
    __shared__ bool s_last;
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
    __syncthreads();
    return s_last;
}

// exclusive scan of one value per thread over the block (Hillis-Steele in LDS);
// the block total goes to *total
__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t v, uint64_t* s, uint64_t* total) {
    const int t = threadIdx.x;
    s[t] = v;
    __syncthreads();
    for (int off = 1; off < kB; off <<= 1) {
        const uint64_t add = t >= off ? s[t - off] : 0;
        __syncthreads();
        s[t] += add;
        __syncthreads();
    }
    const uint64_t incl = s[t];
    *total = s[kB - 1];
    __syncthreads();
    return incl - v;
}

struct SelectArgs {
    double cf;
    int bits, affine;
    fq_int_params* params;
    uint32_t* flags;
};

// Run by the whole last workgroup of pass PASS: the bin holding each statistic's
// rank fixes its next digit; ranks become ranks within those bins.  After the
// last pass the prefixes are the selected keys and the parameters follow.
template <int PASS>
__device__ void select_digit(PctState* __restrict__ st, int64_t n, const SelectArgs& a) {
    constexpr int BINS = digit_bins(PASS), SHIFT = digit_shift(PASS);
    constexpr int PER = BINS / kB;  // consecutive bins per thread
    __shared__ uint64_t scan[kB];
    __shared__ uint64_t s_rank[2];
    __shared__ uint64_t s_nfin;
    __shared__ uint32_t s_prefix[2];
    const int t = threadIdx.x;
    const bool shared = st->shared != 0;
    uint64_t hb[2][PER];
    uint64_t sum[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        // the counts were added by other workgroups: read them at device scope
        hb[0][j] = __hip_atomic_load(&st->hist[PASS][0][t * PER + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hb[1][j] = shared ? hb[0][j]
                          : __hip_atomic_load(&st->hist[PASS][1][t * PER + j], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
        sum[0] += hb[0][j];
        sum[1] += hb[1][j];
    }
    if (t == 0) {
        s_nfin = st->nfin;
        s_rank[0] = st->rank[0];
        s_rank[1] = st->rank[1];
        s_prefix[0] = st->prefix[0];
        s_prefix[1] = st->prefix[1];
    }
    __syncthreads();
    for (int s = 0; s < 2; ++s) {
        uint64_t total;
        const uint64_t excl = block_exclusive_scan(sum[s], scan, &total);
        if (PASS == 0 && s == 0 && t == 0) {
            // every finite value lands in a bin of the first pass: the count of
            // finite values and the two ranks follow from the total
            s_nfin = total;
            if (total > 0) {
                const uint64_t last = total - 1;
                const uint64_t lo = (uint64_t)floor(a.cf * (double)last);
                const uint64_t hi = (uint64_t)ceil((1.0 - a.cf) * (double)last);
                s_rank[0] = lo < last ? lo : last;
                s_rank[1] = hi < last ? hi : last;
            }
        }
        __syncthreads();
        const uint64_t r = s_rank[s];
        __syncthreads();
        if (s_nfin > 0 && excl <= r && r < excl + sum[s]) {
            uint64_t below = excl;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                if (r < below + hb[s][j]) {
                    s_rank[s] = r - below;
                    s_prefix[s] |= (uint32_t)(t * PER + j) << SHIFT;
                    break;
                }
                below += hb[s][j];
            }
        }
        __syncthreads();
    }
    if (t != 0) return;
    const uint64_t nfin = s_nfin;
    st->nfin = nfin;
    st->rank[0] = s_rank[0];
    st->rank[1] = s_rank[1];
    st->prefix[0] = s_prefix[0];
    st->prefix[1] = s_prefix[1];
    st->mask |= (uint32_t)(BINS - 1) << SHIFT;
    st->shared = s_prefix[0] == s_prefix[1] ? 1u : 0u;
    if (PASS != kPasses - 1) return;
    const float mn = nfin > 0 ? key_value(s_prefix[0]) : __builtin_inff();
    const float mx = nfin > 0 ? key_value(s_prefix[1]) : -__builtin_inff();
    const IntRange rg = int_range(a.bits, a.affine != 0);
    const IntCal cal = calibrate(mn, mx, rg, a.affine != 0);
    fq_int_params out;
    out.scale = cal.scale;
    out.zero_point = cal.zp;
    out.real_min = (float)(rg.qmin - cal.zp) * cal.scale;
    out.real_max = (float)(rg.qmax - cal.zp) * cal.scale;
    *a.params = out;
    const uint32_t f = ((int64_t)nfin < n ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
    if (a.flags && f) atomicOr(a.flags, f);
}

// first pass: the top 11 bits of every finite key, one LDS histogram per wave
template <bool AL>
__global__ __launch_bounds__(kB) void k_pct_first(const float* __restrict__ x, int64_t n, PctState* __restrict__ st,
                                                  SelectArgs a) {
    constexpr int BINS = digit_bins(0), SHIFT = digit_shift(0);
    __shared__ uint32_t h[kWaves][BINS];
    for (int i = threadIdx.x; i < kWaves * BINS; i += kB) (&h[0][0])[i] = 0;
    __syncthreads();
    uint32_t* hw = h[threadIdx.x / kWave];
    for_each<AL>(x, n, [&](float v) {
        if (finite(v)) atomicAdd(&hw[sort_key(v) >> SHIFT], 1u);
    });
    __syncthreads();
    for (int b = threadIdx.x; b < BINS; b += kB) {
        uint32_t cnt = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) cnt += h[w][b];
        if (cnt) flush_add(&st->hist[0][0][b], cnt);
    }
    if (last_to_finish(&st->done[0])) select_digit<0>(st, n, a);
}

// second pass: the middle 11 bits of the keys that share a statistic's 11-bit
// prefix; those keys are also kept in this workgroup's candidate slice
template <bool AL>
__global__ __launch_bounds__(kB) void k_pct_second(const float* __restrict__ x, int64_t n,
                                                   PctState* __restrict__ st, uint32_t* __restrict__ cand,
                                                   int64_t cap, SelectArgs a) {
    constexpr int BINS = digit_bins(1), SHIFT = digit_shift(1);
    __shared__ uint32_t h[2][BINS];
    __shared__ uint32_t s_cnt;
    for (int i = threadIdx.x; i < 2 * BINS; i += kB) (&h[0][0])[i] = 0;
    if (threadIdx.x == 0) s_cnt = 0;
    const uint32_t mask = st->mask, p0 = st->prefix[0], p1 = st->prefix[1];
    const bool shared = st->shared != 0;
    uint32_t* slice = cand + blockIdx.x * cap;
    const int lane = threadIdx.x % kWave;
    __syncthreads();
    for_each<AL>(x, n, [&](float v) {
        const bool fin = finite(v);
        const uint32_t k = sort_key(v);
        const bool m0 = fin && (k & mask) == p0;
        const bool m1 = fin && !shared && (k & mask) == p1;
        const uint32_t bin = (k >> SHIFT) & (BINS - 1);
        if (m0) atomicAdd(&h[0][bin], 1u);
        if (m1) atomicAdd(&h[1][bin], 1u);
        // keep the candidates: one LDS reservation per wave
        const uint64_t bal = __ballot(m0 || m1);
        if (bal) {
            const int leader = __builtin_ctzll(bal);
            uint32_t base = 0;
            if (lane == leader) base = atomicAdd(&s_cnt, (uint32_t)__builtin_popcountll(bal));
            base = __builtin_amdgcn_readlane(base, leader);
            const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if ((m0 || m1) && (int64_t)base + below < cap) slice[base + below] = k;
        }
    });
    __syncthreads();
    for (int b = threadIdx.x; b < BINS; b += kB) {
        if (h[0][b]) flush_add(&st->hist[1][0][b], h[0][b]);
        if (h[1][b]) flush_add(&st->hist[1][1][b], h[1][b]);
    }
    if (threadIdx.x == 0) {
        st->cnt[blockIdx.x] = (int64_t)s_cnt < cap ? s_cnt : (uint32_t)cap;
        if ((int64_t)s_cnt > cap) atomicOr(&st->overflow, 1u);
    }
    if (last_to_finish(&st->done[1])) select_digit<1>(st, n, a);
}

// third pass: the last 10 bits of the keys that share a statistic's 22-bit
// prefix, from this workgroup's candidates (or from x after an overflow)
template <bool AL>
__global__ __launch_bounds__(kB) void k_pct_third(const float* __restrict__ x, int64_t n, PctState* __restrict__ st,
                                                  const uint32_t* __restrict__ cand, int64_t cap, SelectArgs a) {
    constexpr int BINS = digit_bins(2), SHIFT = digit_shift(2);
    __shared__ uint32_t h[2][BINS];
    for (int i = threadIdx.x; i < 2 * BINS; i += kB) (&h[0][0])[i] = 0;
    const uint32_t mask = st->mask, p0 = st->prefix[0], p1 = st->prefix[1];
    const bool shared = st->shared != 0;
    const bool from_x = st->overflow != 0;
    __syncthreads();
    auto count = [&](uint32_t k) {
        const uint32_t bin = (k >> SHIFT) & (BINS - 1);
        if ((k & mask) == p0) atomicAdd(&h[0][bin], 1u);
        if (!shared && (k & mask) == p1) atomicAdd(&h[1][bin], 1u);
    };
    if (from_x) {
        for_each<AL>(x, n, [&](float v) {
            if (finite(v)) count(sort_key(v));
        });
    } else {
        const uint32_t* slice = cand + blockIdx.x * cap;
        const uint32_t m = st->cnt[blockIdx.x];
        for (uint32_t i = threadIdx.x; i < m; i += kB) count(slice[i]);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < BINS; b += kB) {
        if (h[0][b]) flush_add(&st->hist[2][0][b], h[0][b]);
        if (h[1][b]) flush_add(&st->hist[2][1][b], h[1][b]);
    }
    if (last_to_finish(&st->done[2])) select_digit<2>(st, n, a);
}

template <bool AL>
void launch_passes(const float* x, int64_t n, PctState* st, uint32_t* cand, int64_t cap, const SelectArgs& a,
                   hipStream_t stream) {
    const unsigned G = (unsigned)hist_blocks(n);
    k_pct_first<AL><<<G, kB, 0, stream>>>(x, n, st, a);
    k_pct_second<AL><<<G, kB, 0, stream>>>(x, n, st, cand, cap, a);
    k_pct_third<AL><<<G, kB, 0, stream>>>(x, n, st, cand, cap, a);
}

}  // namespace

extern "C" {

size_t fq_percentile_workspace_bytes(int64_t n) {
    if (n < 1) return 0;
    return state_bytes() + (size_t)(hist_blocks(n) * cand_per_block(n)) * sizeof(uint32_t);
}

int fq_tensor_params_percentile(const float* x, int64_t n, int bits, int scheme, double clip_fraction,
                                void* workspace, size_t workspace_bytes, fq_int_params* params, uint32_t* flags,
                                hipStream_t stream) {
    if (!fqh::valid_bits(bits) || !fqh::valid_scheme(scheme)) return FQ_E_UNSUPPORTED;
    if (!x || n < 1 || !workspace || !params || !(clip_fraction >= 0.0 && clip_fraction < 0.5)) return FQ_E_INVALID;
    if (workspace_bytes < fq_percentile_workspace_bytes(n) || !fqh::aligned(workspace, 16)) return FQ_E_INVALID;
    if (!fqh::aligned(x, 4) || !fqh::aligned(params, 4) || !fqh::aligned(flags, 4)) return FQ_E_INVALID;
    PctState* st = reinterpret_cast<PctState*>(workspace);
    uint32_t* cand = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(workspace) + state_bytes());
    const SelectArgs a{clip_fraction, bits, scheme == FQ_AFFINE ? 1 : 0, params, flags};
    k_pct_init<<<(kPasses * 2 * kMaxBins + kB - 1) / kB, kB, 0, stream>>>(st);
    if (fqh::aligned(x, 16)) launch_passes<true>(x, n, st, cand, cand_per_block(n), a, stream);
    else launch_passes<false>(x, n, st, cand, cand_per_block(n), a, stream);
    return fqh::launched();
}

}  // extern "C"
