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
// LDS -- in the first pass every finite key counts, in four copies against
// contention -- and adds the non-zero bins to the workspace with 64-bit atomics
// (integer counts: the result does not depend on their order).  Atomics on one
// address serialise, so the device histogram has four replicas (workgroup b adds
// into replica b mod 4) and the grid is capped at 256 workgroups of 1024 threads
// (grid-stride loop).
//
// The digit a pass fixes is selected at the start of the next launch: every
// workgroup of that launch sums the replicas and narrows prefix and rank of both
// statistics itself with a scan over the workgroup (the same integer counts give
// every workgroup the same selection; workgroup 0 stores it for the launches
// after).  The second pass issues the loads of the counts before its first loads
// of x and waits only for the counts, so the selection overlaps those loads; the
// later launches issue all their independent loads at once.  The launch boundary
// orders the counts before those reads, so no pass needs a counter or a fence.  A
// one-workgroup launch selects the last digit and derives the parameters.
//
// The second pass also copies the keys that share either 11-bit prefix into a
// per-workgroup slice of the workspace (one sub-slice per wave, together sized
// for one key in 16 of the workgroup's share; typically a few percent match); the
// third pass then reads only those slices, or x again if any slice overflowed.
//
// From kPredictMin elements on, the zeroing launch also predicts from a sample of
// x which first-digit bins will hold the two statistics, and the first pass keeps
// the keys of those bins as the candidates.  When the first digits the second
// pass selects are among the predicted bins and nothing overflowed, the second
// pass counts its digit over those candidates instead of x.  The selection always
// runs on the full counts, so a wrong prediction costs time, not correctness.
// Five launches (zeroing, three passes, the last selection); x is read once when
// the prediction holds, twice otherwise (three times on an overflow).
#include <cmath>

#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

// 1024 threads per workgroup (one workgroup of 16 waves per CU at the 256-workgroup
// cap): 31.4-31.6 / 45.3-45.6 us cold at 2^20 / 2^24 (33.3-33.4 / 46.6-46.8 with
// four 16-byte loads in flight per thread and a sample of 8192 values; 54.7-54.9
// us at 2^24 with x read twice; 35.3-35.5 / 56.0 with a one-wave selection and
// chained loads).  Measured slower at 2^24:
// 512 threads with 512 or 1024 workgroups (59.4-60.0 / 74.8-74.9 us), 1024 threads
// with 512 workgroups (69.0), eight 16-byte loads in flight (61.4-61.6), eight
// replicas (58.5-58.6); two replicas, eight LDS copies, copies picked by lane,
// plain loads of the counts and zeroing the later histograms in the first pass
// timed the same.  (The selection of a digit by the last workgroup of its own
// pass, found with an agent-scope release counter, took 63.5-64.2 us at 2^24.
// Only the last selection done so, by the workgroup of the third pass that draws
// the last ticket of a done counter, took 49.8 / 34.9 us at 2^24 / 2^20 with one
// agent-scope release per workgroup -- an L2 write-back each -- and 78.4 / 42.3
// with one per wave.)
#ifndef FQ_PCT_THREADS
#define FQ_PCT_THREADS 1024
#endif
constexpr int kPB = FQ_PCT_THREADS;  // threads per workgroup of the passes
constexpr int kPasses = 3;
constexpr int kMaxBins = 2048;
constexpr int kU = 2;       // 16-byte loads in flight per thread (3 or 4: 1.0-1.7 us slower cold; 1 and 8 slower too)
constexpr int kR = 4;       // replicas of the device histograms
constexpr int kCopies = 4;  // LDS copies of the first pass's histogram
constexpr int kCandShare = 16;  // candidate slots: one per 16 elements of a workgroup's share
constexpr int kPred = 8;         // predicted first-digit bins per order statistic, at most
constexpr int kPredShare = 32;   // a prediction holds at most 1 in 32 of the sampled values
constexpr int kSample = 4096;    // values the prediction samples
constexpr int kSampleRun = 16;   // consecutive values per run of the sample
constexpr int kSampleRuns = kSample / kSampleRun;
constexpr int kSampleCopies = 4;  // LDS copies of the sample's histogram (lane l counts into copy l mod 4)
constexpr int kInitThreads = 1024;
constexpr int64_t kPredictMin = (int64_t)1 << 23;  // elements from which the first pass keeps predicted keys

#ifndef FQ_PCT_MAX_BLOCKS
#define FQ_PCT_MAX_BLOCKS 256
#endif
constexpr int64_t kMaxHistBlocks = FQ_PCT_MAX_BLOCKS;

// digit of pass p: bits [shift, shift + log2(bins)) of the key
__host__ __device__ constexpr int digit_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__host__ __device__ constexpr int digit_bins(int p) { return p == 2 ? 1024 : 2048; }

// the selection after a pass's digit: per statistic the key prefix fixed so far
// and the rank among the keys that share it
struct PctSel {
    uint64_t rank[2];
    uint64_t nfin;
    uint32_t prefix[2];
    uint32_t mask;
    uint32_t shared;  // the two prefixes agree: one histogram serves both
};

// per statistic the first-digit bins [lo, lo + nb) expected to hold it (nb = 0:
// no prediction)
struct PctPred {
    uint32_t lo[2], nb[2];
};

struct PctState {
    uint64_t hist[kPasses][kR][2][kMaxBins];  // zeroed by k_pct_init
    PctPred pp;  // the prediction (k_pct_init)
    PctSel sel[kPasses - 1];  // after the digits of passes 0 and 1 (block 0 of the next launch stores it)
    uint32_t overflow;   // a candidate slice of the second pass overflowed: the third pass reads x
    uint32_t overflow1;  // a candidate slice of the first pass overflowed: the second pass reads x
    uint32_t cnt[kMaxHistBlocks][kPB / kWave];  // candidates kept by each wave (first pass, or the second when it reads x)
};

int64_t hist_blocks(int64_t n) {
    int64_t g = ((n >> 2) + (int64_t)kPB * kU - 1) / ((int64_t)kPB * kU);
    return g < 1 ? 1 : (g > kMaxHistBlocks ? kMaxHistBlocks : g);
}
// candidate slots per workgroup: one sub-slice per wave, each a multiple of 4
// slots (together about one per kCandShare elements of the workgroup's share)
int64_t cand_per_block(int64_t n) {
    const int64_t g = hist_blocks(n);
    const int64_t chunks = ((n >> 2) + g - 1) / g;  // 16-byte chunks of one workgroup, at most
    constexpr int64_t waves = kPB / kWave;
    return (((4 * chunks / kCandShare + 64) + waves - 1) / waves + 3) / 4 * 4 * waves;
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

// The raw 16-byte chunks of a group (nfull >= 1).  Every lane loads (a chunk past
// the end reloads the last one), so no branch sits between the loads and their
// use, which the compiler would otherwise close with a wait for the loads.
template <bool AL>
__device__ __forceinline__ void load_group(const float* __restrict__ x, int64_t nfull, int64_t c0, int64_t stride,
                                           float4 (&v)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t cu = c0 + threadIdx.x + u * stride;
        const int64_t cc = cu < nfull ? cu : nfull - 1;
        if (AL) v[u] = reinterpret_cast<const float4*>(x)[cc];
        else v[u] = make_float4(x[4 * cc], x[4 * cc + 1], x[4 * cc + 2], x[4 * cc + 3]);
    }
}

// the group's elements, NaN (not counted) for the chunks past the end
__device__ __forceinline__ void group_elems(const float4 (&v)[kU], int64_t nfull, int64_t c0, int64_t stride,
                                            float (&e)[4 * kU]) {
    const float q = __builtin_nanf("");
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const bool in = c0 + threadIdx.x + u * stride < nfull;
        e[4 * u] = in ? v[u].x : q;
        e[4 * u + 1] = in ? v[u].y : q;
        e[4 * u + 2] = in ? v[u].z : q;
        e[4 * u + 3] = in ? v[u].w : q;
    }
}

// f(e) for each thread's group of 4 kU elements (kU 16-byte chunks), the loop
// uniform over the workgroup: elements past the end are NaN, which no pass
// counts.  The 1-3 elements after the last whole chunk form one more group in
// workgroup 0.  pro() runs once, by every thread, while the first group's loads
// are in flight; each group's loads are issued before f() runs on the group
// before it.
template <bool AL, typename P, typename F>
__device__ __forceinline__ void for_each_group(const float* __restrict__ x, int64_t n, P&& pro, F&& f) {
    const int64_t nfull = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kPB;
    const int64_t step = stride * kU;
    int64_t c0 = (int64_t)blockIdx.x * kPB;
    if (nfull > 0) {
        float4 v[kU];
        load_group<AL>(x, nfull, c0, stride, v);
        pro();
        for (; c0 < nfull; c0 += step) {
            float e[4 * kU];
            group_elems(v, nfull, c0, stride, e);
            load_group<AL>(x, nfull, c0 + step, stride, v);  // the next group (past the end: unused)
            f(e);
        }
    } else {
        pro();
    }
    if (blockIdx.x == 0 && (n & 3)) {
        const float q = __builtin_nanf("");
        float e[4 * kU];
#pragma unroll
        for (int i = 0; i < 4 * kU; ++i) e[i] = q;
        if (threadIdx.x < (n & 3)) e[0] = x[4 * nfull + threadIdx.x];
        f(e);
    }
}

// Adds the non-zero counts of an LDS histogram (BINS bins, cnt(b) the count of
// bin b) to the device histogram g with agent-scope atomics (no value returned);
// the next launch reads the sums.
template <int BINS, typename C>
__device__ __forceinline__ void flush_bins(uint64_t* __restrict__ g, C&& cnt) {
    static_assert(BINS % kPB == 0, "whole bins per thread");
#pragma unroll
    for (int j = 0; j < BINS / kPB; ++j) {
        const int b = threadIdx.x + j * kPB;
        const uint32_t c = cnt(b);
        if (c) __hip_atomic_fetch_add(&g[b], (uint64_t)c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

struct SelectArgs {
    double cf;
    int bits, affine;
    fq_int_params* params;
    uint32_t* flags;
};

__device__ __forceinline__ uint64_t wave_inclusive_scan(uint64_t v) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint64_t y = __shfl_up(v, off);
        if (lane >= off) v += y;
    }
    return v;
}

// The selection before any digit: both statistics start with the empty prefix.
__device__ __forceinline__ PctSel no_selection() {
    PctSel z;
    z.rank[0] = z.rank[1] = 0;
    z.nfin = 0;
    z.prefix[0] = z.prefix[1] = 0;
    z.mask = 0;
    z.shared = 1;
    return z;
}

// This thread's bins of statistic s's replicas of pass PASS's histogram (agent
// scope), in registers
template <int PASS>
using BinCounts = uint64_t[digit_bins(PASS) / kPB][kR];

template <int PASS>
__device__ __forceinline__ void load_counts(PctState* __restrict__ st, int s, BinCounts<PASS>& c) {
    static_assert(digit_bins(PASS) % kPB == 0, "whole bins per thread");
#pragma unroll
    for (int j = 0; j < digit_bins(PASS) / kPB; ++j)
#pragma unroll
        for (int r = 0; r < kR; ++r)
            c[j][r] = __hip_atomic_load(&st->hist[PASS][r][s][threadIdx.x + j * kPB], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
}

// Run by every thread of a workgroup, after the launch that filled pass PASS's
// histograms, with c0 / c1 = load_counts of statistics 0 / 1 (c1 is read only
// when the two prefixes differ; a caller issues these loads together with its
// other independent loads): the replicas are summed into `sh` (LDS, 2 BINS counts),
// then a scan over the workgroup finds the bin holding each statistic's rank:
// that bin fixes the next digit, and the rank becomes the rank within the bin.  The first digit also yields the
// count of finite values and the two ranks ([QAT] per_tensor_percentile:
// floor(cf last), ceil((1 - cf) last) in f64).  The result is left in *out (LDS)
// and returned to every thread; every workgroup of a launch derives the same one
// from the same integer counts.
template <int PASS>
__device__ PctSel select_block(const PctSel& prev, double cf, uint64_t* sh, PctSel* out, const BinCounts<PASS>& c0,
                               const BinCounts<PASS>& c1) {
    constexpr int BINS = digit_bins(PASS), SHIFT = digit_shift(PASS);
    const bool shared = prev.shared != 0;
    auto sum = [&](int s, const BinCounts<PASS>& c) {
#pragma unroll
        for (int j = 0; j < BINS / kPB; ++j) {
            uint64_t t = 0;
#pragma unroll
            for (int r = 0; r < kR; ++r) t += c[j][r];
            sh[s * BINS + threadIdx.x + j * kPB] = t;
        }
    };
    sum(0, c0);
    if (!shared) sum(1, c1);
    __syncthreads();
    // thread t holds bins [t BPT, (t + 1) BPT) of each statistic's histogram (the
    // first histogram for both while they share it); a scan over the workgroup
    // (waves, then the wave totals) gives each thread the count below its bins
    constexpr int BPT = BINS / kPB;
    constexpr int NW = kPB / kWave;
    __shared__ uint64_t s_wave[2][NW];
    __shared__ uint64_t s_within[2];
    __shared__ uint32_t s_digit[2];
    const int t = threadIdx.x, lane = t % kWave, w = t / kWave;
    uint64_t hb[2][BPT], tot[2], incl[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int hs = shared ? 0 : k;
        tot[k] = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            hb[k][j] = sh[hs * BINS + t * BPT + j];
            tot[k] += hb[k][j];
        }
    }
    incl[0] = wave_inclusive_scan(tot[0]);
    incl[1] = shared ? incl[0] : wave_inclusive_scan(tot[1]);
    if (lane == kWave - 1) {
        s_wave[0][w] = incl[0];
        s_wave[1][w] = incl[1];
    }
    if (t == 0) {
        // no bin holds the rank (no finite value): digit 0, rank 0
        s_digit[0] = s_digit[1] = 0;
        s_within[0] = s_within[1] = 0;
    }
    __syncthreads();
    uint64_t below[2] = {0, 0}, all = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const uint64_t a0 = s_wave[0][v], a1 = s_wave[1][v];
        all += a0;
        if (v < w) {
            below[0] += a0;
            below[1] += a1;
        }
    }
    uint64_t nfin = prev.nfin;
    uint64_t rank[2] = {prev.rank[0], prev.rank[1]};
    if (PASS == 0) {
        // every finite value lands in a bin of the first pass
        nfin = all;
        if (nfin > 0) {
            const uint64_t last = nfin - 1;
            const uint64_t lo = (uint64_t)floor(cf * (double)last);
            const uint64_t hi = (uint64_t)ceil((1.0 - cf) * (double)last);
            rank[0] = lo < last ? lo : last;
            rank[1] = hi < last ? hi : last;
        }
    }
    if (nfin > 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint64_t b = below[k] + incl[k] - tot[k];
            const uint64_t r = rank[k];
            if (b <= r && r < b + tot[k]) {
#pragma unroll
                for (int j = 0; j < BPT; ++j) {
                    if (r < b + hb[k][j]) {
                        s_digit[k] = (uint32_t)(t * BPT + j);
                        s_within[k] = r - b;
                        break;
                    }
                    b += hb[k][j];
                }
            }
        }
    }
    __syncthreads();
    if (t == 0) {
        PctSel r;
        r.nfin = nfin;
        r.rank[0] = nfin > 0 ? s_within[0] : rank[0];
        r.rank[1] = nfin > 0 ? s_within[1] : rank[1];
        r.prefix[0] = prev.prefix[0] | (nfin > 0 ? s_digit[0] << SHIFT : 0u);
        r.prefix[1] = prev.prefix[1] | (nfin > 0 ? s_digit[1] << SHIFT : 0u);
        r.mask = prev.mask | ((uint32_t)(BINS - 1) << SHIFT);
        r.shared = r.prefix[0] == r.prefix[1] ? 1u : 0u;
        *out = r;
    }
    __syncthreads();
    return *out;
}

// ---------------------------------------------------------------------------
// Zeroing and prediction (one launch).  The workgroups zero the histograms and
// flags.  For tensors of at least kPredictMin elements one more workgroup
// predicts, per order statistic, the first-digit bins that will hold it, from a
// sample of kSample values spread evenly over x: it counts the sample's first
// digits, finds the sample ranks cf (count - 1) and (1 - cf) (count - 1) widened
// by three standard deviations of a binomial count plus two, and keeps the run of
// bins those ranks span when it is at most kPred bins long and holds at most 1 in
// kPredShare sampled values (a long run or a heavy bin, as ties at a percentile
// make, means no prediction).  A prediction only decides which keys the first
// pass keeps; the selection always runs on the full counts, and a wrong
// prediction sends the second pass back to x.  Below kPredictMin elements the
// second pass reads x again, which costs less than the prediction.
// ---------------------------------------------------------------------------
constexpr int kHistWords = kPasses * kR * 2 * kMaxBins;
constexpr int kSamplePer = kSample / kInitThreads;  // sample values per thread
static_assert(kSample % kInitThreads == 0 && digit_bins(0) % kInitThreads == 0, "whole shares per thread");

__device__ void predict_bins(PctState* __restrict__ st, const float* __restrict__ x, int64_t n, double cf) {
    constexpr int BINS = digit_bins(0), SHIFT = digit_shift(0);
    constexpr int BPT = BINS / kInitThreads, NW = kInitThreads / kWave;
    __shared__ uint32_t h[kSampleCopies * BINS];
    __shared__ uint32_t s_wave[NW];
    __shared__ uint32_t s_bin[4];
    const int t = threadIdx.x, lane = t % kWave, w = t / kWave;
    for (int i = t; i < kSampleCopies * BINS; i += kInitThreads) h[i] = 0;
    if (t < 4) s_bin[t] = 0;
    // the sample: all of x when n <= kSample, else kSampleRuns runs of
    // kSampleRun consecutive values, run r starting at floor(r n / kSampleRuns)
    // rounded down to a multiple of kSampleRun (the runs are distinct and whole
    // cache lines).  Every lane loads (an index past a smaller x reloads its last
    // value and is not counted), so the loads go out together.
    const int64_t S = n < kSample ? n : kSample;
    const double step = (double)n / (double)kSampleRuns;
    float v[kSamplePer];
#pragma unroll
    for (int j = 0; j < kSamplePer; ++j) {
        const int64_t i = t + j * kInitThreads;
        int64_t e;
        if (n <= kSample) {
            e = i < n ? i : n - 1;
        } else {
            const int64_t r = i / kSampleRun;
            e = ((int64_t)((double)r * step) & ~(int64_t)(kSampleRun - 1)) + i % kSampleRun;
        }
        v[j] = x[e];
    }
    __syncthreads();
    // lanes of one instruction spread over kSampleCopies histograms: most sampled
    // values fall in a few bins, whose atomics would otherwise queue on one address
    uint32_t* hc = h + (lane % kSampleCopies) * BINS;
#pragma unroll
    for (int j = 0; j < kSamplePer; ++j)
        if (t + j * kInitThreads < S && finite(v[j])) atomicAdd(&hc[sort_key(v[j]) >> SHIFT], 1u);
    __syncthreads();
    uint32_t hb[BPT], tot = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        hb[j] = 0;
#pragma unroll
        for (int c = 0; c < kSampleCopies; ++c) hb[j] += h[c * BINS + t * BPT + j];
        tot += hb[j];
    }
    __syncthreads();  // every copy is read before the sums overwrite copy 0
#pragma unroll
    for (int j = 0; j < BPT; ++j) h[t * BPT + j] = hb[j];
    const uint32_t incl = (uint32_t)wave_inclusive_scan(tot);
    if (lane == kWave - 1) s_wave[w] = incl;
    __syncthreads();
    uint32_t below = 0, all = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        all += s_wave[k];
        if (k < w) below += s_wave[k];
    }
    if (all > 0) {
        const double last = (double)(all - 1);
        const uint32_t r[2] = {(uint32_t)floor(cf * last), (uint32_t)fmin(ceil((1.0 - cf) * last), last)};
        const uint32_t m = (uint32_t)ceil(3.0 * sqrt((double)all * cf * (1.0 - cf))) + 2u;
        const uint32_t ends[4] = {r[0] > m ? r[0] - m : 0u, r[0] + m < all ? r[0] + m : all - 1,
                                  r[1] > m ? r[1] - m : 0u, r[1] + m < all ? r[1] + m : all - 1};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t b = below + incl - tot;
            if (b <= ends[e] && ends[e] < b + tot) {
#pragma unroll
                for (int j = 0; j < BPT; ++j) {
                    if (ends[e] < b + hb[j]) {
                        s_bin[e] = (uint32_t)(t * BPT + j);
                        break;
                    }
                    b += hb[j];
                }
            }
        }
    }
    __syncthreads();
    if (t == 0) {
        PctPred p;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint32_t lo = s_bin[2 * k], hi = s_bin[2 * k + 1];
            const uint32_t nb = hi - lo + 1;
            uint32_t held = 0;
            if (nb <= kPred)
                for (uint32_t b = lo; b <= hi; ++b) held += h[b];
            p.lo[k] = lo;
            p.nb[k] = all > 0 && nb <= kPred && (uint64_t)held * kPredShare <= all ? nb : 0u;
        }
        st->pp = p;
    }
}

// zeroing workgroups, then (predict != 0) the predicting one
__global__ __launch_bounds__(kInitThreads) void k_pct_init(PctState* __restrict__ st, const float* __restrict__ x,
                                                           int64_t n, double cf, int predict) {
    const unsigned zb = gridDim.x - (predict ? 1u : 0u);  // zeroing workgroups
    if (blockIdx.x >= zb) {
        predict_bins(st, x, n, cf);
        return;
    }
    uint64_t* h = &st->hist[0][0][0][0];
    for (int64_t i = (int64_t)blockIdx.x * kInitThreads + threadIdx.x; i < kHistWords; i += (int64_t)zb * kInitThreads)
        h[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->overflow = 0;
        st->overflow1 = 0;
        if (!predict) st->pp = PctPred{{0u, 0u}, {0u, 0u}};
    }
}
constexpr unsigned kInitBlocks = (kHistWords + kInitThreads - 1) / kInitThreads;

// Keeps the keys of this thread's group whose bit i of mbits is set in its
// wave's sub-slice of the candidate slice (capw slots; wcnt is the wave's count,
// the same in every lane, and runs on past capw so that an overflow shows) and
// calls kept(key) for each.  Candidates are rare, so only an element slot that
// some lane keeps does any of this, and it needs no atomic: a key's position is
// the wave's count plus the number of keeping lanes below its own.
template <int NE, typename K>
__device__ __forceinline__ void keep_in_wave(const uint32_t (&keys)[NE], uint32_t mbits, uint32_t* __restrict__ sub,
                                             uint32_t capw, uint32_t& wcnt, K&& kept) {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const uint64_t bal = __ballot((mbits >> i) & 1u);
        if (bal == 0) continue;
        if ((mbits >> i) & 1u) {
            const uint32_t below =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            const uint32_t pos = wcnt + below;
            if (pos < capw) sub[pos] = keys[i];
            kept(keys[i]);
        }
        wcnt += (uint32_t)__builtin_popcountll(bal);
    }
}

// the wave's count of kept candidates (at most capw) and the overflow flag
__device__ __forceinline__ void store_wave_count(PctState* __restrict__ st, uint32_t wcnt, uint32_t capw,
                                                 uint32_t* __restrict__ overflow) {
    if (threadIdx.x % kWave == 0) {
        st->cnt[blockIdx.x][threadIdx.x / kWave] = wcnt < capw ? wcnt : capw;
        if (wcnt > capw) atomicOr(overflow, 1u);
    }
}

// first pass: the top 11 bits of every finite key, kCopies LDS histograms (waves
// w and w + kCopies share one).  With a prediction, a key in a statistic's
// predicted bins is also kept in its wave's candidate sub-slice.
template <bool AL>
__global__ __launch_bounds__(kPB) void k_pct_first(const float* __restrict__ x, int64_t n, PctState* __restrict__ st,
                                                   uint32_t* __restrict__ cand, int64_t cap) {
    constexpr int BINS = digit_bins(0), SHIFT = digit_shift(0);
    __shared__ uint32_t h[kCopies * BINS];
    const PctPred pp = st->pp;
    const bool pred = pp.nb[0] != 0 && pp.nb[1] != 0;
    for (int i = threadIdx.x; i < kCopies * BINS; i += kPB) h[i] = 0;
    __syncthreads();
    uint32_t* hw = h + ((threadIdx.x / kWave) % kCopies) * BINS;
    const uint32_t capw = (uint32_t)(cap / (kPB / kWave));
    uint32_t* sub = cand + blockIdx.x * cap + (threadIdx.x / kWave) * capw;
    uint32_t wcnt = 0;
    for_each_group<AL>(x, n, [] {}, [&](const float (&e)[4 * kU]) {
        if (!pred) {
#pragma unroll
            for (int i = 0; i < 4 * kU; ++i)
                if (finite(e[i])) atomicAdd(&hw[sort_key(e[i]) >> SHIFT], 1u);
            return;
        }
        uint32_t keys[4 * kU];
        uint32_t mbits = 0;  // bit i: element i is a candidate
#pragma unroll
        for (int i = 0; i < 4 * kU; ++i) {
            const bool fin = finite(e[i]);
            const uint32_t k = sort_key(e[i]);
            const uint32_t b = k >> SHIFT;
            if (fin) atomicAdd(&hw[b], 1u);
            const bool m = fin && (b - pp.lo[0] < pp.nb[0] || b - pp.lo[1] < pp.nb[1]);
            keys[i] = k;
            mbits |= m ? 1u << i : 0u;
        }
        keep_in_wave(keys, mbits, sub, capw, wcnt, [](uint32_t) {});
    });
    __syncthreads();
    flush_bins<BINS>(st->hist[0][blockIdx.x % kR][0], [&](int b) {
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < kCopies; ++w) c += h[w * BINS + b];
        return c;
    });
    if (pred) store_wave_count(st, wcnt, capw, &st->overflow1);
}

// second pass: every workgroup first derives the first digit from the first
// pass's histogram (workgroup 0 stores the selection for the launches after it),
// then counts the middle 11 bits of the keys that share a statistic's 11-bit
// prefix.  When both statistics' bins were predicted and no sub-slice
// overflowed, those keys are among the first pass's candidates, and each wave
// counts its own sub-slice: x is not read again and the candidates stay for the
// third pass.  Otherwise the pass reads x and keeps the matching keys as the new
// candidates.
template <bool AL>
__global__ __launch_bounds__(kPB) void k_pct_second(const float* __restrict__ x, int64_t n,
                                                    PctState* __restrict__ st, uint32_t* __restrict__ cand,
                                                    int64_t cap, double cf) {
    constexpr int BINS = digit_bins(1), SHIFT = digit_shift(1), SHIFT0 = digit_shift(0);
    __shared__ uint64_t sh[2 * digit_bins(0)];
    __shared__ PctSel s_sel;
    __shared__ uint32_t h[2 * BINS];
    uint32_t* h0 = h;
    uint32_t* h1 = h + BINS;
    // the loads that do not depend on the selection go out first: the counts, the
    // prediction, the first pass's overflow flag, this wave's candidate count and
    // its first candidates (slots past the count are read but not used)
    BinCounts<0> c0;
    load_counts<0>(st, 0, c0);
    const PctPred pp = st->pp;
    const uint32_t ovf1 = st->overflow1;
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const uint32_t capw = (uint32_t)(cap / (kPB / kWave));
    uint32_t* sub = cand + blockIdx.x * cap + w * capw;
    const uint32_t m1 = st->cnt[blockIdx.x][w];
    const uint32_t k0 = (uint32_t)lane < capw ? sub[lane] : 0u;
    for (int i = threadIdx.x; i < 2 * BINS; i += kPB) h[i] = 0;
    // the barriers in select_block also order the zeroing above before the counts
    const PctSel sel = select_block<0>(no_selection(), cf, sh, &s_sel, c0, c0);
    if (blockIdx.x == 0 && threadIdx.x == 0) st->sel[0] = sel;
    const uint32_t d0 = (sel.prefix[0] >> SHIFT0) - pp.lo[0], d1 = (sel.prefix[1] >> SHIFT0) - pp.lo[1];
    const bool shared = sel.shared != 0;
    const uint32_t mask = sel.mask, p0 = sel.prefix[0], p1 = sel.prefix[1];
    auto count = [&](uint32_t k) {
        const uint32_t bin = (k >> SHIFT) & (BINS - 1);
        if ((k & mask) == p0) atomicAdd(&h0[bin], 1u);
        if (!shared && (k & mask) == p1) atomicAdd(&h1[bin], 1u);
    };
    if (sel.nfin > 0 && ovf1 == 0 && d0 < pp.nb[0] && d1 < pp.nb[1]) {
        if ((uint32_t)lane < m1) count(k0);
        for (uint32_t i = lane + kWave; i < m1; i += kWave) count(sub[i]);
        __syncthreads();
        flush_bins<BINS>(st->hist[1][blockIdx.x % kR][0], [&](int b) { return h0[b]; });
        if (!shared) flush_bins<BINS>(st->hist[1][blockIdx.x % kR][1], [&](int b) { return h1[b]; });
        return;
    }
    uint32_t wcnt = 0;
    for_each_group<AL>(x, n, [] {}, [&](const float (&e)[4 * kU]) {
        uint32_t keys[4 * kU];
        uint32_t mbits = 0;  // bit i: element i is a candidate
#pragma unroll
        for (int i = 0; i < 4 * kU; ++i) {
            const uint32_t k = sort_key(e[i]);
            const bool fin = finite(e[i]);
            const bool m = fin && ((k & mask) == p0 || (!shared && (k & mask) == p1));
            keys[i] = k;
            mbits |= m ? 1u << i : 0u;
        }
        keep_in_wave(keys, mbits, sub, capw, wcnt, count);
    });
    __syncthreads();
    flush_bins<BINS>(st->hist[1][blockIdx.x % kR][0], [&](int b) { return h0[b]; });
    if (!shared) flush_bins<BINS>(st->hist[1][blockIdx.x % kR][1], [&](int b) { return h1[b]; });
    store_wave_count(st, wcnt, capw, &st->overflow);
}

// third pass: every workgroup derives the second digit (workgroup 0 stores the
// selection), then counts the last 10 bits of the keys that share a statistic's
// 22-bit prefix, from this workgroup's candidates (or from x after an overflow)
template <bool AL>
__global__ __launch_bounds__(kPB) void k_pct_third(const float* __restrict__ x, int64_t n, PctState* __restrict__ st,
                                                   const uint32_t* __restrict__ cand, int64_t cap) {
    constexpr int BINS = digit_bins(2), SHIFT = digit_shift(2);
    __shared__ uint64_t sh[2 * digit_bins(1)];
    __shared__ PctSel s_sel;
    __shared__ uint32_t h[2 * BINS];
    uint32_t* h0 = h;
    uint32_t* h1 = h + BINS;
    for (int i = threadIdx.x; i < 2 * BINS; i += kPB) h[i] = 0;
    // every load that does not depend on another goes out at once: the selection
    // of the first digit, both statistics' counts, the overflow flag, this wave's
    // candidate count and its first candidates (slots past the count are read but
    // not used; the wave's sub-slice holds capw slots).  Wave w reads sub-slice w.
    const PctSel prev = st->sel[0];
    BinCounts<1> c0, c1;
    load_counts<1>(st, 0, c0);
    load_counts<1>(st, 1, c1);
    const bool from_x = st->overflow != 0;
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const uint32_t capw = (uint32_t)(cap / (kPB / kWave));
    const uint32_t* sub = cand + blockIdx.x * cap + w * capw;
    const uint32_t m = st->cnt[blockIdx.x][w];
    const uint32_t k0 = (uint32_t)lane < capw ? sub[lane] : 0u;
    const PctSel sel = select_block<1>(prev, 0.0, sh, &s_sel, c0, c1);
    if (blockIdx.x == 0 && threadIdx.x == 0) st->sel[1] = sel;
    const uint32_t mask = sel.mask, p0 = sel.prefix[0], p1 = sel.prefix[1];
    const bool shared = sel.shared != 0;
    auto count = [&](uint32_t k) {
        const uint32_t bin = (k >> SHIFT) & (BINS - 1);
        if ((k & mask) == p0) atomicAdd(&h0[bin], 1u);
        if (!shared && (k & mask) == p1) atomicAdd(&h1[bin], 1u);
    };
    if (from_x) {
        for_each_group<AL>(x, n, [] {}, [&](const float (&e)[4 * kU]) {
#pragma unroll
            for (int i = 0; i < 4 * kU; ++i)
                if (finite(e[i])) count(sort_key(e[i]));
        });
    } else {
        if ((uint32_t)lane < m) count(k0);
        for (uint32_t i = lane + kWave; i < m; i += kWave) count(sub[i]);
    }
    __syncthreads();
    flush_bins<BINS>(st->hist[2][blockIdx.x % kR][0], [&](int b) { return h0[b]; });
    if (!shared) flush_bins<BINS>(st->hist[2][blockIdx.x % kR][1], [&](int b) { return h1[b]; });
}

// one workgroup: the last digit fixes both keys, whose values are the clip
// range ([QAT] from_minmax(sorted[lo], sorted[hi]))
__global__ __launch_bounds__(kPB) void k_pct_final(PctState* __restrict__ st, int64_t n, SelectArgs a) {
    __shared__ uint64_t sh[2 * digit_bins(2)];
    __shared__ PctSel s_sel;
    const PctSel prev = st->sel[1];
    BinCounts<2> c0, c1;
    load_counts<2>(st, 0, c0);
    load_counts<2>(st, 1, c1);
    const PctSel sel = select_block<2>(prev, a.cf, sh, &s_sel, c0, c1);
    if (threadIdx.x != 0) return;
    const uint64_t nfin = sel.nfin;
    const float mn = nfin > 0 ? key_value(sel.prefix[0]) : __builtin_inff();
    const float mx = nfin > 0 ? key_value(sel.prefix[1]) : -__builtin_inff();
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

template <bool AL>
void launch_passes(const float* x, int64_t n, PctState* st, uint32_t* cand, int64_t cap, const SelectArgs& a,
                   hipStream_t stream) {
    const unsigned G = (unsigned)hist_blocks(n);
    k_pct_first<AL><<<G, kPB, 0, stream>>>(x, n, st, cand, cap);
    k_pct_second<AL><<<G, kPB, 0, stream>>>(x, n, st, cand, cap, a.cf);
    k_pct_third<AL><<<G, kPB, 0, stream>>>(x, n, st, cand, cap);
    k_pct_final<<<1, kPB, 0, stream>>>(st, n, a);
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
    const int predict = n >= kPredictMin;
    k_pct_init<<<kInitBlocks + (predict ? 1u : 0u), kInitThreads, 0, stream>>>(st, x, n, clip_fraction, predict);
    if (fqh::aligned(x, 16)) launch_passes<true>(x, n, st, cand, cand_per_block(n), a, stream);
    else launch_passes<false>(x, n, st, cand, cand_per_block(n), a, stream);
    return fqh::launched();
}

}  // extern "C"
