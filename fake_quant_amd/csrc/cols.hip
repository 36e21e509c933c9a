// cols.hip -- per-column (axis 1) calibration and integer quantization of a
// row-major [rows, cols] tensor.
//
// [QAT] optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
// Training (QAT) primitives": per_channel_params and fake_quant_int_per_channel
// with axis = 1 (each column is a channel, calibrated on that column only).
//
// A column's elements are cols apart, so a block works on a tile of 64 column
// vectors over a band of rows (each wave reads or writes one contiguous run of a
// row per instruction), its four waves taking every fourth row with several row
// loads in flight per thread.  Three launches, none with a global atomic on the
// data path:
//   1. k_cols_minmax: finite min / max / non-finite of each column over each
//      band of rows (at most 64 bands), vectors of 4 fp32 or 8 bf16 columns
//      (16-byte loads), waves merged through LDS, one partial record per
//      (band, column);
//   2. k_cols_fold: four threads per column fold its band partials, merged
//      through LDS into one record per column;
//   3. k_cols_quant: vectors of four columns for either dtype; each block
//      derives the parameters of its tile's columns ([QAT] from_minmax) into LDS
//      once, then quantizes its rows; the blocks of the first band also write
//      the scales, zero-points and flags.
// x is read twice; the workspace holds the partials and the column records.
// Tensors of 1025..4096 rows whose column count is a multiple of the strip width
// (16 fp32 or 32 bf16 columns), with at least half as many strips as compute
// units, take one launch instead, k_cols_strip, which reads x once (below).
#include "fq_device.h"
#include "fq_host.h"

using namespace fqk;

namespace {

constexpr int kB = fqh::kBlock;
constexpr int kWaves = kB / kWave;   // waves per block
constexpr int64_t kMaxBands = 64;    // bands of the min / max pass (partials per column)
constexpr int kQuantVec = 4;         // columns per lane in the quantize pass
constexpr int kU = 4;                // row loads in flight per thread (quantize pass); 8 and 16 measured slower
constexpr int kQuantRows = kWaves * kU;  // rows per band of the quantize pass
constexpr int kFoldU = 16;           // band partials in flight per thread of the fold
constexpr int kUm = 8;  // row loads in flight per thread (min / max pass); 4 and 16 time the same
constexpr int64_t kMaxQuantBands = 65535;  // grid y limit; blocks loop over further bands

int64_t minmax_bands(int64_t rows) { return rows < kMaxBands ? rows : kMaxBands; }

template <int DT>
struct ColVec {
    static constexpr int N = DT == FQ_F32 ? 4 : 8;
};

// element e of the vector of N columns starting at column c0 of row r
// (aligned: one 16-byte load, or 8 bytes for four bf16; otherwise element
// loads, out-of-range as 0)
template <int DT, int N, bool AL>
__device__ __forceinline__ void load_cols(const void* __restrict__ x, int64_t r, int64_t cols, int64_t c0,
                                          float (&v)[N]) {
    static_assert(N == ColVec<DT>::N || (DT == FQ_BF16 && N == 4), "a vector is 16 bytes, or four bf16");
    if constexpr (AL) {
        if constexpr (DT == FQ_BF16 && N == 4) {
            const uint2 q = reinterpret_cast<const uint2*>(x)[(r * cols + c0) / 4];
            v[0] = bf16_lo(q.x);
            v[1] = bf16_hi(q.x);
            v[2] = bf16_lo(q.y);
            v[3] = bf16_hi(q.y);
        } else if constexpr (DT == FQ_F32) {
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
__global__ __launch_bounds__(kB) void k_cols_minmax(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t rows_per_band, float4* __restrict__ part) {
    constexpr int N = ColVec<DT>::N;
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int64_t c0 = ((int64_t)blockIdx.x * kWave + lane) * N;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_band;
    const int64_t r1 = r0 + rows_per_band < rows ? r0 + rows_per_band : rows;
    MinMax m[N];
    if (c0 < cols) {
        for (int64_t r = r0 + w; r < r1; r += kWaves * kUm) {
            float v[kUm][N];
            // rows past the band repeat the band's last row: min / max unchanged
#pragma unroll
            for (int u = 0; u < kUm; ++u) {
                const int64_t rr = r + u * kWaves;
                load_cols<DT, N, AL>(x, rr < r1 ? rr : r1 - 1, cols, c0, v[u]);
            }
#pragma unroll
            for (int u = 0; u < kUm; ++u)
#pragma unroll
                for (int e = 0; e < N; ++e) m[e].add(v[u][e]);
        }
    }
    __shared__ float s_mn[kWaves - 1][N][kWave], s_mx[kWaves - 1][N][kWave];
    __shared__ uint32_t s_nf[kWaves - 1][N][kWave];
    if (w > 0) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            s_mn[w - 1][e][lane] = m[e].mn;
            s_mx[w - 1][e][lane] = m[e].mx;
            s_nf[w - 1][e][lane] = m[e].nf;
        }
    }
    __syncthreads();
    if (w != 0 || c0 >= cols) return;
    float4* prow = part + blockIdx.y * cols;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        for (int k = 0; k < kWaves - 1; ++k) m[e].merge(s_mn[k][e][lane], s_mx[k][e][lane], s_nf[k][e][lane]);
        if (c0 + e < cols) prow[c0 + e] = make_float4(m[e].mn, m[e].mx, as_f(m[e].nf), 0.0f);
    }
}

// record of column c: the fold of its band partials (finite min, finite max,
// max |x| bits); with at most kWaves * kFoldU bands a thread loads all of its
// partials in one round
__global__ __launch_bounds__(kB) void k_cols_fold(const float4* __restrict__ part, int64_t nbands, int64_t cols,
                                                  float4* __restrict__ rec) {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int64_t c = (int64_t)blockIdx.x * kWave + lane;
    MinMax m;
    if (c < cols) {
        for (int64_t b = w; b < nbands; b += kWaves * kFoldU) {
            float4 p[kFoldU];
#pragma unroll
            for (int u = 0; u < kFoldU; ++u) {
                const int64_t bb = b + u * kWaves;
                p[u] = part[(bb < nbands ? bb : b) * cols + c];
            }
#pragma unroll
            for (int u = 0; u < kFoldU; ++u) m.merge(p[u].x, p[u].y, as_u(p[u].z));
        }
    }
    __shared__ float4 s[kWaves - 1][kWave];
    if (w > 0) s[w - 1][lane] = make_float4(m.mn, m.mx, as_f(m.nf), 0.0f);
    __syncthreads();
    if (w != 0 || c >= cols) return;
    for (int k = 0; k < kWaves - 1; ++k) m.merge(s[k][lane].x, s[k][lane].y, as_u(s[k][lane].z));
    rec[c] = make_float4(m.mn, m.mx, as_f(m.nf), 0.0f);
}

// column record: (scale, reciprocal, zero-point bits, mode | kColFinite), mode
// 0 zero scale, 1 divisor in the exact-quotient window, 2 true division;
// kColFinite: the column holds no Inf or NaN
constexpr uint32_t kColFinite = 4u;

// code offset q - zp of x for one column's record (the per-element rule of
// IntQ::offset: zero scale -> code 0, NaN -> code 0, +-Inf clamp, -0 -> +0)
__device__ __forceinline__ float col_offset(float x, const float4& cp, float lo, float hi) {
    const uint32_t mode = as_u(cp.w) & 3u;
    const float zpf = (float)(-(int32_t)as_u(cp.z));
    if (mode == 0u) return zpf;
    const float t = mode == 1u ? ExactDiv(cp.x, cp.y).quick(x) : x / cp.x;  // +-Inf / NaN safe
    const float r = fminf(fmaxf(rintf(t), lo), hi) + 0.0f;
    return (t != t) ? zpf : r;
}

// codes and fake-quant values of the N columns from c0 of row r
template <int N, int BITS, bool AL>
__device__ __forceinline__ void store_row(const int (&code)[N], const float (&o)[N], int64_t r, int64_t cols,
                                          int64_t c0, int64_t pstride, uint8_t* __restrict__ codes,
                                          float* __restrict__ fq) {
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
        return;
    }
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

// Four columns per lane for either dtype, so that every store instruction of a
// wave writes one contiguous run (1 KB of fake-quant values, 256 or 128 bytes of
// codes); a bf16 row is read 8 bytes per lane.
template <int DT, int BITS, bool AL>
__global__ __launch_bounds__(kB) void k_cols_quant(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                   int affine, const float4* __restrict__ rec,
                                                   uint8_t* __restrict__ codes, float* __restrict__ fq,
                                                   float* __restrict__ scale, int32_t* __restrict__ zp,
                                                   uint32_t* __restrict__ flags) {
    constexpr int N = kQuantVec;
    constexpr int TC = kWave * N;  // columns of the tile
    __shared__ float4 s_par[TC];
    const int64_t ct0 = (int64_t)blockIdx.x * TC;
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int64_t c0 = ct0 + (int64_t)lane * N;
    const bool in = c0 < cols;
    // the first band's rows are loaded before the column parameters are derived
    // (they do not depend on them), so the loads overlap that work
    int64_t band = blockIdx.y;
    int64_t r0 = band * kQuantRows;
    int64_t r1 = r0 + kQuantRows < rows ? r0 + kQuantRows : rows;
    float v[kU][N];
    auto load_band = [&]() {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t rr = r0 + w + u * kWaves;
            load_cols<DT, N, AL>(x, rr < r1 ? rr : r1 - 1, cols, c0, v[u]);  // past the band: its last row again
        }
    };
    if (in) load_band();
    const IntRange rg = int_range(BITS, affine != 0);
    for (int j = threadIdx.x; j < TC; j += kB) {
        const int64_t c = ct0 + j;
        if (c >= cols) {
            s_par[j] = make_float4(1.0f, 1.0f, 0.0f, as_f(1u | kColFinite));  // unused; keeps the fast test true
            continue;
        }
        const float4 k = rec[c];
        const IntCal cal = calibrate(k.x, k.y, rg, affine != 0);
        const ExactDiv d(cal.scale == 0.0f ? 1.0f : cal.scale);
        const uint32_t mode = (cal.scale == 0.0f ? 0u : (d.fast ? 1u : 2u)) |
                              (as_u(k.z) < 0x7F800000u ? kColFinite : 0u);
        s_par[j] = make_float4(cal.scale, d.y, as_f((uint32_t)cal.zp), as_f(mode));
        if (blockIdx.y == 0) {
            scale[c] = cal.scale;
            zp[c] = cal.zp;
            const uint32_t f = (as_u(k.z) >= 0x7F800000u ? FQ_FLAG_NONFINITE : 0u) |
                               (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
            if (flags && f) atomicOr(flags, f);
        }
    }
    __syncthreads();
    if (!in) return;
    float4 cp[N];
    float lo[N], hi[N];
    int zpv[N];
    bool lane_fast = true;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        cp[e] = s_par[lane * N + e];
        zpv[e] = (int)as_u(cp[e].z);
        lo[e] = (float)(rg.qmin - zpv[e]);
        hi[e] = (float)(rg.qmax - zpv[e]);
        lane_fast = lane_fast && as_u(cp[e].w) == (1u | kColFinite);
    }
    // every column of the wave finite with a divisor in the exact-quotient
    // window: the bare quotient, a clamp, and the round-to-even of the magic-number
    // add, whose low bits plus the zero-point are the code (the rule of col_offset
    // for finite x, without its NaN / Inf fix-ups)
    const bool fast = __all(lane_fast);
    const int64_t pstride = BITS == 8 ? cols : (cols + 1) / 2;
    for (;;) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t r = r0 + w + u * kWaves;
            if (r >= r1) break;
            int code[N];
            float o[N];
            if (fast) {
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    const float f = __builtin_amdgcn_fmed3f(quick_div(v[u][e], cp[e].x, cp[e].y), lo[e], hi[e]) + kMagic;
                    code[e] = (int)(as_u(f) + (uint32_t)zpv[e]);
                    o[e] = (f - kMagic) * cp[e].x;
                }
            } else {
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    o[e] = col_offset(v[u][e], cp[e], lo[e], hi[e]);
                    code[e] = (int)o[e] + zpv[e];
                    o[e] *= cp[e].x;
                }
            }
            store_row<N, BITS, AL>(code, o, r, cols, c0, pstride, codes, fq);
        }
        band += gridDim.y;
        if (band * kQuantRows >= rows) break;
        r0 = band * kQuantRows;
        r1 = r0 + kQuantRows < rows ? r0 + kQuantRows : rows;
        load_band();
    }
}

// ---------------------------------------------------------------------------
// One-pass per-column path for tensors of at most kStripRows rows whose column
// count is a multiple of the strip width: a 1024-thread workgroup owns a strip of
// columns whose row segment is 64 bytes (16 fp32 or 32 bf16 columns) over all
// rows and keeps it in registers (64 VGPRs of x per thread), so x is read once
// and the strip's column statistics never leave the compute unit.  Every lane
// holds four columns of a row: lane % L picks the lane's piece of the row
// segment (L = 4 pieces of 16 bytes for fp32, 8 of 8 bytes for bf16), lane / L
// + (64 / L) * wave the row, so a load instruction covers 64 / L rows and a
// thread holds every (1024 / L)-th row (16 rows for fp32, 32 for bf16).  Column
// min / max: per thread, across the lanes of a wave that share a piece
// (shuffles), across the waves (LDS); one thread per column then derives the
// parameters.  Adjacent strips share 128-byte lines of x (and of the codes), so
// the strips go to the XCDs (workgroups go to the eight XCDs in turn) in groups
// of eight adjacent strips, whose shared lines one L2 then merges, and each XCD
// takes groups from the whole width of the rows.  Cold (warm), interleaved, three
// rounds on one box: fp32 [4096, 4096] int8 34.6-34.9 (28.6) us with groups of
// eight, 35.2-35.4 (31.5) with a contiguous run of strips per XCD, 36.4-37.0
// (29.9) with groups of four; bf16 [4096, 8192] int8 45.3-45.9 (38.8) with eight,
// 47.2-47.4 (43.7) with a contiguous run, 47.1-48.3 (40.6) with four.  Groups of
// two and of sixteen timed slower on another box.  The kernel this replaced (the
// same layout for fp32 only, with a contiguous run per XCD and loads the
// compiler had serialized two at a time) took 36.0-36.7 (33.0) us; the
// three-launch path takes 46 us for that fp32 tensor and 57.8 (54.5) us for the
// bf16 one, which it reads twice.  Per-workgroup clocks at [4096, 4096] fp32: 222
// strips finish their loads in 10.7-11.5 us, but the strips whose row segment has
// address bits 9:7 = 011 need 16-17 us even when no other strip loads, whatever
// the order, load depth or cache policy; the kernel ends 6-7 us after them.
// ---------------------------------------------------------------------------
constexpr int kStripThreads = 1024;
constexpr int kStripWaves = kStripThreads / kWave;  // 16
constexpr int64_t kStripRows = 4096;                // rows a strip holds
constexpr int kXcds = 8;
constexpr int kStripGroup = 8;  // adjacent strips dealt to one XCD at a time

template <int DT>
struct Strip {
    static constexpr int L = DT == FQ_F32 ? 4 : 8;             // lanes per 64-byte row segment
    static constexpr int C = 4 * L;                            // columns of the strip
    static constexpr int RPL = kStripThreads / L;              // rows per load instruction of the workgroup
    static constexpr int LOADS = (int)(kStripRows / RPL);      // row pieces per thread
    // loads issued per group before their min / max (cold, [4096, 4096] fp32 int8:
    // 35.9-36.3 us with 2, 37.0-37.1 with 4, 38.6 with 8, 38.3-38.9 with all 16;
    // [4096, 8192] bf16: 47.4-48.8 us with 4 or 8, 48.5-49.8 with 16 or 32)
    static constexpr int DEPTH = DT == FQ_F32 ? 2 : 8;
    // the raw 16 (fp32) or 8 (bf16) bytes of a lane's four columns
    typedef uint32_t Piece __attribute__((ext_vector_type(DT == FQ_F32 ? 4 : 2)));
    static_assert(LOADS * (int)sizeof(Piece) == 256, "64 VGPRs of x per thread");
};

// p as a wave-uniform (scalar) address: the readfirstlanes stop the compiler from
// folding a lane offset into it, so base + lane offset becomes one load or store
// with a scalar base and a 32-bit lane offset
// (a global-memory pointer, so that the accesses stay global rather than flat)
#define FQ_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ FQ_GLOBAL char* uniform_base(const void* p) {
    const uint64_t a = (uint64_t)p;
    // readfirstlane returns an int: both halves go back through uint32_t
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    return (FQ_GLOBAL char*)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// column e (0..3) of a lane's piece
template <int DT>
__device__ __forceinline__ float piece_col(const typename Strip<DT>::Piece& p, int e) {
    if constexpr (DT == FQ_F32) {
        return as_f(p[e]);
    } else {
        return (e & 1) ? bf16_hi(p[e >> 1]) : bf16_lo(p[e >> 1]);
    }
}

template <int DT, int BITS>
__global__ __launch_bounds__(kStripThreads) void k_cols_strip(const void* __restrict__ x, int64_t rows,
                                                              int64_t cols, int affine,
                                                              uint8_t* __restrict__ codes, float* __restrict__ fq,
                                                              float* __restrict__ scale, int32_t* __restrict__ zp,
                                                              uint32_t* __restrict__ flags) {
    using S = Strip<DT>;
    using Piece = typename S::Piece;
    // rows * cols < 2^31 and RPL <= rows on this path.  Load j covers the RPL
    // rows from br(j) = min(j RPL, rows - RPL): a wave-uniform base address plus
    // one 32-bit lane offset that is the same for every j.  A block clamped at
    // the end loads some rows a second time, which leaves min / max unchanged;
    // the store phase skips them.
    const int t = threadIdx.x, lane = t % kWave, w = t / kWave;
    const int vq = lane % S::L;  // piece of the row segment
    const uint32_t nstrips = (uint32_t)(cols / S::C), ncols = (uint32_t)cols, nrows = (uint32_t)rows;
    const uint32_t b = blockIdx.x;
    // groups of kStripGroup adjacent strips go to the XCDs in turn (else a
    // contiguous run per XCD, else strip b on workgroup b)
    constexpr uint32_t Q = kStripGroup;
    const uint32_t strip = nstrips % (kXcds * Q) == 0 ? ((b / kXcds) / Q * kXcds + b % kXcds) * Q + (b / kXcds) % Q
                           : nstrips % kXcds == 0     ? (b % kXcds) * (nstrips / kXcds) + b / kXcds
                                                      : b;
    const uint32_t c0 = strip * S::C + vq * 4;
    const uint32_t rbase = (uint32_t)w * (kWave / S::L) + (uint32_t)lane / S::L;
    const uint32_t lane_el = rbase * ncols + c0;  // element offset of the lane in a block of rows
    auto block_row = [&](int j) { return min((uint32_t)j * S::RPL, nrows - S::RPL); };

    constexpr uint32_t ES = sizeof(Piece) / 4;  // bytes per element
    Piece v[S::LOADS];
    MinMax m[4];
#pragma unroll
    for (int g = 0; g < S::LOADS; g += S::DEPTH) {
#pragma unroll
        for (int j = g; j < g + S::DEPTH; ++j) {
            const FQ_GLOBAL char* xb =
                uniform_base(reinterpret_cast<const char*>(x) + (size_t)block_row(j) * ncols * ES);
            v[j] = *reinterpret_cast<const FQ_GLOBAL Piece*>(xb + lane_el * ES);
        }
#pragma unroll
        for (int j = g; j < g + S::DEPTH; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) m[e].add(piece_col<DT>(v[j], e));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int k = S::L; k < kWave; k <<= 1) {
            m[e].merge(__shfl_xor(m[e].mn, k), __shfl_xor(m[e].mx, k), (uint32_t)__shfl_xor((int)m[e].nf, k));
        }
    }
    __shared__ float s_mn[kStripWaves][S::C], s_mx[kStripWaves][S::C];
    __shared__ uint32_t s_nf[kStripWaves][S::C];
    __shared__ float4 s_par[S::C];
    if (lane < S::L) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s_mn[w][vq * 4 + e] = m[e].mn;
            s_mx[w][vq * 4 + e] = m[e].mx;
            s_nf[w][vq * 4 + e] = m[e].nf;
        }
    }
    __syncthreads();
    const IntRange rg = int_range(BITS, affine != 0);
    if (t < S::C) {
        MinMax a;
        for (int k = 0; k < kStripWaves; ++k) a.merge(s_mn[k][t], s_mx[k][t], s_nf[k][t]);
        const IntCal cal = calibrate(a.mn, a.mx, rg, affine != 0);
        const ExactDiv d(cal.scale == 0.0f ? 1.0f : cal.scale);
        const uint32_t mode = (cal.scale == 0.0f ? 0u : (d.fast ? 1u : 2u)) | (a.nonfinite() ? 0u : kColFinite);
        s_par[t] = make_float4(cal.scale, d.y, as_f((uint32_t)cal.zp), as_f(mode));
        const uint32_t c = strip * S::C + t;
        scale[c] = cal.scale;
        zp[c] = cal.zp;
        const uint32_t f = (a.nonfinite() ? FQ_FLAG_NONFINITE : 0u) | (cal.degenerate ? FQ_FLAG_DEGENERATE : 0u);
        if (flags && f) atomicOr(flags, f);
    }
    __syncthreads();
    float4 cp[4];
    float lo[4], hi[4];
    int zpv[4];
    bool lane_fast = true;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        cp[e] = s_par[vq * 4 + e];
        zpv[e] = (int)as_u(cp[e].z);
        lo[e] = (float)(rg.qmin - zpv[e]);
        hi[e] = (float)(rg.qmax - zpv[e]);
        lane_fast = lane_fast && as_u(cp[e].w) == (1u | kColFinite);
    }
    // as k_cols_quant: a wave whose columns are all finite with divisors in the
    // exact-quotient window takes the bare quotient, clamp and magic rounding
    const bool fast = __all(lane_fast);
    if constexpr (DT == FQ_BF16) {
        // unpack x again below rather than keep the statistics phase's unpacked
        // copy (twice the registers of the packed pieces)
#pragma unroll
        for (int j = 0; j < S::LOADS; ++j) asm volatile("" : "+v"(v[j]));
    }
    const uint32_t pstride = BITS == 8 ? ncols : ncols / 2;
    const uint32_t lane_code = rbase * pstride + (BITS == 8 ? c0 : c0 / 2);  // byte offset, as lane_el
#pragma unroll
    for (int j = 0; j < S::LOADS; ++j) {
        const uint32_t br = block_row(j);
        if (br + rbase < (uint32_t)j * S::RPL) continue;  // a row an earlier j stored
        float xv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[e] = piece_col<DT>(v[j], e);
        int code[4];
        float o[4];
        if (fast) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = __builtin_amdgcn_fmed3f(quick_div(xv[e], cp[e].x, cp[e].y), lo[e], hi[e]) + kMagic;
                code[e] = (int)(as_u(f) + (uint32_t)zpv[e]);
                o[e] = (f - kMagic) * cp[e].x;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[e] = col_offset(xv[e], cp[e], lo[e], hi[e]);
                code[e] = (int)o[e] + zpv[e];
                o[e] *= cp[e].x;
            }
        }
        // fake-quant values with plain stores: for fp32 the two halves of a
        // 128-byte line come from adjacent strips on the same XCD and merge in its L2
        if (codes) {
            FQ_GLOBAL char* cb = uniform_base(codes + (size_t)br * pstride) + lane_code;
            if (BITS == 8)
                *reinterpret_cast<FQ_GLOBAL uint32_t*>(cb) = pack4(code[0], code[1], code[2], code[3]);
            else
                *reinterpret_cast<FQ_GLOBAL uint16_t*>(cb) =
                    (uint16_t)(nib2(code[0], code[1]) | (nib2(code[2], code[3]) << 8));
        }
        if (fq)
            *reinterpret_cast<FQ_GLOBAL f32x4*>(uniform_base(fq + (size_t)br * ncols) + lane_el * 4u) =
                f32x4{o[0], o[1], o[2], o[3]};
    }
}

template <int DT, int BITS>
int launch_cols(const void* x, int64_t rows, int64_t cols, int affine, void* ws, uint8_t* codes, float* fq,
                float* scale, int32_t* zp, uint32_t* flags, hipStream_t st) {
    constexpr int N = ColVec<DT>::N;
    const int64_t nb = minmax_bands(rows);
    const int64_t rpb = (rows + nb - 1) / nb;
    float4* part = reinterpret_cast<float4*>(ws);
    float4* rec = part + nb * cols;
    // min / max pass: 16-byte vectors of N columns; quantize pass: four columns
    // (16 bytes of fp32 or 8 of bf16), codes 4 (int8) or 2 (int4) bytes per lane
    const bool al = (cols % N == 0) && fqh::aligned(x, 16);
    const bool alq = (cols % kQuantVec == 0) && fqh::aligned(x, DT == FQ_F32 ? 16 : 8) && fqh::aligned(fq, 16) &&
                     fqh::aligned(codes, BITS == 8 ? 4 : 2);
    const int64_t tiles = (cols + kWave * N - 1) / (kWave * N);
    const int64_t qtiles = (cols + kWave * kQuantVec - 1) / (kWave * kQuantVec);
    if (qtiles > 0x7FFFFFFF) return FQ_E_INVALID;
    constexpr int SC = Strip<DT>::C;
    static_assert(Strip<DT>::RPL <= kStripRows / 4, "a strip's rows fill a block of RPL rows");
    if (alq && rows > kStripRows / 4 && rows <= kStripRows && cols % SC == 0 && cols / SC >= fqh::num_cus() / 2 &&
        rows * cols <= 0x7FFFFFFF) {
        k_cols_strip<DT, BITS><<<(unsigned)(cols / SC), kStripThreads, 0, st>>>(x, rows, cols, affine, codes, fq,
                                                                                scale, zp, flags);
        return fqh::launched();
    }
    const dim3 g1((unsigned)tiles, (unsigned)nb);
    if (al) k_cols_minmax<DT, true><<<g1, kB, 0, st>>>(x, rows, cols, rpb, part);
    else k_cols_minmax<DT, false><<<g1, kB, 0, st>>>(x, rows, cols, rpb, part);
    k_cols_fold<<<(unsigned)((cols + kWave - 1) / kWave), kB, 0, st>>>(part, nb, cols, rec);
    int64_t qb = (rows + kQuantRows - 1) / kQuantRows;
    qb = qb < kMaxQuantBands ? qb : kMaxQuantBands;
    const dim3 g2((unsigned)qtiles, (unsigned)qb);
    if (alq) k_cols_quant<DT, BITS, true><<<g2, kB, 0, st>>>(x, rows, cols, affine, rec, codes, fq, scale, zp, flags);
    else k_cols_quant<DT, BITS, false><<<g2, kB, 0, st>>>(x, rows, cols, affine, rec, codes, fq, scale, zp, flags);
    return fqh::launched();
}

}  // namespace

extern "C" {

size_t fq_cols_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows < 1 || cols < 1) return 0;
    return (size_t)((minmax_bands(rows) + 1) * cols * 16);
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
