// fq_host.h -- host-side helpers of the C ABI: argument checks, launch geometry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fq.h"

namespace fqh {

constexpr int kBlock = 256;  // threads per workgroup (four wave64)

inline bool aligned(const void* p, uintptr_t a) { return p == nullptr || ((uintptr_t)p % a) == 0; }

inline bool valid_bits(int bits) { return bits == 4 || bits == 8; }
inline bool valid_scheme(int s) { return s == FQ_SYM || s == FQ_AFFINE; }
inline bool valid_fmt(int f) { return f == FQ_E4M3 || f == FQ_E5M2; }
inline bool valid_dtype(int d) { return d == FQ_F32 || d == FQ_BF16; }

constexpr int kMaxDevices = 64;  // per-device caches; ids beyond share slot 0

// Compute units of the current device (cached per device id).
int num_cus();
// LDS bytes per compute unit / largest LDS allocation of one workgroup.
int lds_per_cu();
int lds_per_block();

// Dynamic LDS bytes that keep at most `wgs` workgroups of a kernel resident on a
// compute unit (0: no cap).  The streaming kernels here move more bytes per
// second with fewer workgroups in flight than the wave slots allow: the HBM then
// sees a narrower window of addresses at a time.  The allocation sits midway
// between LDS/(wgs + 1) and LDS/wgs, so the kernel's own static LDS (at most
// `static_bytes`, which must stay below the margin) and the allocation
// granularity cannot move it out of that window; if the device cannot express
// the cap the kernel runs uncapped.
inline size_t lds_cap(int wgs, int static_bytes) {
    if (wgs <= 0) return 0;
    const int64_t C = lds_per_cu();
    const int64_t lo = C / (wgs + 1), hi = C / wgs;
    int64_t mid = (lo + hi) / 2 / 256 * 256;
    if (mid + static_bytes + 2048 > hi || mid <= lo + static_bytes) return 0;
    int64_t pad = mid - static_bytes;
    if (pad + static_bytes > lds_per_block()) return 0;
    return (size_t)pad;
}

// Status of the launch(es) just enqueued.
inline int launched() { return hipGetLastError() == hipSuccess ? FQ_OK : FQ_E_HIP; }

// Blocks for a grid-stride loop over `items` work items, `per_block` items per
// block per pass, at most `waves_per_cu` resident blocks per compute unit.
inline unsigned grid_for(int64_t items, int64_t per_block, int blocks_per_cu) {
    int64_t want = (items + per_block - 1) / per_block;
    int64_t cap = (int64_t)num_cus() * blocks_per_cu;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    return (unsigned)want;
}

// One work item per thread over the whole index space: on MI355X many short
// workgroups that sweep memory in order stream faster than a capped grid with a
// grid-stride loop.  Grids beyond 2^31 - 1 blocks fall back to the kernels'
// grid-stride loop.
inline unsigned grid_all(int64_t items, int64_t per_block) {
    int64_t want = (items + per_block - 1) / per_block;
    if (want > 0x7FFFFFFF) want = 0x7FFFFFFF;
    if (want < 1) want = 1;
    return (unsigned)want;
}

// Tensor-scope reduction: the tensor is cut into tiles of kReduceTile
// consecutive 16-byte chunks (four per thread of a kReduceThreads block); block b
// reduces tiles b, b + G, ... into one partial in the workspace, with G at most
// kMaxReduceBlocks.
#ifndef FQ_REDUCE_THREADS
#define FQ_REDUCE_THREADS 512
#endif
#ifndef FQ_REDUCE_CHUNKS
#define FQ_REDUCE_CHUNKS 4
#endif
#ifndef FQ_REDUCE_MAX_BLOCKS
#define FQ_REDUCE_MAX_BLOCKS 16384
#endif
constexpr int kReduceThreads = FQ_REDUCE_THREADS;
constexpr int kReduceChunks = FQ_REDUCE_CHUNKS;
constexpr int64_t kReduceTile = (int64_t)kReduceChunks * kReduceThreads;
constexpr int64_t kMaxReduceBlocks = FQ_REDUCE_MAX_BLOCKS;
constexpr int kFinalThreads = 1024;
inline unsigned reduce_blocks(int64_t n) {
    int64_t chunks = (n + 3) / 4;
    int64_t want = (chunks + kReduceTile - 1) / kReduceTile;
    if (want > kMaxReduceBlocks) want = kMaxReduceBlocks;
    if (want < 1) want = 1;
    return (unsigned)want;
}

// Tensors with at most this many reduction partials take the two-launch
// calibration + fake-quant (every block of the second launch folds them all).
constexpr int64_t kFoldMaxParts = 512;

// Pass 2 of the tensor-scope min / max over `nparts` partial records (float4:
// finite min, finite max, max |x| bits, -) that a fused kernel left in the
// workspace: derives the integer parameters on the device ([QAT] from_minmax,
// real_min / real_max) and ORs NONFINITE / DEGENERATE into flags.
int params_from_partials(const void* workspace, unsigned nparts, int bits, int scheme, fq_int_params* params,
                         uint32_t* flags, hipStream_t stream);

// Fake-quant of x[n] (16-byte aligned operands, at most kFoldGsMaxParts
// partials) whose parameters every block derives itself from the `nparts`
// partial records in the workspace (block 0 stores them and the flags): one
// launch in place of params_from_partials + fq_fake_quant_int_tensor, which it
// falls back to otherwise.  Measured on the 2^24-element QAT step (update pass
// capped at this many workgroups): 512 partials and 16 workgroups per CU ran the
// step in 99.3-100.6 us cold against 101.4-102.9 for three launches (two boxes,
// interleaved runs); 2048 partials 104.8-105.9, 256 partials 112.9-114.6 (an
// update pass of one workgroup per CU), 8 workgroups per CU 101.6-101.8.
constexpr int kFoldGsMaxParts = 512;
constexpr int kFoldGsBlocksPerCu = 16;
int fake_quant_from_partials(const float* x, int64_t n, int bits, int scheme, const void* workspace, unsigned nparts,
                             fq_int_params* params, void* codes, float* fq, uint32_t* flags, hipStream_t stream);

// Finite amax of x[n] (float32; 0 when no element is finite), left as binary32
// bits in word 0 of the workspace (fq_workspace_bytes(n) bytes) by two launches.
int tensor_amax(const float* x, int64_t n, void* workspace, hipStream_t stream);

}  // namespace fqh
