/*
 * fq.h -- C ABI of libfq.so: fake quantization (quantize / dequantize /
 * fake-quant) of tensors on AMD Instinct MI355X (gfx950).
 *
 * Every entry point enqueues hand-written HIP kernels on the caller's stream and
 * returns at once; nothing here allocates device memory or synchronises.
 *
 * Conventions shared by all entry points
 *   - Tensor arguments are DEVICE pointers owned by the caller.  Inputs are read
 *     only; outputs must not overlap inputs or each other.  Any alignment is
 *     accepted (16-byte aligned buffers take the vector path).
 *   - Layouts are dense row-major; sizes are element counts.
 *   - Arithmetic is IEEE binary32 with one rounding per operation, true division
 *     where the method divides, round-half-to-even for codes (round-half-away for
 *     the 8-bit double-quant scale codes).
 *   - Argument errors are returned synchronously, before anything is enqueued:
 *       FQ_E_INVALID      null / empty / too-small argument (the pages' InvalidState
 *                         for arguments: empty tensors cannot be calibrated),
 *       FQ_E_UNSUPPORTED  width other than 4 or 8, unknown scheme / format / dtype
 *                         (the pages' UnsupportedOperation),
 *       FQ_E_DIM          two lengths that must agree do not (DimensionMismatch),
 *       FQ_E_HIP          the HIP launch itself failed.
 *   - Data-dependent conditions are NOT errors: kernels OR FQ_FLAG_* bits into
 *     an optional device uint32_t (`flags`, may be NULL) which the caller zeroes;
 *     the library never clears it.  NONFINITE: a calibration group held Inf or
 *     NaN (it is then calibrated on its finite elements).  DEGENERATE: a group
 *     had no usable range (all zero); its scale and zero-point are 0, its codes 0
 *     and its fake-quant values +0.
 *   - Non-finite inputs: NaN quantizes to integer code 0 and to the fp8 NaN byte
 *     0x7F; +-Inf clamps to the range ends / saturates to +-max-normal.
 *
 * Sources, by page title and section:
 *   [QAT] optirs-gpu 0.3.2 src/optirs_gpu/quantization.rs, "Quantization-Aware
 *         Training (QAT) primitives" (module docs; QuantParams; fake_quant_int;
 *         per_channel_params; fake_quant_fp8; fake_quant_backward).
 *   [DQ]  aprender-train 0.32.0 entrenar/quant/double_quant.rs, "Double
 *         quantization for QLoRA" (quantize_4bit_double, dequantize_4bit_double).
 *   [CS]  CS349E 05_quantization_basics.py, demo 4 `block_scaled` ("e8m0").
 *   [MAR] ferrum-kernels 0.8.0 marlin_repack.rs (zero scale gives fp8 byte 0).
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FQ_ABI_VERSION 1

/* status codes (return values) */
#define FQ_OK 0
#define FQ_E_INVALID (-1)
#define FQ_E_UNSUPPORTED (-2)
#define FQ_E_DIM (-3)
#define FQ_E_HIP (-4)

/* data-dependent flag bits (OR-ed into *flags on the device) */
#define FQ_FLAG_NONFINITE 1u
#define FQ_FLAG_DEGENERATE 2u

/* [QAT] QuantScheme: symmetric (zero-point 0, restricted range -127..127 / -7..7)
 * or affine (full range -128..127 / -8..7, zero-point nudged so 0 is exact). */
enum { FQ_SYM = 0, FQ_AFFINE = 1 };
/* [QAT] Fp8Format, and the FP4 / FP6 element formats of [CS] demo 4 (every code
 * finite: E2M1 max 6, E2M3 max 7.5, E3M2 max 28) */
enum { FQ_E4M3 = 0, FQ_E5M2 = 1, FQ_E2M1 = 2, FQ_E2M3 = 3, FQ_E3M2 = 4 };
/* element type of an input tensor */
enum { FQ_F32 = 0, FQ_BF16 = 1 };

/* Per-tensor integer parameters as they sit in device memory (16 bytes).
 * scale, zero_point: [QAT] QuantParams; real_min / real_max: [QAT]
 * QuantParams::real_min / real_max = dequant(qmin) / dequant(qmax), the STE
 * window.  &p->real_min is a valid `bounds` argument of fq_ste_backward. */
typedef struct fq_int_params {
    float scale;
    int32_t zero_point;
    float real_min;
    float real_max;
} fq_int_params;

/* ABI version (FQ_ABI_VERSION) and a static string naming a status code. */
int fq_version(void);
const char* fq_status_string(int status);

/* Bytes of device workspace that fq_tensor_params_int / fq_fp8_tensor_scale
 * need for a tensor of n elements (partial results of the grid reduction).  The
 * workspace is scratch owned by the caller; its contents need no initialisation
 * and are meaningless afterwards.  Host-only; 0 for n < 1. */
size_t fq_workspace_bytes(int64_t n);

/* Sizes of the double-quantized 4-bit representation of n values ([DQ]
 * DoubleQuantized4Bit): packed data ceil(n/2) bytes, one u8 scale per 64-element
 * block (ceil(n/64)), one fp32 super-scale per 256 blocks.  Host-only; returns
 * FQ_E_INVALID for n < 1 or a NULL output pointer. */
int fq_q4dq_sizes(int64_t n, int64_t* packed_bytes, int64_t* num_blocks, int64_t* num_super);

/* Per-tensor calibration ([QAT] QuantParams::per_tensor_minmax then real_min /
 * real_max): min and max over the finite elements of x[n] (float32), then
 *   symmetric: scale = absmax / qmax, zero_point = 0;
 *   affine:    rmin = min(min, 0), rmax = max(max, 0),
 *              scale = (rmax - rmin) / (qmax - qmin),
 *              zero_point = clamp(RNE(qmin - rmin / scale), qmin, qmax).
 * Writes one fq_int_params to `params` (device).  `bits` in {4, 8}; `scheme`
 * FQ_SYM or FQ_AFFINE.  `workspace` of at least fq_workspace_bytes(n) bytes
 * (workspace_bytes says how many the caller gives).  Two kernel launches. */
int fq_tensor_params_int(const float* x, int64_t n, int bits, int scheme, void* workspace,
                         size_t workspace_bytes, fq_int_params* params, uint32_t* flags,
                         hipStream_t stream);

/* Per-tensor integer quantize / fake-quant ([QAT] module docs "Integer
 * quantization", fake_quant_int): q = clamp(RNE(x / scale) + zero_point, qmin,
 * qmax) (rounded first, zero-point added as an integer), fq = (q - zero_point) *
 * scale.  params: device fq_int_params (e.g. from fq_tensor_params_int).
 * codes (may be NULL): bits = 8 -> int8 [n]; bits = 4 -> two codes per byte,
 * ceil(n/2) bytes, element i in byte i/2, even i in the high nibble (the nibble
 * order of [DQ] dequantize_4bit_double).  fq (may be NULL): float32 [n].  At
 * least one of codes / fq.  scale == 0 gives codes 0 and fq +0. */
int fq_fake_quant_int_tensor(const float* x, int64_t n, int bits, int scheme,
                             const fq_int_params* params, void* codes, float* fq,
                             hipStream_t stream);

/* Per-tensor calibration followed by fake-quant ([QAT] per_tensor_minmax,
 * from_minmax, fake_quant_int): the results of fq_tensor_params_int followed by
 * fq_fake_quant_int_tensor on the same arguments, bit for bit -- params, codes,
 * fq and flags as those two calls define them.  Tensors of up to 2^22 elements
 * with 16-byte aligned x / fq and 4-byte (int8) or 2-byte (int4) aligned codes
 * take two launches instead of three: the reduction's first pass, then a
 * fake-quant pass whose every block folds the partials and derives the
 * parameters itself.  Others make the two calls.  `workspace` of at least
 * fq_workspace_bytes(n) bytes, as for fq_tensor_params_int. */
int fq_calibrate_fake_quant_int_tensor(const float* x, int64_t n, int bits, int scheme, void* workspace,
                                      size_t workspace_bytes, fq_int_params* params, void* codes, float* fq,
                                      uint32_t* flags, hipStream_t stream);

/* fq_calibrate_fake_quant_int_tensor without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments minus
 * workspace / workspace_bytes; same results, bit for bit, and the same launches.
 * The reduction partials go to a static device array inside libfq.so of
 * FQ_NOALLOC_SCRATCH_BYTES (256 KiB) that each GPU holds from module load until
 * the process ends; every n >= 1 fits in it (the first pass never makes more
 * than 16384 partials), and a tensor that needed more would be refused with
 * FQ_E_INVALID.  The call allocates nothing and calls no allocating routine.
 * Its first call on a device looks the array's device address up
 * (hipGetSymbolAddress) and keeps it; a caller about to capture a graph makes
 * one call before capturing.  FQ_E_HIP if the lookup fails or the device id is
 * 64 or more.  All calls on one GPU share that GPU's array: calls that may
 * overlap on one GPU (several streams, several host threads) race on it and
 * must be serialised by the caller.  Nothing in the array needs to start at
 * zero: every launch writes the partials it later reads. */
#define FQ_NOALLOC_SCRATCH_BYTES (256u * 1024u)
int fq_calibrate_fake_quant_int_tensor_noalloc(const float* x, int64_t n, int bits, int scheme,
                                               fq_int_params* params, void* codes, float* fq, uint32_t* flags,
                                               hipStream_t stream);

/* [QAT] dequant(q) = (q - zero_point) * scale over stored codes (layout as
 * fq_fake_quant_int_tensor's `codes`). */
int fq_dequantize_int_tensor(const void* codes, int64_t n, int bits, const fq_int_params* params,
                             float* out, hipStream_t stream);

/* [QAT] fake_quant_backward (straight-through estimator): grad_in[i] = grad[i]
 * if lo <= x[i] <= hi, else +0, with (lo, hi) the two device floats at `bounds`
 * taken in either order.  n_grad must equal n_x (else FQ_E_DIM). */
int fq_ste_backward(const float* grad, int64_t n_grad, const float* x, int64_t n_x,
                    const float* bounds, float* grad_in, hipStream_t stream);

/* Per-row (per-channel along axis 0 / per-token) fused calibration + quantize
 * ([QAT] per_channel_params + fake_quant_int_per_channel, axis 0): every row of
 * x[rows, cols] (dtype FQ_F32 or FQ_BF16, widened exactly) gets its own scale and
 * zero-point from its finite min / max, as in fq_tensor_params_int, and is
 * quantized with them in the same launch (one read of x).
 * codes (may be NULL): bits = 8 -> int8 [rows, cols]; bits = 4 -> packed,
 *   ceil(cols/2) bytes per row, element j of a row in byte j/2, even j high
 *   nibble, an odd row tail leaves the low nibble 0.
 * fq (may be NULL): float32 [rows, cols].  scale: float32 [rows];
 * zero_point: int32 [rows] (both required). */
int fq_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols, int bits, int scheme,
                  void* codes, float* fq, float* scale, int32_t* zero_point, uint32_t* flags,
                  hipStream_t stream);

/* Per-row dequantize of codes stored as fq_quant_rows writes them. */
int fq_dequantize_rows(const void* codes, int64_t rows, int64_t cols, int bits, const float* scale,
                       const int32_t* zero_point, float* out, hipStream_t stream);

/* Per-tensor fp8 scale: amax over the finite elements of x[n] (Inf and NaN are
 * skipped), scale = amax / max-normal (448 for E4M3, 57344 for E5M2; [QAT]
 * Fp8Format, [MAR] absmax / 448).  Either of scale_e4m3 / scale_e5m2 (device
 * float, may be NULL, not both) is written from one pass over x.  A zero scale
 * sets FQ_FLAG_DEGENERATE.  `workspace` as for fq_tensor_params_int. */
int fq_fp8_tensor_scale(const float* x, int64_t n, void* workspace, size_t workspace_bytes,
                        float* scale_e4m3, float* scale_e5m2, uint32_t* flags, hipStream_t stream);

/* Saturating fp8 quantize / fake-quant with a per-tensor scale ([QAT]
 * fake_quant_fp8 and its unified-ULP rounding, ties to even): y = x / scale,
 * byte = cast(y) (NaN -> 0x7F, +-Inf and |y| rounding above max -> +-max, sign
 * and -0 kept, fp8 subnormals produced), fq = decode(byte) * scale.
 * scale: device float; 0 gives byte 0 and fq +0 ([MAR]).  q (may be NULL): u8
 * [n]; fq (may be NULL): float32 [n]; at least one. */
int fq_fp8_quantize(const float* x, int64_t n, int fmt, const float* scale, uint8_t* q, float* fq,
                    hipStream_t stream);

/* fp8 dequantize: out = decode(q) * scale for every byte (E5M2 infinities and
 * all NaN patterns decode as such). */
int fq_fp8_dequantize(const uint8_t* q, int64_t n, int fmt, const float* scale, float* out,
                      hipStream_t stream);

/* 64-element 4-bit absmax blocks with 8-bit double quantization of the block
 * scales over groups of 256 ([DQ] quantize_4bit_double):
 *   s_b = absmax_b / 7 over the finite elements of each 64-element block (the last
 *         block may be partial), code = clamp(RNE(x / s_b), -7, 7) (0 if s_b = 0);
 *   S_k = max(max of the 256 s_b of group k, 1e-8);
 *   u_b = clamp(round_half_away(s_b / S_k * 255), 0, 255).
 * packed: ceil(n/2) bytes (element i in byte i/2, even i high nibble);
 * qscale: u8 [ceil(n/64)]; super_scale: float32 [ceil(n/16384)];
 * block_scale (may be NULL): the fp32 s_b; recon (may be NULL): float32 [n] =
 * dequantize_4bit_double of the result, code * (u_b / 255 * S_k).
 * One launch, one read of x. */
int fq_q4dq_quantize(const float* x, int64_t n, uint8_t* packed, uint8_t* qscale,
                     float* super_scale, float* block_scale, float* recon, uint32_t* flags,
                     hipStream_t stream);

/* [DQ] dequantize_4bit_double: out[i] = code_i * (u_b / 255 * S_k). */
int fq_q4dq_dequantize(const uint8_t* packed, const uint8_t* qscale, const float* super_scale,
                       int64_t n, float* out, hipStream_t stream);

/* 32-element fp8 E4M3 blocks with power-of-two scales along each row ([CS]
 * block_scaled, scale kind "e8m0"): per block of 32 consecutive elements of a row
 * (a partial block at the row end), A = finite amax (1 if 0), k = frexp exponent
 * of A, X = 2^max(k - 1 - 8, -127); q = E4M3 cast of x / X (saturating),
 * e8m0 = log2(X) + 127, fq = decode(q) * X.
 * x: [rows, cols] FQ_F32 or FQ_BF16; q: u8 [rows, cols]; e8m0: u8
 * [rows, ceil(cols/32)]; fq (may be NULL): float32 [rows, cols]. */
int fq_mxfp8_rows(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q, uint8_t* e8m0,
                  float* fq, hipStream_t stream);

/* ---- FP4 / FP6 block formats -------------------------------------------- */

/* [CS] demo 4 block_scaled(x, elem, 32, "e8m0") along rows (MXFP4 / MXFP6):
 * per block of 32 elements of a row (a short block at the row end), X = 2^(k - 1
 * - emax) with k the frexp exponent of the block's finite amax (amax 0 taken as
 * 1, exponent clamped below at -127); codes = elem(x / X) with ties to even and
 * saturation (NaN -> +0, +-Inf -> +-max); fq = decode * X.  elem: FQ_E2M1
 * (emax 2), FQ_E2M3 (emax 2), FQ_E3M2 (emax 4), or FQ_E4M3 (as fq_mxfp8_rows).
 * x: [rows, cols] FQ_F32 or FQ_BF16; q: E2M1 packed two codes per byte,
 * ceil(cols/2) bytes per row, even column in the high nibble; E2M3 / E3M2 one
 * code per byte [rows, cols] (sign in bit 5); e8m0: u8 [rows, ceil(cols/32)]
 * (exponent + 127); fq (may be NULL): float32 [rows, cols].  One launch. */
int fq_mx_rows(const void* x, int dtype, int64_t rows, int64_t cols, int elem, uint8_t* q, uint8_t* e8m0,
               float* fq, hipStream_t stream);

/* [CS] demo 4 block_scaled(x, FP4_E2M1, 16, "e4m3") (NVFP4) over the flattened
 * float32 x[n]: tensor scale g = amax(x) / (6 * 448) over the finite elements;
 * per block of 16 (the last one short when n % 16 != 0), s = E4M3(amax_block /
 * 6 / g) with saturation, X = s * g, or 1 where X is not > 0; codes =
 * E2M1(x / X), fq = decode * X; binary32 throughout, in the page's order.
 * q: packed E2M1 codes, ceil(n/2) bytes, even element in the high nibble;
 * scales: the E4M3 byte of s per block, ceil(n/16) bytes; tensor_scale: one
 * device float (g); fq (may be NULL): float32 [n].  workspace: device memory of
 * fq_workspace_bytes(n), 16-byte aligned, contents not kept.  Three or four
 * launches (the tensor amax in two, then the blocks). */
int fq_nvfp4(const float* x, int64_t n, void* workspace, size_t workspace_bytes, uint8_t* q, uint8_t* scales,
             float* tensor_scale, float* fq, hipStream_t stream);

/* ---- per-column calibration --------------------------------------------- */

/* Workspace bytes fq_quant_cols needs for a [rows, cols] tensor (0 for empty
 * shapes): min(rows, 64) + 1 records of 16 bytes per column. */
size_t fq_cols_workspace_bytes(int64_t rows, int64_t cols);

/* [QAT] per_channel_params + fake_quant_int_per_channel with axis = 1: every
 * column of the row-major x [rows, cols] (FQ_F32 or FQ_BF16) is a channel,
 * calibrated on that column only (finite min / max, [QAT] from_minmax) and
 * quantized with its own scale / zero-point, as fq_quant_rows does per row.
 * codes (may be NULL): int8 [rows, cols] or, for 4 bits, packed nibbles
 * ceil(cols/2) bytes per row (even column in the high nibble); fq (may be NULL):
 * float32 [rows, cols]; scale, zero_point: [cols].  workspace: device memory of
 * fq_cols_workspace_bytes(rows, cols), 16-byte aligned, contents not kept.
 * Three launches (column min / max over at most 64 bands of rows, the fold of
 * the bands, quantize with per-column parameters); x is read twice.  Tensors of
 * 1025 to 4096 rows with rows * cols < 2^31 whose column count is a multiple of
 * the strip width (16 FQ_F32 or 32 FQ_BF16 columns, with at least half as many
 * strips as the device has compute units), with x aligned to 16 (FQ_F32) or 8
 * (FQ_BF16) bytes, fq to 16 and codes to 4 (int8) or 2 (int4) bytes, take one
 * launch that reads x once and leaves the workspace untouched. */
int fq_quant_cols(const void* x, int dtype, int64_t rows, int64_t cols, int bits, int scheme, void* workspace,
                  size_t workspace_bytes, void* codes, float* fq, float* scale, int32_t* zero_point, uint32_t* flags,
                  hipStream_t stream);

/* ---- group-wise calibration ---------------------------------------------- */

/* [CS] demo 3 "granularity": groups of `group` consecutive elements along each
 * row of the row-major x [rows, cols] (FQ_F32 or FQ_BF16), each calibrated and
 * quantized as a [QAT] channel is (finite min / max, from_minmax, RNE; as
 * fq_quant_rows does per row).  When group does not divide cols, the last group
 * of each row holds the cols mod group elements left.  group >= 1 (group >= cols
 * is per-row quantization).
 * codes (may be NULL): int8 [rows, cols] or, for 4 bits, packed nibbles
 * ceil(cols/2) bytes per row (even column in the high nibble); fq (may be NULL):
 * float32 [rows, cols]; scale, zero_point: [rows, ceil(cols / group)], group g of
 * row r at r * ceil(cols / group) + g.  One launch when group divides cols:
 * groups of 16..1024 elements run sixteen elements per lane, a group being 1..64
 * lanes reduced in registers (groups of 4 and 8, and buffers not 16-byte aligned,
 * four elements per lane); other dividing sizes run as the rows of the
 * [rows * cols / group, group] reshape; otherwise one thread per group. */
int fq_quant_groups(const void* x, int dtype, int64_t rows, int64_t cols, int64_t group, int bits, int scheme,
                    void* codes, float* fq, float* scale, int32_t* zero_point, uint32_t* flags, hipStream_t stream);

/* ---- percentile calibration ---------------------------------------------- */

/* Workspace bytes fq_tensor_params_percentile needs for n elements (0 for
 * n < 1): the selection state plus candidate slots for about one element in 16. */
size_t fq_percentile_workspace_bytes(int64_t n);

/* [QAT] QuantParams::per_tensor_percentile: calibration on the clipped tails of
 * x[n] (float32, device).  With the m finite elements in ascending order
 * (-0 before +0) and last = m - 1, lo = floor(cf * last) and
 * hi = ceil((1 - cf) * last), both in double and at most last; the order
 * statistics f[lo] and f[hi] take the place of min and max in the calibration of
 * fq_tensor_params_int.  Non-finite elements are left out and set
 * FQ_FLAG_NONFINITE (the page refuses them); no finite element gives scale 0 and
 * FQ_FLAG_DEGENERATE as well.  clip_fraction cf in [0, 0.5) (FQ_E_INVALID
 * otherwise; 0 gives the min / max calibration).  workspace: device memory of
 * fq_percentile_workspace_bytes(n), 16-byte aligned, cleared by the call itself,
 * contents not kept.  params, flags: device, as fq_tensor_params_int.  Five
 * launches (zeroing, three passes that narrow both order statistics by 11, 11
 * and 10 bits of an order-preserving key, each pass's digit selected at the start
 * of the next launch, and a one-workgroup launch for the last digit and the
 * parameters; x is read twice, the third pass reading only the candidates the
 * second one kept, or x once more if they did not fit).  From 2^23 elements on,
 * a sample of x predicts the statistics' first-digit bins, the first pass keeps
 * their keys, and when the prediction holds the second pass reads those instead
 * of x (x read once); the result does not depend on the prediction.  No host
 * synchronisation. */
int fq_tensor_params_percentile(const float* x, int64_t n, int bits, int scheme, double clip_fraction,
                                void* workspace, size_t workspace_bytes, fq_int_params* params, uint32_t* flags,
                                hipStream_t stream);

/* ---- stochastic rounding ------------------------------------------------
 * [QAT] module docs "Rounding modes", RoundingMode::Stochastic: a quotient t is
 * rounded to floor(t) + 1 with probability equal to its fractional part and to
 * floor(t) otherwise (unbiased).  Here: up iff u < fl(t - floor(t)), where the
 * variate of element index i is u = (w >> 8) * 2^-24 and w is word (i mod 4) of
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) at counter
 * (floor(i/4) mod 2^32, floor(i/4) div 2^32, 0, 0) under key
 * (seed mod 2^32, seed div 2^32).  x[k] has index offset + k, so a tensor split
 * over calls (or devices) with matching offsets draws the same numbers. */

/* fq_fake_quant_int_tensor with stochastic rounding of t = x / scale:
 * code = clamp(round_sr(t), qmin - zp, qmax - zp) + zp (NaN -> 0, +-Inf clamp,
 * scale 0 -> 0); fq = (code - zp) * scale.  Arguments and layouts as
 * fq_fake_quant_int_tensor, plus seed and offset. */
int fq_fake_quant_int_tensor_sr(const float* x, int64_t n, int bits, int scheme, const fq_int_params* params,
                                uint64_t seed, uint64_t offset, void* codes, float* fq, hipStream_t stream);

/* fq_fp8_quantize with stochastic rounding on the fp8 grid ([QAT]
 * fp8_quantize_magnitude with the stochastic mode): for y = x / scale with
 * binade step 2^(max(e, emin) - mbits), |y| / step is rounded stochastically,
 * times step, saturated at max-normal; NaN -> 0x7F, +-Inf -> +-max, sign kept,
 * scale 0 -> byte 0.  Arguments and layouts as fq_fp8_quantize, plus seed and
 * offset. */
int fq_fp8_quantize_sr(const float* x, int64_t n, int fmt, const float* scale, uint64_t seed, uint64_t offset,
                       uint8_t* q, float* fq, hipStream_t stream);

/* ---- QAT optimizer step -------------------------------------------------
 * [QAT] QatOptimizer::step: an Adam / AdamW update of the fp32 master weights
 * (QatConfig lr, beta1, beta2, eps, weight_decay), then the quantized view
 * re-derived from the updated master (requantize).  Per element, binary32, one
 * rounding per operation, in the page's order:
 *   m = beta1 m + (1 - beta1) g;   v = beta2 v + ((1 - beta2) g) g;
 *   m_hat = m / bc1;   v_hat = v / bc2;   (bc = 1 - beta^t, formed in double
 *   from the binary32 beta and rounded once)
 *   if weight_decay != 0: w = w - (lr weight_decay) w;
 *   w = w - (lr m_hat) / (sqrt(v_hat) + eps).
 * master, m, v are updated in place (caller-owned optimizer state, zero before
 * step t = 1); grad is read.  All are float32 [n], device memory.  cfg is a HOST
 * pointer; t >= 1 is the step number (FQ_E_INVALID otherwise, or when a beta is
 * outside [0, 1)). */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
} fq_adamw_config;

/* rounding of the view ([QAT] RoundingMode) */
#define FQ_ROUND_NEAREST 0
#define FQ_ROUND_STOCHASTIC 1

/* Integer target: the update, then per_tensor_minmax of the updated master
 * (params, flags as fq_tensor_params_int, same workspace size
 * fq_workspace_bytes(n)) and fake_quant_int with `rounding` (stochastic: the
 * stream of fq_fake_quant_int_tensor_sr at seed / offset).  codes (as
 * fq_fake_quant_int_tensor) and view (float32 [n], the fake-quant view) may each
 * be NULL, not both.  Nearest rounding: two launches (the requantize folds the
 * update pass's partials) when master, codes and view are 16-byte aligned, else
 * three; stochastic rounding: three.  No host synchronisation. */
int fq_qat_step_int(float* master, const float* grad, float* m, float* v, int64_t n, const fq_adamw_config* cfg,
                    int64_t t, int bits, int scheme, int rounding, uint64_t seed, uint64_t offset, void* workspace,
                    size_t workspace_bytes, fq_int_params* params, void* codes, float* view, uint32_t* flags,
                    hipStream_t stream);

/* fp8 target: the update, then fake_quant_fp8 of the updated master itself (no
 * scale, as the page's optimizer): q (bytes as fq_fp8_quantize, may be NULL) and
 * view = decode(q) (float32 [n], may be NULL; not both NULL).  One launch. */
int fq_qat_step_fp8(float* master, const float* grad, float* m, float* v, int64_t n, const fq_adamw_config* cfg,
                    int64_t t, int fmt, int rounding, uint64_t seed, uint64_t offset, uint8_t* q, float* view,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FQ_H */
