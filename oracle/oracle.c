/*
 * oracle.c -- plain, slow, scalar CPU reference of the fake-quant hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no header, constant, table or helper with
 * the HIP kernels: every value below is written out here from the pages.
 *
 * Sources (cited by page title and section):
 *   [QAT]  optirs-gpu 0.3.2, src/optirs_gpu/quantization.rs ("Quantization-Aware
 *          Training (QAT) primitives"): module docs, QuantParams, fp8 helpers,
 *          fake_quant_backward and its unit tests.
 *   [DQ]   aprender-train 0.32.0, entrenar/quant/double_quant.rs ("Double
 *          quantization for QLoRA"): quantize_4bit_double, dequantize_4bit_double,
 *          reconstruct_scales.
 *   [CS]   CS349E 05_quantization_basics.py, demo 4 `block_scaled` ("e8m0" kind).
 *   [MAR]  ferrum-kernels 0.8.0 marlin_repack.rs, `quantized_fp8_bits` (zero scale
 *          gives code 0) and the per-channel scale absmax / 448.
 *
 * Arithmetic: IEEE binary32, one rounding per operation.  Build with
 *   gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math
 * so no FMA contraction or re-association happens.  Round-half-even comes from
 * nearbyintf() in the default rounding mode, round-half-away from roundf().
 *
 * Readings of points the pages leave open are marked READING and listed with
 * the design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Data-dependent condition flags, OR-ed into a flags word. */
#define ORC_FLAG_NONFINITE 1u  /* a calibration group held Inf or NaN            */
#define ORC_FLAG_DEGENERATE 2u /* a calibration group had no usable range (zero) */

enum { ORC_SYM = 0, ORC_AFFINE = 1 };
enum { ORC_E4M3 = 0, ORC_E5M2 = 1, ORC_E2M1 = 2, ORC_E2M3 = 3, ORC_E3M2 = 4 };
enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* ------------------------------------------------------------------------- */
/* Small helpers                                                              */
/* ------------------------------------------------------------------------- */

static float bits_to_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* bfloat16 is the upper half of a binary32; widening is exact. */
float orc_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

static float widen(const void* x, int dtype, int64_t i) {
    if (dtype == ORC_BF16) return orc_bf16_to_f32(((const uint16_t*)x)[i]);
    return ((const float*)x)[i];
}

/* ------------------------------------------------------------------------- */
/* Integer grid: [QAT] IntDtype::q_range, QuantParams                         */
/* ------------------------------------------------------------------------- */

/* [QAT] IntDtype::from_bits / q_range: symmetric uses the restricted range
 * (-127..127, -7..7), affine the full two's-complement range (-128..127, -8..7).
 * Any width other than 4 or 8 is unsupported (returns -2). */
int orc_q_range(int bits, int scheme, int32_t* qmin, int32_t* qmax) {
    if (bits != 8 && bits != 4) return -2;
    if (scheme != ORC_SYM && scheme != ORC_AFFINE) return -2;
    if (bits == 8) {
        *qmin = scheme == ORC_SYM ? -127 : -128;
        *qmax = 127;
    } else {
        *qmin = scheme == ORC_SYM ? -7 : -8;
        *qmax = 7;
    }
    return 0;
}

/* [QAT] finite_min_max, with the calibration error turned into a flag.
 * READING: a non-finite element sets NONFINITE and the reduction continues over
 * the finite elements; a group with no finite element reports min = max = 0
 * (which the parameter step then flags as DEGENERATE). */
uint32_t orc_finite_min_max(const void* x, int dtype, int64_t n, int64_t stride,
                            float* mn, float* mx) {
    uint32_t flags = 0;
    float lo = INFINITY, hi = -INFINITY;
    int64_t count = 0;
    for (int64_t i = 0; i < n; ++i) {
        float v = widen(x, dtype, i * stride);
        if (!isfinite(v)) {
            flags |= ORC_FLAG_NONFINITE;
            continue;
        }
        if (v < lo) lo = v;
        if (v > hi) hi = v;
        ++count;
    }
    if (count == 0) {
        lo = 0.0f;
        hi = 0.0f;
    }
    *mn = lo;
    *mx = hi;
    return flags;
}

/* [QAT] QuantParams::from_absmax: scale = absmax / qmax, zero_point = 0; the
 * page rejects a non-finite or non-positive absmax and a non-positive scale.
 * READING: rejection becomes DEGENERATE with scale = 0, zero_point = 0. */
static uint32_t params_from_absmax(float absmax, int32_t qmax, float* scale, int32_t* zp) {
    *zp = 0;
    if (!isfinite(absmax) || !(absmax > 0.0f)) {
        *scale = 0.0f;
        return ORC_FLAG_DEGENERATE;
    }
    float s = absmax / (float)qmax;
    if (!isfinite(s) || !(s > 0.0f)) {
        *scale = 0.0f;
        return ORC_FLAG_DEGENERATE;
    }
    *scale = s;
    return 0;
}

/* [QAT] QuantParams::from_minmax.
 * Symmetric: from_absmax(max(|min|, |max|)).
 * Affine: nudge the interval to contain 0 (rmin = min(min, 0), rmax = max(max, 0)),
 * scale = (rmax - rmin) / (qmax - qmin), zero_point = clamp(RNE(qmin - rmin/scale)).
 * Operation order is the page's: rmin/scale first, then qmin minus that. */
uint32_t orc_params_from_minmax(float mn, float mx, int bits, int scheme, float* scale,
                                int32_t* zp) {
    int32_t qmin, qmax;
    if (orc_q_range(bits, scheme, &qmin, &qmax) != 0) return 0;
    if (!isfinite(mn) || !isfinite(mx) || mx < mn) {
        *scale = 0.0f;
        *zp = 0;
        return ORC_FLAG_DEGENERATE;
    }
    if (scheme == ORC_SYM) {
        float amin = fabsf(mn), amax = fabsf(mx);
        return params_from_absmax(amin > amax ? amin : amax, qmax, scale, zp);
    }
    float rmin = mn < 0.0f ? mn : 0.0f;
    float rmax = mx > 0.0f ? mx : 0.0f;
    float range = rmax - rmin;
    if (!(range > 0.0f)) {
        *scale = 0.0f;
        *zp = 0;
        return ORC_FLAG_DEGENERATE;
    }
    float s = range / (float)(qmax - qmin);
    if (!isfinite(s) || !(s > 0.0f)) {
        *scale = 0.0f;
        *zp = 0;
        return ORC_FLAG_DEGENERATE;
    }
    float z = nearbyintf((float)qmin - rmin / s);
    if (z < (float)qmin) z = (float)qmin;
    if (z > (float)qmax) z = (float)qmax;
    *scale = s;
    *zp = (int32_t)z;
    return 0;
}

/* [QAT] module docs "Integer quantization": quant(x) = clamp(round(x/scale) + zp,
 * qmin, qmax), round = ties-to-even (RoundingMode::Nearest).
 * READING (doc formula, not the f64 code order): the quotient is rounded to an
 * integer first and the integer zero-point is added after, exactly.
 * READING: scale == 0 (degenerate params) gives code 0; a NaN quotient gives code 0
 * (the page's integer cast of NaN); +-Inf clamp to the range ends. */
int32_t orc_quantize(float x, float scale, int32_t zp, int32_t qmin, int32_t qmax) {
    if (scale == 0.0f) return 0;
    float t = x / scale;
    if (isnan(t)) return 0;
    double v = (double)nearbyintf(t) + (double)zp; /* exact for |t| < 2^53 */
    if (v < (double)qmin) v = (double)qmin;
    if (v > (double)qmax) v = (double)qmax;
    return (int32_t)v;
}

/* [QAT] dequant(q) = (q - zero_point) * scale. */
float orc_dequantize(int32_t q, float scale, int32_t zp) { return (float)(q - zp) * scale; }

/* [QAT] QuantParams::real_min / real_max: dequant(qmin), dequant(qmax). */
void orc_real_bounds(float scale, int32_t zp, int32_t qmin, int32_t qmax, float* lo,
                     float* hi) {
    *lo = orc_dequantize(qmin, scale, zp);
    *hi = orc_dequantize(qmax, scale, zp);
}

/* [QAT] QuantParams::per_tensor_minmax followed by real_min / real_max. */
uint32_t orc_tensor_params_int(const float* x, int64_t n, int bits, int scheme, float* scale,
                               int32_t* zp, float* lo, float* hi) {
    int32_t qmin, qmax;
    if (orc_q_range(bits, scheme, &qmin, &qmax) != 0) return 0;
    float mn, mx;
    uint32_t flags = orc_finite_min_max(x, ORC_F32, n, 1, &mn, &mx);
    flags |= orc_params_from_minmax(mn, mx, bits, scheme, scale, zp);
    orc_real_bounds(*scale, *zp, qmin, qmax, lo, hi);
    return flags;
}

/* [QAT] fake_quant_int: dequant(quant(x)) element-wise with one parameter set.
 * Either output may be NULL. */
void orc_fake_quant_int(const float* x, int64_t n, int bits, int scheme, float scale, int32_t zp,
                        int8_t* codes, float* fq) {
    int32_t qmin, qmax;
    if (orc_q_range(bits, scheme, &qmin, &qmax) != 0) return;
    for (int64_t i = 0; i < n; ++i) {
        int32_t q = orc_quantize(x[i], scale, zp, qmin, qmax);
        if (codes) codes[i] = (int8_t)q;
        if (fq) fq[i] = orc_dequantize(q, scale, zp);
    }
}

/* [QAT] dequant over an array of stored codes. */
void orc_dequantize_int(const int8_t* codes, int64_t n, float scale, int32_t zp, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_dequantize(codes[i], scale, zp);
}

/* [QAT] fake_quant_backward: the gradient passes where lo <= x <= hi (both ends
 * inclusive) and is zero elsewhere; the bounds may come in either order.
 * A NaN x fails both comparisons and gets +0. */
void orc_ste_backward(const float* g, const float* x, int64_t n, float b0, float b1, float* out) {
    float lo = b0 <= b1 ? b0 : b1;
    float hi = b0 <= b1 ? b1 : b0;
    for (int64_t i = 0; i < n; ++i) out[i] = (x[i] >= lo && x[i] <= hi) ? g[i] : 0.0f;
}

/* [QAT] per_channel_params + fake_quant_int_per_channel along axis 0: every row
 * is a channel with its own (scale, zero_point).  x is [rows, cols] row-major,
 * float32 or bfloat16 (widened exactly).
 * codes: int8 [rows, cols] for bits = 8; for bits = 4 two codes per byte,
 *   ceil(cols/2) bytes per row, element j in byte j/2, even j in the high nibble,
 *   two's-complement nibbles, an odd tail leaves the low nibble 0 (the nibble
 *   layout of [DQ] dequantize_4bit_double).
 * Any of codes, fq may be NULL; scale / zp get one entry per row. */
uint32_t orc_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols, int bits,
                        int scheme, uint8_t* codes, float* fq, float* scale, int32_t* zp) {
    int32_t qmin, qmax;
    if (orc_q_range(bits, scheme, &qmin, &qmax) != 0) return 0;
    uint32_t flags = 0;
    int64_t packed_row = (cols + 1) / 2;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t base = r * cols;
        const void* row = dtype == ORC_BF16 ? (const void*)((const uint16_t*)x + base)
                                            : (const void*)((const float*)x + base);
        float mn, mx, s;
        int32_t z;
        flags |= orc_finite_min_max(row, dtype, cols, 1, &mn, &mx);
        flags |= orc_params_from_minmax(mn, mx, bits, scheme, &s, &z);
        scale[r] = s;
        zp[r] = z;
        if (codes && bits == 4) memset(codes + r * packed_row, 0, (size_t)packed_row);
        for (int64_t c = 0; c < cols; ++c) {
            int32_t q = orc_quantize(widen(row, dtype, c), s, z, qmin, qmax);
            if (fq) fq[base + c] = orc_dequantize(q, s, z);
            if (!codes) continue;
            if (bits == 8) {
                ((int8_t*)codes)[base + c] = (int8_t)q;
            } else {
                uint8_t nib = (uint8_t)(q & 0xF);
                codes[r * packed_row + c / 2] |= (c % 2 == 0) ? (uint8_t)(nib << 4) : nib;
            }
        }
    }
    return flags;
}

/* [QAT] per_channel_params + fake_quant_int_per_channel along axis 1: every
 * column is a channel with its own parameters, calibrated on that column only.
 * Layouts as orc_quant_rows (codes: int8 [rows, cols] or, for 4 bits, packed
 * nibbles ceil(cols/2) bytes per row); scale / zp: one per column. */
uint32_t orc_quant_cols(const void* x, int dtype, int64_t rows, int64_t cols, int bits,
                        int scheme, uint8_t* codes, float* fq, float* scale, int32_t* zp) {
    int32_t qmin, qmax;
    if (orc_q_range(bits, scheme, &qmin, &qmax) != 0) return 0;
    uint32_t flags = 0;
    int64_t packed_row = (cols + 1) / 2;
    for (int64_t c = 0; c < cols; ++c) {
        const void* col = dtype == ORC_BF16 ? (const void*)((const uint16_t*)x + c)
                                            : (const void*)((const float*)x + c);
        float mn, mx;
        flags |= orc_finite_min_max(col, dtype, rows, cols, &mn, &mx);
        flags |= orc_params_from_minmax(mn, mx, bits, scheme, &scale[c], &zp[c]);
    }
    if (codes && bits == 4) memset(codes, 0, (size_t)(rows * packed_row));
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            int32_t q = orc_quantize(widen(x, dtype, r * cols + c), scale[c], zp[c], qmin, qmax);
            if (fq) fq[r * cols + c] = orc_dequantize(q, scale[c], zp[c]);
            if (!codes) continue;
            if (bits == 8) {
                ((int8_t*)codes)[r * cols + c] = (int8_t)q;
            } else {
                uint8_t nib = (uint8_t)(q & 0xF);
                codes[r * packed_row + c / 2] |= (c % 2 == 0) ? (uint8_t)(nib << 4) : nib;
            }
        }
    }
    return flags;
}

/* [CS] demo 3 "granularity": group-wise quantization -- groups of `group`
 * consecutive elements along the last dimension of each row, one scale per
 * group.
 * READING (the body of quantize_int is not on the pages): a group is calibrated
 * as a channel is ([QAT] per_channel_params: finite min / max, from_minmax) and
 * quantized with the channel rule; when group does not divide cols, the last
 * group of a row holds the cols mod group elements left; scales are binary32
 * (the demo's FP16 scale enters only its bits-per-element count).
 * Layouts: codes as orc_quant_rows; scale / zp: [rows, ceil(cols / group)]. */
uint32_t orc_quant_groups(const void* x, int dtype, int64_t rows, int64_t cols, int64_t group, int bits,
                          int scheme, uint8_t* codes, float* fq, float* scale, int32_t* zp) {
    int32_t qmin, qmax;
    if (orc_q_range(bits, scheme, &qmin, &qmax) != 0 || group < 1) return 0;
    uint32_t flags = 0;
    int64_t packed_row = (cols + 1) / 2;
    int64_t ngroups = (cols + group - 1) / group;
    if (codes && bits == 4) memset(codes, 0, (size_t)(rows * packed_row));
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < ngroups; ++g) {
            int64_t start = g * group;
            int64_t len = cols - start < group ? cols - start : group;
            int64_t base = r * cols + start;
            const void* grp = dtype == ORC_BF16 ? (const void*)((const uint16_t*)x + base)
                                                : (const void*)((const float*)x + base);
            float mn, mx, s;
            int32_t z;
            flags |= orc_finite_min_max(grp, dtype, len, 1, &mn, &mx);
            flags |= orc_params_from_minmax(mn, mx, bits, scheme, &s, &z);
            scale[r * ngroups + g] = s;
            zp[r * ngroups + g] = z;
            for (int64_t i = 0; i < len; ++i) {
                int64_t c = start + i;
                int32_t q = orc_quantize(widen(grp, dtype, i), s, z, qmin, qmax);
                if (fq) fq[r * cols + c] = orc_dequantize(q, s, z);
                if (!codes) continue;
                if (bits == 8) {
                    ((int8_t*)codes)[r * cols + c] = (int8_t)q;
                } else {
                    uint8_t nib = (uint8_t)(q & 0xF);
                    codes[r * packed_row + c / 2] |= (c % 2 == 0) ? (uint8_t)(nib << 4) : nib;
                }
            }
        }
    }
    return flags;
}

/* Ascending total order of binary32 values (-0 before +0), as the page's
 * f64::total_cmp on finite values. */
static int cmp_total(const void* a, const void* b) {
    uint32_t ua, ub;
    memcpy(&ua, a, 4);
    memcpy(&ub, b, 4);
    uint32_t ka = (ua & 0x80000000u) ? ~ua : (ua | 0x80000000u);
    uint32_t kb = (ub & 0x80000000u) ? ~ub : (ub | 0x80000000u);
    return ka < kb ? -1 : (ka > kb ? 1 : 0);
}

/* [QAT] QuantParams::per_tensor_percentile: sort the values, take the
 * nearest-rank quantiles lo = floor(cf * last), hi = ceil((1 - cf) * last)
 * (f64 arithmetic, last = count - 1, indices capped at last) and calibrate with
 * from_minmax(sorted[lo], sorted[hi]).
 * READING: non-finite values set NONFINITE and are left out (the page rejects
 * them); with no finite value the result is DEGENERATE (scale 0, zp 0).  The
 * caller checks 0 <= cf < 0.5.  Also returns the two selected values. */
uint32_t orc_percentile_params(const float* x, int64_t n, int bits, int scheme, double clip_fraction,
                               float* scale, int32_t* zp, float* lo, float* hi, float* sel_min, float* sel_max) {
    int32_t qmin, qmax;
    if (orc_q_range(bits, scheme, &qmin, &qmax) != 0) return 0;
    uint32_t flags = 0;
    float* f = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (isfinite(x[i])) f[m++] = x[i];
        else flags |= ORC_FLAG_NONFINITE;
    }
    float mn = INFINITY, mx = -INFINITY;
    if (m > 0) {
        qsort(f, (size_t)m, sizeof(float), cmp_total);
        int64_t last = m - 1;
        int64_t lo_idx = (int64_t)floor(clip_fraction * (double)last);
        int64_t hi_idx = (int64_t)ceil((1.0 - clip_fraction) * (double)last);
        if (lo_idx > last) lo_idx = last;
        if (hi_idx > last) hi_idx = last;
        mn = f[lo_idx];
        mx = f[hi_idx];
    }
    free(f);
    *sel_min = mn;
    *sel_max = mx;
    flags |= orc_params_from_minmax(mn, mx, bits, scheme, scale, zp);
    orc_real_bounds(*scale, *zp, qmin, qmax, lo, hi);
    return flags;
}

/* ------------------------------------------------------------------------- */
/* fp8: [QAT] module docs "fp8 quantization", Fp8Format, fp8_quantize_magnitude */
/* ------------------------------------------------------------------------- */

/* [QAT] Fp8Format table: E4M3 = 3 mantissa bits, bias 7, max-normal 448;
 * E5M2 = 2 mantissa bits, bias 15, max-normal 57344. */
static void fp8_format(int fmt, int* mbits, int* ebits, int* bias, float* maxv) {
    if (fmt == ORC_E4M3) {
        *mbits = 3;
        *ebits = 4;
        *bias = 7;
        *maxv = 448.0f;
    } else {
        *mbits = 2;
        *ebits = 5;
        *bias = 15;
        *maxv = 57344.0f;
    }
}

/* floor(log2(a)) for finite a > 0, exact (frexp gives a = m 2^e, m in [0.5, 1)). */
static int floor_log2(float a) {
    int e;
    frexpf(a, &e);
    return e - 1;
}

/* [QAT] fp8_quantize_magnitude with RoundingMode::Nearest: for a > 0 with binade
 * e = floor(log2 a), the step is 2^(max(e, emin) - mbits), emin = 1 - bias; a is
 * rounded to the nearest multiple of the step (ties to even) and a rounded
 * magnitude above max-normal saturates to max-normal.
 * READING: e is the true floor(log2 a), so binary32 subnormal inputs are handled
 * by the same rule (they all round to 0 in both formats). */
static float fp8_round_magnitude(float a, int mbits, int bias, float maxv) {
    if (a == 0.0f) return 0.0f;
    int emin = 1 - bias;
    int e = floor_log2(a);
    int step_exp = (e > emin ? e : emin) - mbits;
    float step = ldexpf(1.0f, step_exp);
    float k = nearbyintf(a / step); /* a / step is exact: division by a power of two */
    float m = k * step;
    return m > maxv ? maxv : m;
}

/* [QAT] fake_quant_fp8 per element (NaN -> NaN, +-Inf -> +-max, sign kept,
 * including -0) followed by the bit encoding of the result.
 * READING (byte layout): sign | biased exponent | mantissa with the Fp8Format
 * biases; an fp8 subnormal has exponent field 0.  Every NaN input encodes to 0x7F
 * in both formats (E4M3's only NaN pattern is S.1111.111; 0x7F is also a NaN of
 * E5M2). */
/* Byte of a magnitude m already on the fp8 grid (0 <= m <= max-normal). */
static uint8_t fp8_bits(float m, uint8_t sign, int mbits, int bias) {
    if (m == 0.0f) return sign;
    float min_normal = ldexpf(1.0f, 1 - bias);
    uint32_t E, M;
    if (m < min_normal) {
        E = 0;
        M = (uint32_t)(m / ldexpf(1.0f, 1 - bias - mbits));
    } else {
        int e = floor_log2(m);
        E = (uint32_t)(e + bias);
        M = (uint32_t)((m / ldexpf(1.0f, e) - 1.0f) * (float)(1 << mbits));
    }
    return (uint8_t)(sign | (E << mbits) | M);
}

uint8_t orc_fp8_encode(float y, int fmt) {
    int mbits, ebits, bias;
    float maxv;
    fp8_format(fmt, &mbits, &ebits, &bias, &maxv);
    if (isnan(y)) return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    float a = fabsf(y);
    float m = isinf(a) ? maxv : fp8_round_magnitude(a, mbits, bias, maxv);
    return fp8_bits(m, sign, mbits, bias);
}

/* Value of an fp8 byte ([QAT] table): E4M3 has no infinities and S.1111.111 is
 * its NaN; E5M2 is IEEE-like (exponent field all ones: Inf if mantissa 0, else
 * NaN).  Exponent field 0 is subnormal: M * 2^(1 - bias - mbits). */
float orc_fp8_decode(uint8_t b, int fmt) {
    int mbits, ebits, bias;
    float maxv;
    fp8_format(fmt, &mbits, &ebits, &bias, &maxv);
    uint32_t E = (b >> mbits) & ((1u << ebits) - 1u);
    uint32_t M = b & ((1u << mbits) - 1u);
    float v;
    if (fmt == ORC_E4M3 && E == 15 && M == 7) return NAN;
    if (fmt == ORC_E5M2 && E == 31) {
        if (M != 0) return NAN;
        v = INFINITY;
    } else if (E == 0) {
        v = ldexpf((float)M, 1 - bias - mbits);
    } else {
        v = ldexpf(1.0f + (float)M / (float)(1 << mbits), (int)E - bias);
    }
    return (b & 0x80) ? -v : v;
}

void orc_fp8_encode_n(const float* y, int64_t n, int fmt, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(y[i], fmt);
}

void orc_fp8_decode_n(const uint8_t* b, int64_t n, int fmt, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_decode(b[i], fmt);
}

/* Largest |x| over the finite elements (0 when there are none).
 * READING: the per-tensor fp8 calibration skips Inf and NaN. */
float orc_amax_finite(const float* x, int64_t n) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (isfinite(a) && a > m) m = a;
    }
    return m;
}

/* Per-tensor fp8 scale = amax / max-normal ([MAR] per-channel absmax / 448 rule
 * applied per tensor).  A zero scale is flagged DEGENERATE. */
uint32_t orc_fp8_scale(float amax, int fmt, float* scale) {
    int mbits, ebits, bias;
    float maxv;
    fp8_format(fmt, &mbits, &ebits, &bias, &maxv);
    *scale = amax / maxv;
    return *scale == 0.0f ? ORC_FLAG_DEGENERATE : 0u;
}

/* fp8 quantize (byte = encode(x / scale)) and fake-quant
 * (fq = decode(byte) * scale, [QAT] fake_quant(x) = dequant(quant(x))).
 * [MAR] quantized_fp8_bits: a zero scale gives byte 0 (and so fq = +0).
 * Either output may be NULL. */
void orc_fp8_quantize(const float* x, int64_t n, int fmt, float scale, uint8_t* q, float* fq) {
    for (int64_t i = 0; i < n; ++i) {
        uint8_t b = scale == 0.0f ? 0 : orc_fp8_encode(x[i] / scale, fmt);
        if (q) q[i] = b;
        if (fq) fq[i] = orc_fp8_decode(b, fmt) * scale;
    }
}

/* fp8 dequantize: decode(byte) * scale. */
void orc_fp8_dequantize(const uint8_t* q, int64_t n, int fmt, float scale, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_decode(q[i], fmt) * scale;
}

/* ------------------------------------------------------------------------- */
/* 4-bit blocks + double quantization: [DQ]                                   */
/* ------------------------------------------------------------------------- */

#define DQ_BLOCK 64       /* [DQ] "Level 1: ... 64-element blocks"        */
#define DQ_SUPER 256      /* [DQ] DOUBLE_QUANT_BLOCK_SIZE                 */

/* First-level 4-bit quantizer ([DQ] imports quantize_4bit; its body is not on the
 * page).  READING, from the page's hints: blocks of 64 consecutive elements (the
 * last may be partial), scale = absmax / 7 ("Scales are always non-negative
 * (absmax / 7)"), code = RNE(x / scale) clamped to [-7, 7], an all-zero block has
 * scale 0 and codes 0.  Non-finite elements: NONFINITE flag, left out of the
 * absmax, NaN -> code 0, +-Inf clamp to +-7.
 * Packing follows dequantize_4bit_double: the element with global index i sits in
 * byte i/2, even i in the high nibble, as a two's-complement nibble. */
static uint32_t quantize_4bit_blocks(const float* x, int64_t n, uint8_t* packed, float* s) {
    uint32_t flags = 0;
    if (n <= 0) return 0;
    int64_t nb = (n + DQ_BLOCK - 1) / DQ_BLOCK;
    memset(packed, 0, (size_t)((n + 1) / 2));
    for (int64_t b = 0; b < nb; ++b) {
        int64_t start = b * DQ_BLOCK;
        int64_t end = start + DQ_BLOCK < n ? start + DQ_BLOCK : n;
        float absmax = 0.0f;
        for (int64_t i = start; i < end; ++i) {
            float a = fabsf(x[i]);
            if (!isfinite(a)) {
                flags |= ORC_FLAG_NONFINITE;
                continue;
            }
            if (a > absmax) absmax = a;
        }
        float sb = absmax / 7.0f;
        s[b] = sb;
        for (int64_t i = start; i < end; ++i) {
            int32_t code = 0;
            if (sb != 0.0f) {
                float t = x[i] / sb;
                if (!isnan(t)) {
                    float r = nearbyintf(t);
                    if (r < -7.0f) r = -7.0f;
                    if (r > 7.0f) r = 7.0f;
                    code = (int32_t)r;
                }
            }
            uint8_t nib = (uint8_t)(code & 0xF);
            packed[i / 2] |= (i % 2 == 0) ? (uint8_t)(nib << 4) : nib;
        }
    }
    return flags;
}

/* [DQ] reconstruct_scales: scale = q / 255 * super_scale (left to right). */
static float reconstruct_scale(uint8_t q, float super_scale) {
    return (float)q / 255.0f * super_scale;
}

/* [DQ] dequantize_4bit_double inner step: nibble -> sign-extended code. */
static int32_t unpack_code(const uint8_t* packed, int64_t i) {
    uint8_t byte = packed[i / 2];
    uint8_t nib = (i % 2 == 0) ? (uint8_t)((byte >> 4) & 0x0F) : (uint8_t)(byte & 0x0F);
    return (nib & 0x08) ? (int32_t)nib - 16 : (int32_t)nib;
}

/* [DQ] quantize_4bit_double: first-level 4-bit blocks, then per group of 256
 * block scales the super-scale = max(max scale, 1e-8) and each scale becomes
 * u8 = clamp(round(scale / super * 255), 0, 255); round is the page's f32::round
 * (half away from zero).  The packed data are the first-level codes unchanged.
 * Outputs: packed ceil(n/2) bytes, qscale ceil(n/64) bytes, super ceil(nb/256)
 * floats; block_scale (the fp32 first-level scales) and recon
 * (dequantize_4bit_double of the result) may be NULL. */
uint32_t orc_q4dq_quantize(const float* x, int64_t n, uint8_t* packed, uint8_t* qscale,
                           float* super_scale, float* block_scale, float* recon) {
    int64_t nb = (n + DQ_BLOCK - 1) / DQ_BLOCK;
    int64_t ns = (nb + DQ_SUPER - 1) / DQ_SUPER;
    float* s = (float*)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(float));
    uint32_t flags = quantize_4bit_blocks(x, n, packed, s);
    const float floor_scale = 1e-8f; /* the page's f32 literal 1e-8 */
    for (int64_t k = 0; k < ns; ++k) {
        int64_t start = k * DQ_SUPER;
        int64_t end = start + DQ_SUPER < nb ? start + DQ_SUPER : nb;
        float mx = s[start];
        for (int64_t b = start + 1; b < end; ++b)
            if (s[b] > mx) mx = s[b];
        if (mx < floor_scale) mx = floor_scale;
        super_scale[k] = mx;
        for (int64_t b = start; b < end; ++b) {
            float normalized = s[b] / mx;
            float r = roundf(normalized * 255.0f);
            if (r < 0.0f) r = 0.0f;
            if (r > 255.0f) r = 255.0f;
            qscale[b] = (uint8_t)r;
        }
    }
    if (block_scale) memcpy(block_scale, s, (size_t)nb * sizeof(float));
    free(s);
    if (recon) {
        for (int64_t b = 0; b < nb; ++b) {
            float sc = reconstruct_scale(qscale[b], super_scale[b / DQ_SUPER]);
            int64_t start = b * DQ_BLOCK;
            int64_t end = start + DQ_BLOCK < n ? start + DQ_BLOCK : n;
            for (int64_t i = start; i < end; ++i) recon[i] = (float)unpack_code(packed, i) * sc;
        }
    }
    return flags;
}

/* [DQ] dequantize_4bit_double: code * reconstructed block scale. */
void orc_q4dq_dequantize(const uint8_t* packed, const uint8_t* qscale, const float* super_scale,
                         int64_t n, float* out) {
    int64_t nb = (n + DQ_BLOCK - 1) / DQ_BLOCK;
    for (int64_t b = 0; b < nb; ++b) {
        float sc = reconstruct_scale(qscale[b], super_scale[b / DQ_SUPER]);
        int64_t start = b * DQ_BLOCK;
        int64_t end = start + DQ_BLOCK < n ? start + DQ_BLOCK : n;
        for (int64_t i = start; i < end; ++i) out[i] = (float)unpack_code(packed, i) * sc;
    }
}

/* ------------------------------------------------------------------------- */
/* 32-element fp8 E4M3 blocks with power-of-two scales: [CS] block_scaled e8m0 */
/* ------------------------------------------------------------------------- */

#define MX_BLOCK 32
#define E4M3_EMAX 8 /* 448 = 1.75 * 2^8 */

/* [CS] block_scaled(x, FP8_E4M3, 32, "e8m0"): per block amax (0 treated as 1),
 * k from frexp(amax), X = 2^(k - 1 - emax); elements y = x / X go through the
 * saturating element cast and come back as cast(y) * X.
 * READINGS: blocks run along each row (32 consecutive elements, a partial block
 * at the row end when cols % 32 != 0); amax is over finite elements; the
 * exponent of X is clamped below at -127 (the E8M0 minimum) and the E8M0 byte is
 * that exponent + 127.  q: [rows, cols] bytes; e8m0: [rows, ceil(cols/32)];
 * fq (NULL allowed): cast(y) * X as float32. */
void orc_mxfp8_rows(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q,
                    uint8_t* e8m0, float* fq) {
    int64_t nbr = (cols + MX_BLOCK - 1) / MX_BLOCK;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nbr; ++b) {
            int64_t c0 = b * MX_BLOCK;
            int64_t c1 = c0 + MX_BLOCK < cols ? c0 + MX_BLOCK : cols;
            float amax = 0.0f;
            for (int64_t c = c0; c < c1; ++c) {
                float a = fabsf(widen(x, dtype, r * cols + c));
                if (isfinite(a) && a > amax) amax = a;
            }
            int k;
            frexpf(amax > 0.0f ? amax : 1.0f, &k);
            int xe = k - 1 - E4M3_EMAX;
            if (xe < -127) xe = -127;
            float X = ldexpf(1.0f, xe);
            e8m0[r * nbr + b] = (uint8_t)(xe + 127);
            for (int64_t c = c0; c < c1; ++c) {
                float y = widen(x, dtype, r * cols + c) / X;
                uint8_t byte = orc_fp8_encode(y, ORC_E4M3);
                q[r * cols + c] = byte;
                if (fq) fq[r * cols + c] = orc_fp8_decode(byte, ORC_E4M3) * X;
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Narrow element formats in block-scaled tensors: [CS] demo 4 block_scaled,   */
/* "e8m0" (MXFP4 / MXFP6) and "e4m3" with a tensor scale (NVFP4)               */
/* ------------------------------------------------------------------------- */

/* READING (the element tables sit in a module the pages do not show): the FP4
 * and FP6 elements follow the same minifloat rule as the page's fp8 formats --
 * sign, E exponent bits with bias 2^(E-1) - 1, M mantissa bits, exponent field
 * 0 subnormal -- and every code is a finite number (no Inf or NaN codes), so the
 * largest magnitude is (2 - 2^-M) 2^(2^E - 1 - bias).  This gives E2M1 max 6
 * and emax 2, which the page states (scaled block maxima in [4, 8), values
 * beyond 6 clipped); E2M3 max 7.5, emax 2; E3M2 max 28, emax 4. */
static void narrow_format(int elem, int* ebits, int* mbits, int* bias, int* emax, float* maxv) {
    switch (elem) {
        case ORC_E2M1: *ebits = 2; *mbits = 1; break;
        case ORC_E2M3: *ebits = 2; *mbits = 3; break;
        default: *ebits = 3; *mbits = 2; break; /* ORC_E3M2 */
    }
    *bias = (1 << (*ebits - 1)) - 1;
    *emax = (1 << *ebits) - 1 - *bias;
    *maxv = ldexpf(2.0f - ldexpf(1.0f, -*mbits), *emax);
}

/* Element cast with saturation (elem.round(y, saturate=True)): the page's
 * magnitude rule (step 2^(max(e, emin) - M), ties to even, saturate at max),
 * sign kept (-0 included), +-Inf -> +-max.
 * READING: these formats cannot hold NaN; a NaN element encodes to +0, as NaN
 * does in the integer formats. */
uint8_t orc_narrow_encode(float y, int elem) {
    int ebits, mbits, bias, emax;
    float maxv;
    narrow_format(elem, &ebits, &mbits, &bias, &emax, &maxv);
    if (isnan(y)) return 0;
    uint8_t sign = signbit(y) ? (uint8_t)(1u << (ebits + mbits)) : 0;
    float a = fabsf(y);
    float m = isinf(a) ? maxv : fp8_round_magnitude(a, mbits, bias, maxv);
    return fp8_bits(m, sign, mbits, bias);
}

float orc_narrow_decode(uint8_t code, int elem) {
    int ebits, mbits, bias, emax;
    float maxv;
    narrow_format(elem, &ebits, &mbits, &bias, &emax, &maxv);
    uint32_t E = (code >> mbits) & ((1u << ebits) - 1u);
    uint32_t M = code & ((1u << mbits) - 1u);
    float v = E == 0 ? ldexpf((float)M, 1 - bias - mbits) : ldexpf(1.0f + (float)M / (float)(1 << mbits), (int)E - bias);
    return (code >> (ebits + mbits)) & 1u ? -v : v;
}

/* [CS] block_scaled(x, elem, 32, "e8m0") along rows, as orc_mxfp8_rows with the
 * element's emax: X = 2^(k - 1 - emax), k from frexp of the block's finite amax
 * (amax 0 taken as 1), exponent clamped below at -127, E8M0 byte = exponent +
 * 127; q = elem(x / X), fq = decode(q) * X.
 * Layouts: q for E2M1 is packed two codes per byte, ceil(cols/2) bytes per row,
 * the even column in the high nibble (the nibble order of the 4-bit integer
 * codes); for E2M3 / E3M2 one code per byte [rows, cols] (low six bits); e8m0:
 * [rows, ceil(cols/32)]; fq (NULL allowed): float32 [rows, cols]. */
void orc_mx_rows(const void* x, int dtype, int64_t rows, int64_t cols, int elem, uint8_t* q, uint8_t* e8m0,
                 float* fq) {
    int ebits, mbits, bias, emax;
    float maxv;
    narrow_format(elem, &ebits, &mbits, &bias, &emax, &maxv);
    int64_t nbr = (cols + MX_BLOCK - 1) / MX_BLOCK;
    int64_t pstride = (cols + 1) / 2;
    if (elem == ORC_E2M1) memset(q, 0, (size_t)(rows * pstride));
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nbr; ++b) {
            int64_t c0 = b * MX_BLOCK;
            int64_t c1 = c0 + MX_BLOCK < cols ? c0 + MX_BLOCK : cols;
            float amax = 0.0f;
            for (int64_t c = c0; c < c1; ++c) {
                float a = fabsf(widen(x, dtype, r * cols + c));
                if (isfinite(a) && a > amax) amax = a;
            }
            int k;
            frexpf(amax > 0.0f ? amax : 1.0f, &k);
            int xe = k - 1 - emax;
            if (xe < -127) xe = -127;
            float X = ldexpf(1.0f, xe);
            e8m0[r * nbr + b] = (uint8_t)(xe + 127);
            for (int64_t c = c0; c < c1; ++c) {
                uint8_t code = orc_narrow_encode(widen(x, dtype, r * cols + c) / X, elem);
                if (elem == ORC_E2M1) q[r * pstride + c / 2] |= (c % 2 == 0) ? (uint8_t)(code << 4) : code;
                else q[r * cols + c] = code;
                if (fq) fq[r * cols + c] = orc_narrow_decode(code, elem) * X;
            }
        }
    }
}

/* [CS] block_scaled(x, FP4_E2M1, 16, "e4m3") over the flattened tensor (the
 * page's nvfp4_quantize): tensor scale g = amax(x) / (6 * 448); block scale
 * s = E4M3(amax_block / 6 / g) with saturation, X = s * g, and X = 1 where that
 * is not > 0; elements y = x / X cast to E2M1, fq = decode * X.
 * READINGS: binary32 throughout, one rounding per operation, in the page's
 * order; amax over finite elements; a partial last block when n % 16 != 0.
 * q: packed E2M1 codes, ceil(n/2) bytes (even element in the high nibble);
 * sbytes: the E4M3 byte of s per block, ceil(n/16); *g: the tensor scale. */
#define NV_BLOCK 16
void orc_nvfp4(const float* x, int64_t n, uint8_t* q, uint8_t* sbytes, float* g_out, float* fq) {
    float g = orc_amax_finite(x, n) / (6.0f * 448.0f);
    *g_out = g;
    memset(q, 0, (size_t)((n + 1) / 2));
    int64_t nb = (n + NV_BLOCK - 1) / NV_BLOCK;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t i0 = b * NV_BLOCK, i1 = i0 + NV_BLOCK < n ? i0 + NV_BLOCK : n;
        float amax = 0.0f;
        for (int64_t i = i0; i < i1; ++i) {
            float a = fabsf(x[i]);
            if (isfinite(a) && a > amax) amax = a;
        }
        float ratio = amax / 6.0f / g;
        uint8_t sb = orc_fp8_encode(ratio, ORC_E4M3);
        float s = orc_fp8_decode(sb, ORC_E4M3);
        float X = s * g;
        if (!(X > 0.0f)) X = 1.0f;
        sbytes[b] = sb;
        for (int64_t i = i0; i < i1; ++i) {
            uint8_t code = orc_narrow_encode(x[i] / X, ORC_E2M1);
            q[i / 2] |= (i % 2 == 0) ? (uint8_t)(code << 4) : code;
            if (fq) fq[i] = orc_narrow_decode(code, ORC_E2M1) * X;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Stochastic rounding: [QAT] module docs "Rounding modes",                    */
/* RoundingMode::Stochastic (round_to_int), quantize, fp8_quantize_magnitude   */
/* ------------------------------------------------------------------------- */

/* Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC'11).  One round maps the counter
 * (c0, c1, c2, c3) with key (k0, k1) to
 *   (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0))
 * where hi / lo are the halves of the 64-bit product; the key grows by the Weyl
 * constants (W0, W1) between rounds; ten rounds. */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* The uniform [0, 1) variate of element index i (the page draws one per rounded
 * element from a sequential Rng).
 * READING: the variate is a function of (seed, i), so any split of a tensor draws
 * the same numbers: word i mod 4 of Philox4x32-10 at counter
 * (floor(i/4) mod 2^32, floor(i/4) div 2^32, 0, 0) under key
 * (seed mod 2^32, seed div 2^32), scaled as (word >> 8) * 2^-24 -- a binary32
 * with 24 random bits, exactly representable. */
float orc_sr_uniform(uint64_t seed, uint64_t i) {
    uint64_t b = i >> 2;
    uint32_t ctr[4] = {(uint32_t)b, (uint32_t)(b >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    return (float)(w[i & 3] >> 8) * 0x1p-24f;
}

/* [QAT] RoundingMode::Stochastic: floor(t) + 1 when the draw is below the
 * fractional part, floor(t) otherwise.
 * READING: binary32 throughout, frac = fl(t - floor(t)) compared with the 24-bit
 * draw u (so the probability of rounding up is ceil(frac 2^24) / 2^24). */
static float round_stochastic(float t, float u) {
    float lower = floorf(t);
    float frac = t - lower;
    return u < frac ? lower + 1.0f : lower;
}

/* [QAT] quantize with RoundingMode::Stochastic.  Same readings as orc_quantize
 * (the quotient is rounded, then the integer zero-point is added; scale 0 and a
 * NaN quotient give code 0; +-Inf clamp to the range ends). */
int32_t orc_quantize_sr(float x, float scale, int32_t zp, int32_t qmin, int32_t qmax, float u) {
    if (scale == 0.0f) return 0;
    float t = x / scale;
    if (isnan(t)) return 0;
    double r = isinf(t) ? (double)t : (double)round_stochastic(t, u);
    double v = r + (double)zp;
    if (v < (double)qmin) v = (double)qmin;
    if (v > (double)qmax) v = (double)qmax;
    return (int32_t)v;
}

/* [QAT] fake_quant_int with RoundingMode::Stochastic; element i of x uses the
 * variate of index offset + i.  Either output may be NULL. */
void orc_fake_quant_int_sr(const float* x, int64_t n, int bits, int scheme, float scale, int32_t zp,
                           uint64_t seed, uint64_t offset, int8_t* codes, float* fq) {
    int32_t qmin, qmax;
    if (orc_q_range(bits, scheme, &qmin, &qmax) != 0) return;
    for (int64_t i = 0; i < n; ++i) {
        float u = orc_sr_uniform(seed, offset + (uint64_t)i);
        int32_t q = orc_quantize_sr(x[i], scale, zp, qmin, qmax, u);
        if (codes) codes[i] = (int8_t)q;
        if (fq) fq[i] = orc_dequantize(q, scale, zp);
    }
}

/* [QAT] fp8_quantize_magnitude with RoundingMode::Stochastic: the ratio a / step
 * (exact) is rounded stochastically, then saturated as for Nearest. */
static float fp8_round_magnitude_sr(float a, int mbits, int bias, float maxv, float u) {
    if (a == 0.0f) return 0.0f;
    int emin = 1 - bias;
    int e = floor_log2(a);
    int step_exp = (e > emin ? e : emin) - mbits;
    float step = ldexpf(1.0f, step_exp);
    float m = round_stochastic(a / step, u) * step;
    return m > maxv ? maxv : m;
}

/* [QAT] fake_quant_fp8 with RoundingMode::Stochastic, then the byte encoding of
 * orc_fp8_encode (NaN -> 0x7F, +-Inf -> +-max, sign kept). */
uint8_t orc_fp8_encode_sr(float y, int fmt, float u) {
    int mbits, ebits, bias;
    float maxv;
    fp8_format(fmt, &mbits, &ebits, &bias, &maxv);
    if (isnan(y)) return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    float a = fabsf(y);
    float m = isinf(a) ? maxv : fp8_round_magnitude_sr(a, mbits, bias, maxv, u);
    return fp8_bits(m, sign, mbits, bias);
}

/* Per-tensor fp8 quantize / fake-quant with stochastic rounding: byte =
 * encode_sr(x / scale), fq = decode(byte) * scale; a zero scale gives byte 0;
 * element i uses the variate of index offset + i.  Either output may be NULL. */
void orc_fp8_quantize_sr(const float* x, int64_t n, int fmt, float scale, uint64_t seed,
                         uint64_t offset, uint8_t* q, float* fq) {
    for (int64_t i = 0; i < n; ++i) {
        float u = orc_sr_uniform(seed, offset + (uint64_t)i);
        uint8_t b = scale == 0.0f ? 0 : orc_fp8_encode_sr(x[i] / scale, fmt, u);
        if (q) q[i] = b;
        if (fq) fq[i] = orc_fp8_decode(b, fmt) * scale;
    }
}

/* Variates of indices offset .. offset + n - 1 (for tests of the stream). */
void orc_sr_uniform_n(uint64_t seed, uint64_t offset, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_sr_uniform(seed, offset + (uint64_t)i);
}

/* ------------------------------------------------------------------------- */
/* QAT step: [QAT] QatOptimizer::step (AdamW master update) and requantize     */
/* ------------------------------------------------------------------------- */

/* Bias corrections 1 - beta1^t and 1 - beta2^t for step t >= 1.
 * READING: the page forms them in f64 (beta.powi(t)); here they are formed in
 * double from the binary32 betas and rounded to binary32 once. */
void orc_adamw_bias_corrections(float beta1, float beta2, int64_t t, float* bc1, float* bc2) {
    *bc1 = (float)(1.0 - pow((double)beta1, (double)t));
    *bc2 = (float)(1.0 - pow((double)beta2, (double)t));
}

/* [QAT] QatOptimizer::step, the master update, element by element in the page's
 * order (READING: binary32, one rounding per operation, left to right):
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g g;
 *   m_hat = m / bc1;  v_hat = v / bc2;
 *   if wd != 0: w = w - lr wd w   (decoupled weight decay, before the step);
 *   w = w - lr m_hat / (sqrt(v_hat) + eps). */
void orc_adamw_update(float* w, const float* g, float* m, float* v, int64_t n, float lr, float beta1,
                      float beta2, float eps, float wd, float bc1, float bc2) {
    const float c1 = 1.0f - beta1, c2 = 1.0f - beta2, lrwd = lr * wd;
    for (int64_t i = 0; i < n; ++i) {
        float mi = beta1 * m[i] + c1 * g[i];
        float vi = beta2 * v[i] + c2 * g[i] * g[i];
        m[i] = mi;
        v[i] = vi;
        float m_hat = mi / bc1;
        float v_hat = vi / bc2;
        float wi = w[i];
        if (wd != 0.0f) wi = wi - lrwd * wi;
        wi = wi - lr * m_hat / (sqrtf(v_hat) + eps);
        w[i] = wi;
    }
}

/* [QAT] QatOptimizer::step with an integer target: the update, then requantize:
 * QuantParams::per_tensor_minmax of the updated master (finite min / max, flags
 * as orc_tensor_params_int) and fake_quant_int with the rounding mode
 * (0 nearest, 1 stochastic with the stream of orc_sr_uniform at offset + i).
 * Outputs: params (scale, zp, real_min, real_max), codes (int8 per element, may
 * be NULL), view = the fake-quant view. */
uint32_t orc_qat_step_int(float* w, const float* g, float* m, float* v, int64_t n, float lr, float beta1,
                          float beta2, float eps, float wd, int64_t t, int bits, int scheme, int rounding,
                          uint64_t seed, uint64_t offset, float* scale, int32_t* zp, float* lo, float* hi,
                          int8_t* codes, float* view) {
    float bc1, bc2;
    orc_adamw_bias_corrections(beta1, beta2, t, &bc1, &bc2);
    orc_adamw_update(w, g, m, v, n, lr, beta1, beta2, eps, wd, bc1, bc2);
    uint32_t flags = orc_tensor_params_int(w, n, bits, scheme, scale, zp, lo, hi);
    if (rounding == 0) orc_fake_quant_int(w, n, bits, scheme, *scale, *zp, codes, view);
    else orc_fake_quant_int_sr(w, n, bits, scheme, *scale, *zp, seed, offset, codes, view);
    return flags;
}

/* [QAT] QatOptimizer::step with an fp8 target: the update, then fake_quant_fp8 of
 * the master itself (the page's fp8 view has no scale): byte = encode(w) or
 * encode_sr(w, u), view = decode(byte).  q (may be NULL): the bytes. */
void orc_qat_step_fp8(float* w, const float* g, float* m, float* v, int64_t n, float lr, float beta1,
                      float beta2, float eps, float wd, int64_t t, int fmt, int rounding, uint64_t seed,
                      uint64_t offset, uint8_t* q, float* view) {
    float bc1, bc2;
    orc_adamw_bias_corrections(beta1, beta2, t, &bc1, &bc2);
    orc_adamw_update(w, g, m, v, n, lr, beta1, beta2, eps, wd, bc1, bc2);
    for (int64_t i = 0; i < n; ++i) {
        uint8_t b = rounding == 0 ? orc_fp8_encode(w[i], fmt)
                                  : orc_fp8_encode_sr(w[i], fmt, orc_sr_uniform(seed, offset + (uint64_t)i));
        if (q) q[i] = b;
        if (view) view[i] = orc_fp8_decode(b, fmt);
    }
}
