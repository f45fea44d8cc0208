/*
 * rmsq_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, float64 CPU reference for fused (residual +) RMSNorm with
 * dynamic FP8 (per-row scale) or block-scaled FP4 (E2M1 + E4M3 per 16
 * elements) quantization.  It exists to check the GPU library; nothing in the
 * product may call it.  It shares no code, header, table or constant with the
 * GPU path: every format is rebuilt here from its bit-level definition.
 *
 * Sources of the definitions (cited by page title and section):
 *   [P1] Mojo docs, "rms_norm_fused_fp8": in/out/scales dtype lists,
 *        per-row dynamic scales, epsilon, weight_offset, scale_ub arguments.
 *   [P2] Mojo docs, "allreduce_residual_rmsnorm_fp8": residual input and the
 *        pre-norm sum written to residual_output; weight_offset described as
 *        an additive offset to gamma.
 *   [P3] FlashInfer "rmsnorm_fp4quant.py": section "Constants" (E2M1 max 6,
 *        E4M3 max 448, 16 elements per scale), section "FP8 E4M3 Intrinsics"
 *        (round-to-nearest-even with saturation to the largest finite value,
 *        decode of scale code 0 gives a zero reciprocal), section "E2M1
 *        Conversion" (same rounding, element 2k in the low nibble),
 *        kernel "Phase 2" (mean of squares over the full row, reciprocal
 *        square root of mean + eps) and "Phase 3" (block scale =
 *        global_scale * block_amax / 6 clamped to 448, then RNE to E4M3;
 *        quantize with global_scale / decoded_scale); section "UE8M0
 *        Intrinsics (for MXFP4)" (scale code = ceil(log2(v)) + 127 clamped
 *        to [0, 255], zero for v <= 0; element factor 2^(127 - code), zero
 *        for code 0; no global scale) and the kernel's constructor and API
 *        docstring (block_size 16 or 32, scale_format e4m3 or ue8m0).
 *
 * Readings where the pages are silent or disagree (each listed in the
 * project's design notes):
 *   - y = s * rstd * (gamma + weight_offset), all in float64.
 *   - FP8 scale is a dequant scale: sc = min(amax(|y|) / FMAX, scale_ub);
 *     FMAX = 448 (e4m3fn) or 240 (e4m3fnuz).  Codes use the STORED scale.
 *   - A zero scale quantizes with factor 0 (q = y * 0, sign kept).
 *   - Where floating point decides an integer code, the decision is taken on
 *     the value rounded to fp32 (the precision the conversion instructions
 *     on the pages and in the kernel take), after an exact float64 path.
 *   - Residual: s = round_to_in_dtype(x + r) (exact sum, one rounding) and
 *     the normalized value is this stored s.
 *   - FP4 page-compatible mode (optional): the product s * g' is rounded once
 *     to the input type before the rstd scaling, as [P3]'s kernel multiplies
 *     x and w in 16 bits; everything else stays exact.
 *
 * Formats (magnitude code m = (exponent field << mbits) | mantissa field):
 *   E4M3FN  : 4 exp bits, 3 mantissa, bias 7, largest finite code 0x7E = 448,
 *             sign in bit 7, negative zero 0x80 exists.
 *   E4M3FNUZ: 4 exp bits, 3 mantissa, bias 8, largest finite code 0x7F = 240,
 *             code 0x80 is NaN, so a zero result is always 0x00.
 *   E2M1    : 2 exp bits, 1 mantissa, bias 1, largest code 7 = 6.0, sign in
 *             bit 3.
 *   UE8M0   : 8 exponent bits, no sign, no mantissa: code c stands for
 *             2^(c - 127); used only as a block scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- dtype and format identifiers private to the oracle ---------------- */
enum { ORQ_F32 = 0, ORQ_F16 = 1, ORQ_BF16 = 2 };
enum { ORQ_E4M3FN = 0, ORQ_E4M3FNUZ = 1, ORQ_E2M1 = 2, ORQ_UE8M0 = 3 };
enum { ORQ_SF_E4M3 = 0, ORQ_SF_UE8M0 = 1 }; /* FP4 block-scale formats */

typedef struct {
    int ebits, mbits, bias;
    int max_mag;      /* largest finite magnitude code */
    int sign_bit;     /* bit position of the sign */
    int has_neg_zero; /* 0 for fnuz */
} minifloat;

static minifloat fmt_of(int fmt) {
    minifloat f;
    switch (fmt) {
    case ORQ_E4M3FN:   f.ebits = 4; f.mbits = 3; f.bias = 7; f.max_mag = 0x7E; f.sign_bit = 7; f.has_neg_zero = 1; break;
    case ORQ_E4M3FNUZ: f.ebits = 4; f.mbits = 3; f.bias = 8; f.max_mag = 0x7F; f.sign_bit = 7; f.has_neg_zero = 0; break;
    default:           f.ebits = 2; f.mbits = 1; f.bias = 1; f.max_mag = 7;    f.sign_bit = 3; f.has_neg_zero = 1; break;
    }
    return f;
}

/* Value of a magnitude code, straight from the exponent/mantissa definition. */
static double mag_value(const minifloat* f, int m) {
    int e = m >> f->mbits;
    int man = m & ((1 << f->mbits) - 1);
    if (e == 0) /* subnormal: man * 2^(1 - bias - mbits) */
        return ldexp((double)man, 1 - f->bias - f->mbits);
    return ldexp((double)((1 << f->mbits) + man), e - f->bias - f->mbits);
}

/* UE8M0 block scale of a value v ([P3] "UE8M0 Intrinsics"): the exponent of
 * the smallest power of two >= v, biased by 127 and clamped to [0, 255];
 * v <= 0 (or NaN) gives 0.  frexp splits v = m * 2^e with m in [0.5, 1), so
 * ceil(log2(v)) is e, or e - 1 when m is exactly 0.5 (v = 2^(e-1)). */
static int ue8m0_encode(double v) {
    if (!(v > 0.0)) return 0;
    if (isinf(v)) return 255;
    int e;
    double m = frexp(v, &e);
    int c = (m == 0.5 ? e - 1 : e) + 127;
    return c < 0 ? 0 : (c > 255 ? 255 : c);
}

/* The factor elements of a UE8M0-scaled block are multiplied by:
 * 1 / 2^(code - 127) = 2^(127 - code), and 0 for code 0 ([P3] "UE8M0
 * Intrinsics", its zero check). */
static double ue8m0_inverse(int code) { return code == 0 ? 0.0 : ldexp(1.0, 127 - code); }

double oracle_decode(int fmt, int code) {
    if (fmt == ORQ_UE8M0) return ldexp(1.0, code - 127);
    minifloat f = fmt_of(fmt);
    int sign = (code >> f.sign_bit) & 1;
    int m = code & ((1 << f.sign_bit) - 1);
    if (fmt == ORQ_E4M3FN && m == 0x7F) return NAN;
    if (fmt == ORQ_E4M3FNUZ && code == 0x80) return NAN;
    double v = mag_value(&f, m);
    return sign ? -v : v;
}

/* Round to the nearest representable magnitude, ties to the even code,
 * saturating to the largest finite value.  Sign is the sign bit of v.
 * Found by walking the ordered magnitude codes: slow and plain. */
int oracle_encode(int fmt, double v) {
    if (fmt == ORQ_UE8M0) return ue8m0_encode(v);
    minifloat f = fmt_of(fmt);
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    int m;
    if (isnan(v)) return fmt == ORQ_E4M3FNUZ ? 0x80 : (fmt == ORQ_E4M3FN ? 0x7F : 0); /* outside the contract */
    if (a >= mag_value(&f, f.max_mag)) {
        m = f.max_mag;
    } else {
        m = 0;
        while (m + 1 <= f.max_mag && mag_value(&f, m + 1) <= a) m++;
        /* now value(m) <= a < value(m+1) */
        double lo = mag_value(&f, m), hi = mag_value(&f, m + 1);
        double dlo = a - lo, dhi = hi - a;
        if (dhi < dlo) m = m + 1;
        else if (dhi == dlo && (m & 1)) m = m + 1;
    }
    if (m == 0 && !f.has_neg_zero) return 0;
    return m | (neg << f.sign_bit);
}

/* ---- IEEE binary16 / bfloat16 / binary32 rounding from float64 --------- */

/* Round-half-even of a non-negative double to an integer-valued double. */
static double round_half_even(double t) {
    double fl = floor(t);
    double diff = t - fl;
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;
}

/* Round |v| to a binary format with p significant bits and minimum normal
 * exponent emin (exponent of the leading bit).  Overflow is not handled
 * here (callers stay in range). */
static double round_binary(double v, int p, int emin) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    double a = fabs(v);
    int ex;
    frexp(a, &ex);          /* a = fr * 2^ex, fr in [0.5, 1): leading bit at ex-1 */
    int lead = ex - 1;
    if (lead < emin) lead = emin; /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, lead - (p - 1));
    double r = round_half_even(a / quantum) * quantum;
    return v < 0 ? -r : r;
}

static uint16_t bits_bf16(double v) {
    /* bfloat16: 8 significant bits, emin -126; every bf16 value is an fp32
     * value whose low 16 bits are zero. */
    double r = round_binary(v, 8, -126);
    if (fabs(r) > 3.3895313892515355e38) /* beyond the largest finite: inf */
        return signbit(r) ? 0xFF80 : 0x7F80;
    float rf = (float)r; /* exact */
    uint32_t u;
    memcpy(&u, &rf, 4);
    return (uint16_t)(u >> 16);
}

static uint16_t bits_f16(double v) {
    /* binary16: 11 significant bits, emin -14, max 65504, exponent bias 15. */
    double r = round_binary(v, 11, -14);
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (a > 65504.0) return sign | 0x7C00;
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int lead = ex - 1;
    if (lead < -14) { /* subnormal: a = man * 2^-24 */
        return sign | (uint16_t)(a / ldexp(1.0, -24));
    }
    uint16_t efield = (uint16_t)(lead + 15);
    uint16_t man = (uint16_t)((a / ldexp(1.0, lead) - 1.0) * 1024.0);
    return sign | (uint16_t)(efield << 10) | man;
}

static double value_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double value_f16(uint16_t b) {
    int sign = b >> 15, e = (b >> 10) & 0x1F, man = b & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)man, -24);
    else if (e == 31) v = man ? NAN : INFINITY;
    else v = ldexp((double)(1024 + man), e - 15 - 10);
    return sign ? -v : v;
}

uint16_t oracle_round_bf16(double v) { return bits_bf16(v); }
uint16_t oracle_round_f16(double v) { return bits_f16(v); }
double oracle_value_bf16(uint16_t b) { return value_bf16(b); }
double oracle_value_f16(uint16_t b) { return value_f16(b); }

/* Element j of a row stored in dtype dt, widened exactly to double. */
static double load_elem(int dt, const void* p, int64_t i) {
    if (dt == ORQ_F32) return (double)((const float*)p)[i];
    if (dt == ORQ_F16) return value_f16(((const uint16_t*)p)[i]);
    return value_bf16(((const uint16_t*)p)[i]);
}

/* Round v to dtype dt, store its bits at element i, return the stored value. */
static double store_elem(int dt, void* p, int64_t i, double v) {
    if (dt == ORQ_F32) {
        float f = (float)v; /* IEEE conversion: round to nearest even */
        ((float*)p)[i] = f;
        return (double)f;
    }
    if (dt == ORQ_F16) {
        uint16_t b = bits_f16(v);
        ((uint16_t*)p)[i] = b;
        return value_f16(b);
    }
    uint16_t b = bits_bf16(v);
    ((uint16_t*)p)[i] = b;
    return value_bf16(b);
}

/* ---- the row pipeline --------------------------------------------------- */

/* Steps shared by both outputs, one row: s (optionally x + residual, rounded
 * and written to residual_out), then y = s * rstd * (gamma + offset).
 * Returns rstd.  s and y are caller buffers of length hidden. */
/* The product s * g' rounded once to the input type ([P3] kernel: it
 * multiplies x and w as 16-bit pairs, mul.bf16x2 / mul.f16x2, before scaling
 * by rstd); fp32 inputs are rounded to fp32.  Used by the FP4 path's
 * page-compatible mode only. */
static double round_to_dt(int dt, double v) {
    if (dt == ORQ_F32) return (double)(float)v;
    if (dt == ORQ_F16) return value_f16(bits_f16(v));
    return value_bf16(bits_bf16(v));
}

static double norm_row_mode(int64_t hidden, int in_dt, const void* x, const void* residual,
                            void* residual_out, const void* gamma, double eps, double offset,
                            int round_product, double* s, double* y);

static double norm_row(int64_t hidden, int in_dt, const void* x, const void* residual,
                       void* residual_out, const void* gamma, double eps, double offset,
                       double* s, double* y) {
    return norm_row_mode(hidden, in_dt, x, residual, residual_out, gamma, eps, offset, 0, s, y);
}

/* With round_product, y = round_to_dt(s * g') * rstd (the FP4 page's order);
 * otherwise y = s * rstd * g'. */
static double norm_row_mode(int64_t hidden, int in_dt, const void* x, const void* residual,
                            void* residual_out, const void* gamma, double eps, double offset,
                            int round_product, double* s, double* y) {
    for (int64_t j = 0; j < hidden; j++) {
        double xj = load_elem(in_dt, x, j);
        if (residual) {
            double rj = load_elem(in_dt, residual, j);
            s[j] = store_elem(in_dt, residual_out, j, xj + rj);
        } else {
            s[j] = xj;
        }
    }
    double sumsq = 0.0;
    for (int64_t j = 0; j < hidden; j++) sumsq += s[j] * s[j];
    double mean_sq = sumsq / (double)hidden;  /* mean over the full row */
    double rstd = 1.0 / sqrt(mean_sq + eps);
    for (int64_t j = 0; j < hidden; j++) {
        double g = load_elem(in_dt, gamma, j) + offset;
        y[j] = round_product ? round_to_dt(in_dt, s[j] * g) * rstd : s[j] * rstd * g;
    }
    return rstd;
}

/* FP8 per-row quantization.
 *   x, residual, residual_out: [rows, hidden] in in_dt (residual may be NULL,
 *   then residual_out is ignored); gamma: [hidden] in in_dt.
 *   out: [rows, hidden] FP8 codes; scales: [rows] in scales_dt.
 *   q_out (optional): [rows, hidden] the unrounded float64 quantizer input.
 *   sc_out (optional): [rows] the unrounded float64 scale (after the clamp).
 * Returns 0, or -1 on allocation failure. */
int oracle_rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dt,
                       const void* x, const void* residual, void* residual_out,
                       const void* gamma, double eps, double offset, double scale_ub,
                       int out_fmt, uint8_t* out, int scales_dt, void* scales,
                       double* q_out, double* sc_out) {
    minifloat f = fmt_of(out_fmt);
    const double fmt_max = mag_value(&f, f.max_mag);
    size_t esz = in_dt == ORQ_F32 ? 4 : 2;
    double* s = (double*)malloc(sizeof(double) * (size_t)hidden);
    double* y = (double*)malloc(sizeof(double) * (size_t)hidden);
    if (!s || !y) { free(s); free(y); return -1; }
    for (int64_t r = 0; r < rows; r++) {
        const char* xr = (const char*)x + (size_t)r * hidden * esz;
        const char* rr = residual ? (const char*)residual + (size_t)r * hidden * esz : NULL;
        char* ro = residual ? (char*)residual_out + (size_t)r * hidden * esz : NULL;
        norm_row(hidden, in_dt, xr, rr, ro, gamma, eps, offset, s, y);

        double amax = 0.0;
        for (int64_t j = 0; j < hidden; j++)
            if (fabs(y[j]) > amax) amax = fabs(y[j]);
        double sc = amax / fmt_max;
        if (sc > scale_ub) sc = scale_ub;
        if (sc_out) sc_out[r] = sc;
        /* stored scale: decision on the fp32 value, then the scales dtype */
        double sc_st = store_elem(scales_dt, scales, r, (double)(float)sc);
        for (int64_t j = 0; j < hidden; j++) {
            double q = sc_st > 0.0 ? y[j] / sc_st : y[j] * 0.0;
            if (q_out) q_out[r * hidden + j] = q;
            out[r * hidden + j] = (uint8_t)oracle_encode(out_fmt, (double)(float)q);
        }
    }
    free(s);
    free(y);
    return 0;
}

/* FP4 block-scaled quantization ([P3] "Phase 3"), blocks of `block` (16 or
 * 32) consecutive elements of a row, one scale per block:
 *   sfmt ORQ_SF_E4M3 : scale = min(gs * amax / 6, 448) rounded to E4M3FN,
 *                      element factor gs / decoded scale (0 if it is 0);
 *   sfmt ORQ_SF_UE8M0: scale code = UE8M0(amax / 6), element factor
 *                      2^(127 - code) (0 for code 0); gs is not used.
 * Elements are then E2M1 codes of y * factor (saturating RNE).
 *   x, residual, residual_out: [rows, hidden] in in_dt; with a residual the
 *   row is s = round_to_in_dt(x + r), written to residual_out, as in the FP8
 *   path ([P2] residual_output; the FP4 page has no residual, so this pairs
 *   its quantizer with [P2]'s pre-norm sum).  residual may be NULL.
 *   round_product: the FP4 page's numerics -- s * g' is rounded once to the
 *   input type before the rstd scaling ([P3] kernel, 16-bit x * w).
 *   out: [rows, hidden/2] bytes, element 2k in the low nibble of byte k.
 *   block_scales: [rows, hidden/block] scale codes, row-major.
 *   global_scale: the fp32 value, widened.
 *   q_out (optional): [rows, hidden] unrounded float64 quantizer input.
 *   sf_out (optional): [rows, hidden/block] unrounded float64 block scale
 *   (after the clamp to 448 for E4M3; amax / 6 for UE8M0).
 * Returns 0, -1 on allocation failure, -2 on a bad hidden / block / format. */
int oracle_rmsnorm_fp4q(int64_t rows, int64_t hidden, int in_dt,
                        const void* x, const void* residual, void* residual_out,
                        const void* gamma, double eps, double offset,
                        double global_scale, int block, int sfmt, int round_product,
                        uint8_t* out, uint8_t* block_scales, double* q_out, double* sf_out) {
    minifloat e4m3 = fmt_of(ORQ_E4M3FN), e2m1 = fmt_of(ORQ_E2M1);
    const double e4m3_max = mag_value(&e4m3, e4m3.max_mag); /* 448 */
    const double e2m1_max = mag_value(&e2m1, e2m1.max_mag); /* 6 */
    if ((block != 16 && block != 32) || (sfmt != ORQ_SF_E4M3 && sfmt != ORQ_SF_UE8M0)) return -2;
    if (hidden % block) return -2;
    size_t esz = in_dt == ORQ_F32 ? 4 : 2;
    int64_t nblk = hidden / block;
    double* s = (double*)malloc(sizeof(double) * (size_t)hidden);
    double* y = (double*)malloc(sizeof(double) * (size_t)hidden);
    int* c = (int*)malloc(sizeof(int) * (size_t)hidden);
    if (!s || !y || !c) { free(s); free(y); free(c); return -1; }
    for (int64_t r = 0; r < rows; r++) {
        const char* xr = (const char*)x + (size_t)r * hidden * esz;
        const char* rr = residual ? (const char*)residual + (size_t)r * hidden * esz : NULL;
        char* ro = residual ? (char*)residual_out + (size_t)r * hidden * esz : NULL;
        norm_row_mode(hidden, in_dt, xr, rr, ro, gamma, eps, offset, round_product, s, y);
        for (int64_t b = 0; b < nblk; b++) {
            double amax = 0.0;
            for (int k = 0; k < block; k++)
                if (fabs(y[b * block + k]) > amax) amax = fabs(y[b * block + k]);
            double sf, d = 0.0, inv = 0.0;
            int S;
            if (sfmt == ORQ_SF_E4M3) {
                sf = global_scale * amax / e2m1_max;
                if (sf > e4m3_max) sf = e4m3_max;
                S = oracle_encode(ORQ_E4M3FN, (double)(float)sf);
                d = oracle_decode(ORQ_E4M3FN, S);
            } else {
                sf = amax / e2m1_max;
                S = ue8m0_encode((double)(float)sf);
                inv = ue8m0_inverse(S); /* a power of two: y * inv is exact */
            }
            if (sf_out) sf_out[r * nblk + b] = sf;
            block_scales[r * nblk + b] = (uint8_t)S;
            for (int k = 0; k < block; k++) {
                int64_t j = b * block + k;
                /* a zero factor keeps the sign of y */
                double q = sfmt == ORQ_SF_UE8M0 ? y[j] * inv : (d > 0.0 ? y[j] * global_scale / d : y[j] * 0.0);
                if (q_out) q_out[r * hidden + j] = q;
                c[j] = oracle_encode(ORQ_E2M1, (double)(float)q);
            }
        }
        for (int64_t k = 0; k < hidden / 2; k++)
            out[r * (hidden / 2) + k] = (uint8_t)(c[2 * k] | (c[2 * k + 1] << 4));
    }
    free(s);
    free(y);
    free(c);
    return 0;
}

/* The page's default configuration: 16-element blocks, E4M3 scales. */
int oracle_rmsnorm_fp4(int64_t rows, int64_t hidden, int in_dt,
                       const void* x, const void* gamma, double eps, double offset,
                       double global_scale, uint8_t* out, uint8_t* block_scales,
                       double* q_out, double* sf_out) {
    return oracle_rmsnorm_fp4q(rows, hidden, in_dt, x, NULL, NULL, gamma, eps, offset, global_scale, 16,
                               ORQ_SF_E4M3, 0, out, block_scales, q_out, sf_out);
}

/* The normalized values y = s * rstd * (gamma + offset) as float64
 * ([rows, hidden]); residual may be NULL.  residual_out is written when
 * residual is given.  rstd_out (optional): [rows]. */
int oracle_rmsnorm_y(int64_t rows, int64_t hidden, int in_dt,
                     const void* x, const void* residual, void* residual_out,
                     const void* gamma, double eps, double offset, int round_product,
                     double* y_out, double* rstd_out) {
    size_t esz = in_dt == ORQ_F32 ? 4 : 2;
    double* s = (double*)malloc(sizeof(double) * (size_t)hidden);
    if (!s) return -1;
    for (int64_t r = 0; r < rows; r++) {
        const char* xr = (const char*)x + (size_t)r * hidden * esz;
        const char* rr = residual ? (const char*)residual + (size_t)r * hidden * esz : NULL;
        char* ro = residual ? (char*)residual_out + (size_t)r * hidden * esz : NULL;
        double rstd = norm_row_mode(hidden, in_dt, xr, rr, ro, gamma, eps, offset, round_product, s,
                                    y_out + r * hidden);
        if (rstd_out) rstd_out[r] = rstd;
    }
    free(s);
    return 0;
}

/* max |y| over all rows (the "global amax" a calibration step would give). */
double oracle_rmsnorm_absmax(int64_t rows, int64_t hidden, int in_dt,
                             const void* x, const void* gamma, double eps, double offset) {
    size_t esz = in_dt == ORQ_F32 ? 4 : 2;
    double* s = (double*)malloc(sizeof(double) * (size_t)hidden);
    double* y = (double*)malloc(sizeof(double) * (size_t)hidden);
    double amax = 0.0;
    if (!s || !y) { free(s); free(y); return -1.0; }
    for (int64_t r = 0; r < rows; r++) {
        const char* xr = (const char*)x + (size_t)r * hidden * esz;
        norm_row(hidden, in_dt, xr, NULL, NULL, gamma, eps, offset, s, y);
        for (int64_t j = 0; j < hidden; j++)
            if (fabs(y[j]) > amax) amax = fabs(y[j]);
    }
    free(s);
    free(y);
    return amax;
}

/* Array forms of the codecs, for tests. */
/* The pre-norm sum of Mojo "allreduce_residual_rmsnorm_fp8" over several
 * input buffers (Args: input_buffers, one per GPU; residual;
 * residual_output): s_i = round_to_dt(residual_i + sum_g inputs[g]_i), the
 * sum exact in float64 (in order: residual, then the inputs) and rounded
 * once.  n elements of each buffer, all in dt.  ninputs >= 1. */
void oracle_sum_round(int dt, int ninputs, const void* const* inputs, const void* residual, int64_t n,
                      void* out) {
    for (int64_t i = 0; i < n; i++) {
        double s = load_elem(dt, residual, i);
        for (int g = 0; g < ninputs; g++) s += load_elem(dt, inputs[g], i);
        store_elem(dt, out, i, s);
    }
}

void oracle_encode_array(int fmt, const double* v, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)oracle_encode(fmt, v[i]);
}

void oracle_decode_array(int fmt, const uint8_t* codes, int64_t n, double* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_decode(fmt, codes[i]);
}

void oracle_round_array(int dt, const double* v, int64_t n, void* out) {
    for (int64_t i = 0; i < n; i++) store_elem(dt, out, i, v[i]);
}

void oracle_value_array(int dt, const void* bits, int64_t n, double* out) {
    for (int64_t i = 0; i < n; i++) out[i] = load_elem(dt, bits, i);
}
