/*
 * mx_oracle.c -- plain CPU reference for MXFP8 block-scaled quantization and
 * the block-scaled matrix product.
 *
 * TEST INFRASTRUCTURE. This file is the yardstick the HIP library is checked
 * against. It shares no code, header, table or helper with that library, and
 * only the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg may load it. Nothing on the product path calls it.
 *
 * Sources (web pages; cited by title and section):
 *   [SM120]  "MXFP8 SM120 software support" (xuesongtap.github.io, 2026-09-22)
 *   [GLOSS]  "MXFP8 quantization" glossary (robocikowo.com)
 *   [FP8DS]  "FP8 训练为什么能稳：把缩放因子的粒度与累加精度算清楚" (magicnetworld.com)
 *   [NVFP4]  "NVFP4 如何用 4 bit 实现高精度" (theluyuan.com)
 *
 * Precision. Every quantity is held in IEEE double. All of them are exact
 * there: bf16/f32 inputs, their power-of-two rescalings, FP8 code values,
 * E8M0 scales, and products of two decoded codes. Rounding happens only where
 * the method rounds: the element encode (to E4M3/E5M2), the dequantize output
 * (to f32/bf16), and the fp64 summation of the matrix product.
 *
 * Readings taken where the pages leave a step open:
 *   - scale rule: X = 2^(floor(log2 amax) - emax_elem), emax_elem = 8 (E4M3),
 *     15 (E5M2); E8M0 code = that exponent + 127 clamped to [0, 254];
 *   - element rounding: round to nearest, ties to even, saturating at the
 *     largest finite magnitude (448 / 57344);
 *   - amax == 0 gives scale code 0 and all-zero codes;
 *   - a block holding NaN or Inf gets scale code 0xFF and element codes 0x7F;
 *   - the sign of x is kept, so negative values that round to zero give 0x80.
 *   - MXFP4 [NVFP4 §2.4, §5.5]: E2M1 elements with the same E8M0 scale per 32
 *     and the same rule (emax_elem = 2, largest finite 6); codes packed two
 *     per byte, element 2i in the low nibble; a NaN/Inf block gets scale
 *     0xFF and element codes 0 (E2M1 has no NaN code).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "mx_oracle.h"

/* ---------------------------------------------------------------------------
 * Element formats. [SM120 §0.1, table of element encodings]: E4M3 has 1 sign,
 * 4 exponent and 3 mantissa bits, largest finite 448, smallest subnormal 2^-9;
 * E5M2 has 1/5/2 bits, largest finite 57344, smallest subnormal 2^-16.
 * [FP8DS §4.1]: the smallest E4M3 normal is 2^-6; [FP8DS §三]: the E5M2 normal
 * range is 57344 * 2^14, so its smallest normal is 2^-14. Together these fix
 * the exponent biases at 7 and 15.
 * ------------------------------------------------------------------------- */
typedef struct {
    int mbits;        /* stored mantissa bits */
    int emin;         /* exponent of the smallest normal */
    int bias;         /* exponent bias */
    double maxfinite; /* largest finite magnitude */
    int emax_elem;    /* floor(log2(maxfinite)), used by the scale rule */
} fp8_format;

static const fp8_format FMT_E4M3 = {3, -6, 7, 448.0, 8};
static const fp8_format FMT_E5M2 = {2, -14, 15, 57344.0, 15};
/* E2M1 (the MXFP4 element) [NVFP4 §2.4]: 1 sign, 2 exponent and 1 mantissa
 * bit, exponent bias 1, exponent field 0 subnormal (0.m); the 8 magnitudes are
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6, so the smallest normal is 2^0 and the largest
 * finite 6 = 1.5 * 2^2. No Inf or NaN encodings. */
static const fp8_format FMT_E2M1 = {1, 0, 1, 6.0, 2};

static const fp8_format* fmt_of(int fmt) {
    return fmt == MXO_E5M2 ? &FMT_E5M2 : fmt == MXO_E2M1 ? &FMT_E2M1 : &FMT_E4M3;
}

/* Code bits of an element and its sign bit. */
static unsigned code_bits(int fmt) { return fmt == MXO_E2M1 ? 4u : 8u; }

/* Value of an E4M3 code: exponent field 0 is subnormal (m * 2^-9); the one
 * pattern S.1111.111 is NaN and there is no infinity [FP8DS §三]. */
double mxo_decode_e4m3(unsigned code) {
    unsigned s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, (int)e - 7);
    return s ? -v : v;
}

/* Value of an E5M2 code: IEEE-style, exponent field 31 holds Inf (m = 0) and
 * NaN (m != 0) [FP8DS §三]; exponent field 0 is subnormal (m * 2^-16). */
double mxo_decode_e5m2(unsigned code) {
    unsigned s = (code >> 7) & 1, e = (code >> 2) & 31, m = code & 3;
    double v;
    if (e == 31) {
        if (m != 0) return NAN;
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -16);
    } else {
        v = ldexp(1.0 + m / 4.0, (int)e - 15);
    }
    return s ? -v : v;
}

/* Value of an E2M1 code [NVFP4 §2.4]: sign bit 3, exponent bits 2-1 with
 * bias 1, mantissa bit 0; exponent field 0 gives 0.m (0 or 0.5). */
double mxo_decode_e2m1(unsigned code) {
    unsigned s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + m / 2.0, (int)e - 1);
    return s ? -v : v;
}

double mxo_decode(int fmt, unsigned code) {
    if (fmt == MXO_E2M1) return mxo_decode_e2m1(code & 0xF);
    return fmt == MXO_E5M2 ? mxo_decode_e5m2(code & 0xFF) : mxo_decode_e4m3(code & 0xFF);
}

/* E8M0 scale: no sign, no mantissa; finite values 2^k for -127 <= k <= 127
 * plus one NaN encoding [SM120 §0.1]; value 2^(e-127) [NVFP4 §5.3]. */
double mxo_decode_e8m0(unsigned e) {
    e &= 0xFF;
    if (e == 255) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* ---------------------------------------------------------------------------
 * Rounding to a binary grid.
 *
 * Round a >= 0 (finite) to the nearest multiple of the local grid spacing of a
 * binary format with `mbits` fraction bits whose smallest normal exponent is
 * `emin` (below it the spacing stays at 2^(emin - mbits): subnormals). Ties go
 * to the even multiple, i.e. to the value whose last mantissa bit is 0.
 * [SM120 §0.1]: elements are rounded to nearest; [FP8DS §4.1] works the
 * subnormal spacing 2^-9 and the half-spacing zero threshold 2^-10 for E4M3.
 * No upper bound is applied here.
 * ------------------------------------------------------------------------- */
static double round_to_grid(double a, int mbits, int emin) {
    if (a == 0.0) return 0.0;
    int e = ilogb(a);
    if (e < emin) e = emin;
    double spacing = ldexp(1.0, e - mbits);
    double units = a / spacing; /* exact: division by a power of two */
    double n = floor(units);
    double rem = units - n;     /* exact */
    if (rem > 0.5 || (rem == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
    return n * spacing;
}

/* Bit pattern of a finite magnitude r that lies on the format's grid. */
static unsigned grid_bits(double r, int mbits, int emin, int bias) {
    if (r < ldexp(1.0, emin)) /* zero or subnormal: exponent field 0 */
        return (unsigned)(r / ldexp(1.0, emin - mbits));
    int e = ilogb(r);
    unsigned m = (unsigned)((ldexp(r, -e) - 1.0) * (double)(1 << mbits));
    return ((unsigned)(e + bias) << mbits) | m;
}

/* Code of the element value nearest to y (ties to even), saturating at the
 * largest finite magnitude; the sign bit is taken from y. E2M1 has no NaN
 * code: a NaN gives code 0 (its block carries the NaN scale). */
unsigned mxo_encode(int fmt, double y) {
    const fp8_format* f = fmt_of(fmt);
    unsigned sign = signbit(y) ? 1u << (code_bits(fmt) - 1) : 0u;
    if (isnan(y)) return fmt == MXO_E2M1 ? 0u : 0x7Fu;
    double a = fabs(y);
    double r = a >= f->maxfinite ? f->maxfinite : round_to_grid(a, f->mbits, f->emin);
    if (r > f->maxfinite) r = f->maxfinite;
    return sign | grid_bits(r, f->mbits, f->emin, f->bias);
}

/* ---------------------------------------------------------------------------
 * Scale selection for one block. [GLOSS]: one shared E8M0 factor per block of
 * 32, usually derived from the block's largest absolute value; [SM120 §0.2]:
 * take the amax of 32 values, choose a power of two that E8M0 can hold, then
 * round x / scale to FP8. The rule itself is left to the implementation
 * [SM120 §0.1]; this file uses X = 2^(floor(log2 amax) - emax_elem).
 * ------------------------------------------------------------------------- */
/* Scale rules. MXO_RULE_FLOOR (the default): X = 2^(floor(log2 amax) -
 * emax_elem), which can leave amax / X up to just under 2 * 2^emax_elem, past
 * the largest finite element, so the block maximum may saturate.
 * MXO_RULE_CEIL: the smallest power of two X with amax / X <= the largest
 * finite element, i.e. X = 2^ceil(log2(amax / maxfinite)), so nothing
 * saturates. The pages note that how the E8M0 scale is chosen and rounded
 * matters for accuracy [GLOSS]; the second rule is that alternative. */
unsigned mxo_scale_code_rule(int fmt, const double* x, int64_t n, int rule) {
    const fp8_format* f = fmt_of(fmt);
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(x[i])) return 0xFFu;
        double a = fabs(x[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0) return 0u;
    int k = ilogb(amax) - f->emax_elem; /* ilogb is floor(log2) exactly */
    /* the ceiling rule's exponent is k or k + 1: amax / 2^k lies in
     * [2^emax_elem, 2^(emax_elem + 1)) and maxfinite is in the same binade */
    if (rule == MXO_RULE_CEIL && ldexp(f->maxfinite, k) < amax) k += 1;
    k += 127;
    if (k < 0) k = 0;
    if (k > 254) k = 254;
    return (unsigned)k;
}

unsigned mxo_scale_code(int fmt, const double* x, int64_t n) { return mxo_scale_code_rule(fmt, x, n, MXO_RULE_FLOOR); }

/* Quantize one block: scale code, then q_i = Q_FP8(x_i / s) [SM120 §0.1].
 * A block holding NaN or Inf gets element codes 0x7F (FP8) or 0 (E2M1).
 * Codes are stored from codes[0] on: one byte each, or for E2M1 two per byte
 * with element 2i in the low nibble [NVFP4 §5.5: 4 bits per element]. */
static void quantize_block_rule(int fmt, int rule, const double* x, int64_t n, uint8_t* codes, uint8_t* scale) {
    unsigned s = mxo_scale_code_rule(fmt, x, n, rule);
    *scale = (uint8_t)s;
    for (int64_t i = 0; i < n; ++i) {
        unsigned c = (s == 0xFFu) ? (fmt == MXO_E2M1 ? 0u : 0x7Fu) : mxo_encode(fmt, ldexp(x[i], -((int)s - 127)));
        if (fmt == MXO_E2M1) {
            if (i % 2 == 0)
                codes[i / 2] = (uint8_t)c;
            else
                codes[i / 2] |= (uint8_t)(c << 4);
        } else {
            codes[i] = (uint8_t)c;
        }
    }
}

static void quantize_block(int fmt, const double* x, int64_t n, uint8_t* codes, uint8_t* scale) {
    quantize_block_rule(fmt, MXO_RULE_FLOOR, x, n, codes, scale);
}

/* Bytes of codes per block, and the code of element k of a row. */
static int64_t block_bytes(int fmt) { return fmt == MXO_E2M1 ? MXO_BLOCK / 2 : MXO_BLOCK; }
static unsigned code_at(int fmt, const uint8_t* row, int64_t k) {
    return fmt == MXO_E2M1 ? (row[k / 2] >> (4 * (k & 1))) & 0xFu : row[k];
}

/* ---------------------------------------------------------------------------
 * Input element access: f32, or bf16 given as its 16-bit pattern.
 * ------------------------------------------------------------------------- */
static double load_elem(const void* x, int dt, int64_t idx) {
    if (dt == MXO_F32) return (double)((const float*)x)[idx];
    uint32_t u = (uint32_t)((const uint16_t*)x)[idx] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Rowwise: blocks of 32 consecutive elements along each row (the contiguous
 * axis) [GLOSS]; codes and scales in separate arrays [SM120 §0.1]. */
int mxo_quantize_rows(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                      int64_t ldq, uint8_t* s, int64_t lds) {
    return mxo_quantize_rows_rule(x, xdt, rows, cols, ldx, fmt, MXO_RULE_FLOOR, q, ldq, s, lds);
}

int mxo_quantize_rows_rule(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, int rule,
                           uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds) {
    if (cols % MXO_BLOCK != 0 || rows < 0 || cols < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double v[MXO_BLOCK];
        for (int64_t b = 0; b < cols / MXO_BLOCK; ++b) {
            for (int i = 0; i < MXO_BLOCK; ++i) v[i] = load_elem(x, xdt, r * ldx + b * MXO_BLOCK + i);
            quantize_block_rule(fmt, rule, v, MXO_BLOCK, q + r * ldq + b * block_bytes(fmt), s + r * lds + b);
        }
    }
    return 0;
}

/* Colwise: blocks of 32 consecutive elements down each column. Blocks are
 * directional, so this is a second quantization from the high-precision input,
 * not a transpose of the rowwise codes [SM120 §1.2; GLOSS]. The result is
 * stored transposed: qt[c][r] (row pitch ldq), st[c][r/32] (row pitch lds). */
int mxo_quantize_cols(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* qt,
                      int64_t ldq, uint8_t* st, int64_t lds) {
    return mxo_quantize_cols_rule(x, xdt, rows, cols, ldx, fmt, MXO_RULE_FLOOR, qt, ldq, st, lds);
}

int mxo_quantize_cols_rule(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, int rule,
                           uint8_t* qt, int64_t ldq, uint8_t* st, int64_t lds) {
    if (rows % MXO_BLOCK != 0 || rows < 0 || cols < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        double v[MXO_BLOCK];
        for (int64_t b = 0; b < rows / MXO_BLOCK; ++b) {
            for (int i = 0; i < MXO_BLOCK; ++i) v[i] = load_elem(x, xdt, (b * MXO_BLOCK + i) * ldx + c);
            quantize_block_rule(fmt, rule, v, MXO_BLOCK, qt + c * ldq + b * block_bytes(fmt), st + c * lds + b);
        }
    }
    return 0;
}

/* Two-dimensional blocks [SM120 §1.3: weights may share one scale per 32 x 32
 * block, expanded afterwards to the MXFP8 scale layout, with the FP8 element
 * and E8M0 encodings unchanged]. Each 32 x 32 block of x gets one scale from
 * its 1024 values (same rule as a 32-element block); every element is encoded
 * with it. Outputs, either pair may be NULL:
 *   q [rows x cols], s [rows x cols/32]: s[r][c/32] = the scale of block
 *     (r/32, c/32), repeated on the block's 32 rows (the expanded layout);
 *   qt [cols x rows], st [cols x rows/32]: the same codes and scales for x^T.
 * Because a 32 x 32 block holds the same elements after a transpose, qt is
 * exactly the transpose of q. rows % 32 == 0, cols % 32 == 0; E4M3 or E5M2. */
int mxo_quantize_2d(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, int rule, uint8_t* q,
                    int64_t ldq, uint8_t* s, int64_t lds, uint8_t* qt, int64_t ldqt, uint8_t* st, int64_t ldst) {
    if (rows % MXO_BLOCK != 0 || cols % MXO_BLOCK != 0 || rows < 0 || cols < 0 || fmt == MXO_E2M1) return -2;
    const int64_t br = rows / MXO_BLOCK, bc = cols / MXO_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < br * bc; ++blk) {
        const int64_t r0 = (blk / bc) * MXO_BLOCK, c0 = (blk % bc) * MXO_BLOCK;
        double v[MXO_BLOCK * MXO_BLOCK];
        for (int i = 0; i < MXO_BLOCK; ++i)
            for (int j = 0; j < MXO_BLOCK; ++j) v[i * MXO_BLOCK + j] = load_elem(x, xdt, (r0 + i) * ldx + c0 + j);
        const unsigned sc = mxo_scale_code_rule(fmt, v, MXO_BLOCK * MXO_BLOCK, rule);
        for (int i = 0; i < MXO_BLOCK; ++i) {
            for (int j = 0; j < MXO_BLOCK; ++j) {
                const unsigned c = sc == 0xFFu ? 0x7Fu : mxo_encode(fmt, ldexp(v[i * MXO_BLOCK + j], -((int)sc - 127)));
                if (q) q[(r0 + i) * ldq + c0 + j] = (uint8_t)c;
                if (qt) qt[(c0 + j) * ldqt + r0 + i] = (uint8_t)c;
            }
            if (s) s[(r0 + i) * lds + c0 / MXO_BLOCK] = (uint8_t)sc;
            if (st) st[(c0 + i) * ldst + r0 / MXO_BLOCK] = (uint8_t)sc;
        }
    }
    return 0;
}

/* Float8BlockScaling -> MXFP8 scales [SM120 §1.3]: a power-of-two scale of a
 * 128-element block (layout 0: s_in[r][c/128]) or of a 128 x 128 block
 * (layout 1: s_in[r/128][c/128]) becomes the E8M0 code of every 32-element
 * block it covers; the FP8 codes are reused unchanged. s is the dequantizing
 * factor (x_hat = q * s). A scale that is not a positive power of two 2^k with
 * -127 <= k <= 127 cannot be held by E8M0 and gives 0xFF (NaN), so its blocks
 * decode to NaN instead of to wrong values. cols % 128 == 0. */
static unsigned e8m0_of_pow2(float v) {
    const double d = (double)v;
    if (!(d > 0.0) || isinf(d)) return 0xFFu;
    int e;
    const double m = frexp(d, &e); /* d = m * 2^e, m in [0.5, 1) */
    if (m != 0.5) return 0xFFu;
    const int k = e - 1;
    if (k < -127 || k > 127) return 0xFFu;
    return (unsigned)(k + 127);
}

int mxo_scale_broadcast(const float* s_in, int64_t ld_in, int layout, int64_t rows, int64_t cols, uint8_t* out,
                        int64_t ld_out) {
    if (cols % 128 != 0 || rows < 0 || cols < 0 || (layout != 0 && layout != 1)) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < cols / MXO_BLOCK; ++b) {
            const int64_t src_row = layout == 0 ? r : r / 128;
            out[r * ld_out + b] = (uint8_t)e8m0_of_pow2(s_in[src_row * ld_in + (b * MXO_BLOCK) / 128]);
        }
    return 0;
}

/* Fused KV-cache write [SM120 §0.2]: for each token t and head h, the D values
 * are quantized to E4M3 in blocks of 32 along the head dimension and written
 * to the cache slot slot_mapping[t]; page = slot / page_size, offset = slot %
 * page_size. Cache layout [page][offset][h][d], scales [page][offset][h][d/32].
 * A negative slot marks a padding token and is skipped. */
int mxo_kv_quant_write(const void* k, const void* v, int dt, int64_t T, int64_t H, int64_t D, int64_t ld_token,
                       const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* k_scale, uint8_t* v_cache,
                       uint8_t* v_scale, int64_t page_size, int64_t num_pages) {
    if (D % MXO_BLOCK != 0 || T < 0 || H < 0 || D < 0 || page_size <= 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= page_size * num_pages) continue;
        int64_t page = slot / page_size, off = slot % page_size;
        int64_t cache_row = (page * page_size + off) * H; /* first (slot, h=0) row */
        double buf[MXO_BLOCK];
        for (int which = 0; which < 2; ++which) {
            const void* src = which == 0 ? k : v;
            uint8_t* cache = which == 0 ? k_cache : v_cache;
            uint8_t* scale = which == 0 ? k_scale : v_scale;
            for (int64_t h = 0; h < H; ++h)
                for (int64_t b = 0; b < D / MXO_BLOCK; ++b) {
                    for (int i = 0; i < MXO_BLOCK; ++i) buf[i] = load_elem(src, dt, t * ld_token + h * D + b * MXO_BLOCK + i);
                    quantize_block(MXO_E4M3, buf, MXO_BLOCK, cache + (cache_row + h) * D + b * MXO_BLOCK,
                                   scale + (cache_row + h) * (D / MXO_BLOCK) + b);
                }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Dequantize: x_hat = s_b * q_i [SM120 §0.1], in double (exact), then rounded
 * to the output type. f32 output uses C's double-to-float conversion (round to
 * nearest even, overflow to infinity). bf16 output is rounded here directly
 * from the double, to 8 significant bits with subnormals below 2^-126.
 * ------------------------------------------------------------------------- */
uint16_t mxo_double_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0u;
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80u;
    double r = round_to_grid(a, 7, -126);
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80u; /* past the largest finite bf16 */
    return sign | (uint16_t)grid_bits(r, 7, -126, 127);
}

double mxo_dequant_value(int fmt, unsigned code, unsigned scale) {
    if ((scale & 0xFF) == 0xFF) return NAN; /* a NaN scale makes the whole block NaN */
    return mxo_decode(fmt, code) * mxo_decode_e8m0(scale);
}

int mxo_dequantize(const uint8_t* q, int64_t ldq, const uint8_t* s, int64_t lds, int fmt, int64_t rows, int64_t cols,
                   void* y, int ydt, int64_t ldy) {
    if (cols % MXO_BLOCK != 0 || rows < 0 || cols < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double v = mxo_dequant_value(fmt, code_at(fmt, q + r * ldq, c), s[r * lds + c / MXO_BLOCK]);
            if (ydt == MXO_F32)
                ((float*)y)[r * ldy + c] = (float)v;
            else
                ((uint16_t*)y)[r * ldy + c] = mxo_double_to_bf16(v);
        }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Block-scaled matrix product [SM120 §0.3; NVFP4 §7.1, §7.4]:
 *   y[m][n] = sum_b sA[m][b] * sB[n][b] * sum_{i<32} qA[m][32b+i] * qB[n][32b+i]
 * with A codes [M x K] and B codes [N x K], both K-contiguous (y = A * B^T).
 * Each block's inner sum is formed in double, multiplied by the two block
 * scales, and added to the running double total in block order, exactly the
 * shape of the equation. t[m][n] = sum_k |a_hat_k * b_hat_k| is returned
 * beside it: the magnitude against which a tolerance is stated.
 * ------------------------------------------------------------------------- */
static void gemm_one(int64_t K, const uint8_t* a, const uint8_t* sa, int afmt, const double* lut_a, const uint8_t* b,
                     const uint8_t* sb, int bfmt, const double* lut_b, double* y_out, double* t_out) {
    double y = 0.0, t = 0.0;
    for (int64_t blk = 0; blk < K / MXO_BLOCK; ++blk) {
        double inner = 0.0, inner_abs = 0.0;
        for (int i = 0; i < MXO_BLOCK; ++i) {
            const int64_t k = blk * MXO_BLOCK + i;
            double p = lut_a[code_at(afmt, a, k)] * lut_b[code_at(bfmt, b, k)];
            inner += p;
            inner_abs += fabs(p);
        }
        double ss = mxo_decode_e8m0(sa[blk]) * mxo_decode_e8m0(sb[blk]);
        y += ss * inner;
        t += ss * inner_abs;
    }
    *y_out = y;
    *t_out = t;
}

static void build_lut(int fmt, double* lut) {
    for (unsigned c = 0; c < 256; ++c) lut[c] = mxo_decode(fmt, c);
}

int mxo_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t ldsa,
             int afmt, const uint8_t* b, int64_t ldb, const uint8_t* sb, int64_t ldsb, int bfmt, double* y,
             int64_t ldy, double* t, int64_t ldt) {
    if (K % MXO_BLOCK != 0 || M < 0 || N < 0 || K < 0) return -2;
    double lut_a[256], lut_b[256];
    build_lut(afmt, lut_a);
    build_lut(bfmt, lut_b);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            gemm_one(K, a + m * lda, sa + m * ldsa, afmt, lut_a, b + n * ldb, sb + n * ldsb, bfmt, lut_b,
                     &y[m * ldy + n], &t[m * ldt + n]);
    return 0;
}

/* The same product at a list of (m, n) output coordinates only. */
int mxo_gemm_at(int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t ldsa, int afmt, const uint8_t* b,
                int64_t ldb, const uint8_t* sb, int64_t ldsb, int bfmt, const int64_t* mi, const int64_t* ni,
                int64_t count, double* y, double* t) {
    if (K % MXO_BLOCK != 0 || count < 0) return -2;
    double lut_a[256], lut_b[256];
    build_lut(afmt, lut_a);
    build_lut(bfmt, lut_b);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        gemm_one(K, a + mi[i] * lda, sa + mi[i] * ldsa, afmt, lut_a, b + ni[i] * ldb, sb + ni[i] * ldsb, bfmt, lut_b,
                 &y[i], &t[i]);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Paged attention over the MXFP8 KV cache [SM120 §0.2]. The KV cache holds K
 * and V as E4M3 codes with one E8M0 scale per 32 values along the head
 * dimension; the query arrives with its own scales. The consumer the page
 * describes forms the scores Q K^T as a block-scaled FP8 product, restores V
 * to BF16 and then forms P V. Written out for one query row (token t =
 * seq * q_len + i, query head h), with L = kv_lens[seq]:
 *   key j is allowed when j < L and, with `causal`, j <= L - q_len + i (the
 *   query sits at absolute position L - q_len + i of its sequence);
 *   S_j   = the block-scaled product of the query row and key row j over the
 *           head dimension (the same sum as mxo_gemm);
 *   z_j   = sm_scale * S_j;  P_j = exp(z_j - max z) / sum_k exp(z_k - max z);
 *   Vb_jd = V code * scale, rounded to bf16 (the "restored to BF16" step);
 *   O_d   = sum_j P_j * Vb_jd.
 * Readings where the page is silent: the softmax runs over the allowed keys
 * only; a row with no allowed key gives O = 0 and lse = -inf; the causal
 * offset aligns the last query with the last key. Key j of the sequence is
 * read from page page_table[seq * pages_per_seq + j / page_size], row
 * j % page_size, kv head h / (hq / hkv); L is clamped to pages_per_seq *
 * page_size. Also returned, for stating
 * tolerances: W_d = sum_j P_j |Vb_jd|, lse = log sum_j exp(z_j), and
 * tmax = max_j sum_d |q_hat_d k_hat_jd|. A NaN score makes the whole row NaN.
 * ------------------------------------------------------------------------- */
static double bf16_value(uint16_t bits) {
    if ((bits & 0x7F80u) == 0x7F80u) {
        if (bits & 0x7Fu) return NAN;
        return (bits & 0x8000u) ? -INFINITY : INFINITY;
    }
    int e = (bits >> 7) & 0xFF;
    double mant = (double)(bits & 0x7F);
    double v = e == 0 ? ldexp(mant, -133) : ldexp(128.0 + mant, e - 134);
    return (bits & 0x8000u) ? -v : v;
}

static void attention_one(const uint8_t* q, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                          const uint8_t* vc, const uint8_t* vs, const int32_t* ptab, int64_t n_allowed,
                          int64_t hkv, int64_t hk, int64_t D, int64_t page_size, double sm_scale,
                          const double* lut, double* z, double* o, double* w, double* lse, double* tmax) {
    for (int64_t d = 0; d < D; ++d) o[d] = w[d] = 0.0;
    if (n_allowed <= 0) {
        *lse = -INFINITY;
        *tmax = 0.0;
        return;
    }
    const int64_t nb = D / MXO_BLOCK;
    double m = -INFINITY, tm = 0.0;
    int has_nan = 0;
    for (int64_t j = 0; j < n_allowed; ++j) {
        int64_t slot = (int64_t)ptab[j / page_size] * page_size + j % page_size;
        int64_t row = slot * hkv + hk;
        double sj, tj;
        gemm_one(D, q, qs, MXO_E4M3, lut, kc + row * D, ks + row * nb, MXO_E4M3, lut, &sj, &tj);
        z[j] = sm_scale * sj;
        if (isnan(z[j])) has_nan = 1;
        if (z[j] > m) m = z[j];
        if (tj > tm) tm = tj;
    }
    *tmax = tm;
    if (has_nan) {
        for (int64_t d = 0; d < D; ++d) o[d] = w[d] = NAN;
        *lse = NAN;
        return;
    }
    double denom = 0.0;
    for (int64_t j = 0; j < n_allowed; ++j) {
        z[j] = exp(z[j] - m); /* now the unnormalised weight */
        denom += z[j];
    }
    *lse = m + log(denom);
    for (int64_t j = 0; j < n_allowed; ++j) {
        double pj = z[j] / denom;
        int64_t slot = (int64_t)ptab[j / page_size] * page_size + j % page_size;
        int64_t row = slot * hkv + hk;
        for (int64_t d = 0; d < D; ++d) {
            double vb = bf16_value(mxo_double_to_bf16(mxo_dequant_value(MXO_E4M3, vc[row * D + d], vs[row * nb + d / MXO_BLOCK])));
            o[d] += pj * vb;
            w[d] += pj * fabs(vb);
        }
    }
}

int mxo_paged_attention(const uint8_t* q, const uint8_t* qs, int64_t ld_q, int64_t ld_qs, const uint8_t* kc,
                        const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, const int32_t* page_table,
                        int64_t pages_per_seq, const int32_t* kv_lens, int64_t num_seqs, int64_t q_len, int64_t hq,
                        int64_t hkv, int64_t D, int64_t page_size, double sm_scale, int causal, const int64_t* rows,
                        int64_t count, double* o, double* w, double* lse, double* tmax) {
    if (D % MXO_BLOCK != 0 || D <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || page_size <= 0 || q_len < 0 ||
        num_seqs < 0)
        return -2;
    const int64_t total = num_seqs * q_len * hq;
    const int64_t n = rows ? count : total;
    const int64_t max_keys = pages_per_seq * page_size;
    double lut[256];
    build_lut(MXO_E4M3, lut);
    int bad = 0;
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(max_keys > 0 ? max_keys : 1));
        if (!z) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < n; ++r) {
                const int64_t idx = rows ? rows[r] : r;
                const int64_t t = idx / hq, h = idx % hq;
                const int64_t seq = t / q_len, i = t % q_len;
                const int64_t L = kv_lens[seq];
                int64_t allowed = L < max_keys ? L : max_keys;
                if (causal && L - q_len + i + 1 < allowed) allowed = L - q_len + i + 1;
                attention_one(q + t * ld_q + h * D, qs + t * ld_qs + h * (D / MXO_BLOCK), kc, ks, vc, vs,
                              page_table + seq * pages_per_seq, allowed, hkv, h / (hq / hkv), D, page_size,
                              sm_scale, lut, z, o + r * D, w + r * D, lse + r, tmax + r);
            }
            free(z);
        }
    }
    return bad ? -1 : 0;
}

int mxo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void mxo_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
