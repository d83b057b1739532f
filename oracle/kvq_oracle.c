/*
 * kvq_oracle.c -- plain CPU oracle for the KV compress -> quantise -> paged-store path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header, table or constant with the HIP library: every layout
 * constant, encoder and decoder below is written out again from the definitions.
 *
 * Sources (web pages this follows):
 *  [P1] "sglang, DeepSeek V4.1 Paged KV Cache: V41 and FP4 formats" (sglang PR #39123
 *       analysis), section 1 "kv_layout.cuh and related files" (layouts, PagedKV
 *       addressing, store_row), section 2 "c1.cuh and c2.cuh" (compressor writes, FP4
 *       quantised once), section 4 "dequant_k_cache.py" (pages -> bf16 workspace),
 *       "memory usage reduction" (528 / 288 vs 584 B/token).
 *  [P2] "SGLang: DeepSeek-v4 SWA index translation hoisting" (sglang PR #34890
 *       analysis), section 1 (the preallocated int32 buffer and its fill function).
 *  [P3] "DeepSeek V4 Sparse FP8 Compressor kernel optimisation with CuteDSL" (vLLM PR
 *       #44161 analysis), section 2 (per-channel online softmax over the window) and
 *       section 3 (RoPE with bf16 casts, per-32 absmax for the fp8 scale).
 *
 * Precision: pooling is evaluated in float64 and rounded once to bf16.  RoPE is done in
 * float32 with every product and sum rounded (no fused multiply-add; build with
 * -ffp-contract=off), then rounded to bf16.  Encoders are exact definitions.
 *
 * Parity status of each function is listed in the module docstring of oracle/__init__.py
 * together with the test that pins it.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

/* Threads the OpenMP loops below use (reported with CPU timings). */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* Sets that thread count for later calls (n >= 1); used to time a single-thread run. */
void orc_set_num_threads(int n) { omp_set_num_threads(n < 1 ? 1 : n); }

/* ---------------------------------------------------------------- layout facts */
/* [P1] section 1: V41 keeps 512 fp8 e4m3 codes and one ue8m0 scale per 32 values
 * (16 scales) = 528 B/token; V41_FP4 keeps 512 e2m1 codes (two per byte, 256 B) and one
 * e4m3 scale per 32 values (16 B) and is quoted at 288 B/token, so 16 B are padding.
 * Reading used here: the 16 pad bytes follow the 16 scale bytes in each token's scale
 * row, and a page is 64 code rows followed by 64 scale rows (page / row / scale-row
 * addressing of PagedKV). */
#define ORC_LAYOUT_V41 1
#define ORC_LAYOUT_V41_FP4 2

static const int kHead = 512;   /* channels per token row                          */
static const int kRopeDim = 64;  /* rope channels: the last 64                      */
static const int kBlock = 32;    /* values per scale                                */
static const int kPageRows = 64; /* tokens per page                                 */

int64_t orc_code_row_bytes(int32_t layout) {
    if (layout == ORC_LAYOUT_V41) return kHead;          /* one byte per fp8 code   */
    if (layout == ORC_LAYOUT_V41_FP4) return kHead / 2;  /* two e2m1 codes per byte */
    return -2;
}

int64_t orc_scale_row_bytes(int32_t layout) {
    if (layout == ORC_LAYOUT_V41) return kHead / kBlock;              /* 16 ue8m0 bytes */
    if (layout == ORC_LAYOUT_V41_FP4) return kHead / kBlock + 16;     /* 16 e4m3 + pad  */
    return -2;
}

int64_t orc_bytes_per_token(int32_t layout) {
    int64_t c = orc_code_row_bytes(layout);
    if (c < 0) return c;
    return c + orc_scale_row_bytes(layout);
}

int64_t orc_page_bytes(int32_t layout) {
    int64_t b = orc_bytes_per_token(layout);
    if (b < 0) return b;
    return (int64_t)kPageRows * b;
}

/* ---------------------------------------------------------------- bf16 */
static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float orc_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Nearest bfloat16 to x (8 significant bits, exponent range of float32, subnormal
 * quantum 2^-133), ties to the even significand, overflow to infinity. */
uint16_t orc_bf16_from_double(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    frexp(a, &e);                 /* a = f * 2^e with f in [0.5, 1)                 */
    int qexp = e - 8;             /* quantum of an 8-bit significand in this binade */
    if (qexp < -133) qexp = -133; /* subnormal bf16 spacing                          */
    double m = ldexp(a, -qexp);   /* exact power-of-two scaling                      */
    double r = nearbyint(m);      /* round half to even (default rounding mode)      */
    double v = ldexp(r, qexp);
    const double kMax = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (v > kMax) return sign | 0x7F80;
    float f = (float)v;           /* exact: v has at most 8 significant bits          */
    return sign | (uint16_t)(bits_from_f32(f) >> 16);
}

/* ---------------------------------------------------------------- fp8 e4m3 (OCP e4m3fn) */
/* Format: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinities; S.1111.111
 * is NaN; largest finite 448; subnormals m * 2^-9. */
double orc_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Round-to-nearest-even encoding of q; |q| must not exceed 448 after rounding (callers
 * guarantee it).  Sign kept, so -0 and values that round to zero from below give 0x80. */
uint8_t orc_e4m3_encode(double q) {
    uint8_t s = signbit(q) ? 0x80 : 0;
    double a = fabs(q);
    if (a == 0.0) return s;
    int e;
    frexp(a, &e);
    int E = e - 1;                /* a in [2^E, 2^(E+1))                        */
    if (E < -6) E = -6;           /* below the normal range the spacing is 2^-9 */
    double quantum = ldexp(1.0, E - 3);
    double n = nearbyint(a / quantum); /* exact division by a power of two; RNE */
    double v = n * quantum;
    if (v == 0.0) return s;
    frexp(v, &e);
    E = e - 1;
    if (E < -6) return s | (uint8_t)(v / ldexp(1.0, -9));        /* subnormal code  */
    int mant = (int)((v / ldexp(1.0, E) - 1.0) * 8.0);           /* 0..7, exact     */
    return s | (uint8_t)(((E + 7) << 3) | mant);
}

/* ---------------------------------------------------------------- ue8m0 */
/* The power-of-two scale 2^k of a 32-value block: the smallest integer k (not below
 * -127, the smallest ue8m0 value) with amax <= 448 * 2^k, so every scaled value fits the
 * e4m3 range.  The byte stored is k + 127.  [P1] section 1 says the exponent is taken
 * from the amax bits without a division; this is the same quantity, found by search. */
int orc_ue8m0_exponent(float amax) {
    int k = -127;
    while (k < 127 && (double)amax > ldexp(448.0, k)) k++;
    return k;
}

uint8_t orc_ue8m0_byte(float amax) { return (uint8_t)(orc_ue8m0_exponent(amax) + 127); }

/* ---------------------------------------------------------------- fp4 e2m1 */
static const double kE2m1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_decode(uint8_t nib) {
    double v = kE2m1Mag[nib & 7];
    return (nib & 8) ? -v : v;
}

/* Nearest e2m1 magnitude to |q| (ties to the even code), magnitudes above 6 clamp to 6,
 * sign bit kept. */
uint8_t orc_e2m1_encode(float q) {
    uint8_t s = signbit(q) ? 8 : 0;
    double a = fabs((double)q);
    if (a > 6.0) return s | 7;
    int best = 0;
    double bestd = a;
    for (int i = 1; i < 8; i++) {
        double d = fabs(a - kE2m1Mag[i]);
        if (d < bestd || (d == bestd && (i % 2) == 0)) {
            best = i;
            bestd = d;
        }
    }
    return s | (uint8_t)best;
}

/* e4m3 scale of an FP4 block: the e4m3 value nearest to fl32(amax / 6) (RNE), held at
 * 448 when that quotient exceeds the e4m3 range. */
uint8_t orc_fp4_scale_code(float amax) {
    float t = amax / 6.0f; /* IEEE single-precision division */
    if ((double)t > 448.0) return 0x7E;
    return orc_e4m3_encode((double)t);
}

/* ---------------------------------------------------------------- one token row */
/* Quantise one row of 512 bf16-valued floats into its code row and scale row.
 * [P1] section 1 (block scaling per 32 values) and section 2 (FP4 quantised once,
 * straight from the bf16 values, with no fp8 step in between). */
static void quant_row(int32_t layout, const float* v, uint8_t* code, uint8_t* scale) {
    for (int b = 0; b < kHead / kBlock; b++) {
        const float* x = v + b * kBlock;
        float amax = 0.0f;
        for (int j = 0; j < kBlock; j++) {
            float a = fabsf(x[j]);
            if (a > amax) amax = a;
        }
        if (layout == ORC_LAYOUT_V41) {
            int k = orc_ue8m0_exponent(amax);
            scale[b] = (uint8_t)(k + 127);
            for (int j = 0; j < kBlock; j++)
                code[b * kBlock + j] = orc_e4m3_encode(ldexp((double)x[j], -k));
        } else {
            uint8_t sc = orc_fp4_scale_code(amax);
            scale[b] = sc;
            float s = (float)orc_e4m3_decode(sc);
            for (int j = 0; j < kBlock; j += 2) {
                uint8_t lo = 0, hi = 0;
                if (s != 0.0f) {
                    lo = orc_e2m1_encode(x[j] / s);
                    hi = orc_e2m1_encode(x[j + 1] / s);
                }
                code[(b * kBlock + j) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    if (layout == ORC_LAYOUT_V41_FP4)
        memset(scale + kHead / kBlock, 0, 16); /* documented padding */
}

int orc_quant_row(int32_t layout, const uint16_t* v_bf16, uint8_t* code, uint8_t* scale) {
    if (orc_bytes_per_token(layout) < 0) return -2;
    float v[512];
    for (int c = 0; c < kHead; c++) v[c] = orc_bf16_to_f32(v_bf16[c]);
    quant_row(layout, v, code, scale);
    return 0;
}

/* ---------------------------------------------------------------- RoPE */
/* NeoX half rotation of the 64 rope channels at the end of the row: channel 448+i is
 * paired with 480+i (i < 32) and rotated by the angle whose cosine and sine are
 * cos_sin[pos][i] and cos_sin[pos][32+i].  Single-precision, each product and sum
 * rounded, results rounded to bf16 ([P3] section 3: RoPE then bf16 casts). */
static void rope_row(float* v, const float* cs) {
    const int base = kHead - kRopeDim, half = kRopeDim / 2;
    for (int i = 0; i < half; i++) {
        float x1 = v[base + i], x2 = v[base + half + i];
        float c = cs[i], s = cs[half + i];
        float a = x1 * c, b = x2 * s, d = x2 * c, e = x1 * s;
        float o1 = a - b, o2 = d + e;
        v[base + i] = orc_bf16_to_f32(orc_bf16_from_double((double)o1));
        v[base + half + i] = orc_bf16_to_f32(orc_bf16_from_double((double)o2));
    }
}

int orc_rope_row(uint16_t* v_bf16, const float* cos_sin_row) {
    float v[512];
    for (int c = 0; c < kHead; c++) v[c] = orc_bf16_to_f32(v_bf16[c]);
    rope_row(v, cos_sin_row);
    for (int c = 0; c < kHead; c++) v_bf16[c] = orc_bf16_from_double((double)v[c]);
    return 0;
}

/* ---------------------------------------------------------------- addressing */
/* PagedKV addressing ([P1] section 1): slot -> (page, row); a page holds 64 code rows
 * followed by 64 scale rows.  Returns 0 when the slot is outside the pool (row skipped). */
static int row_address(int32_t layout, uint8_t* pool, int64_t num_pages, int64_t slot,
                       uint8_t** code, uint8_t** scale) {
    if (slot < 0 || slot >= num_pages * kPageRows) return 0;
    int64_t page = slot / kPageRows, row = slot % kPageRows;
    int64_t cr = orc_code_row_bytes(layout), sr = orc_scale_row_bytes(layout);
    uint8_t* pg = pool + page * orc_page_bytes(layout);
    *code = pg + row * cr;
    *scale = pg + kPageRows * cr + row * sr;
    return 1;
}

/* ---------------------------------------------------------------- store paths */
/* Plain store: quantise bf16 rows k[i][0:512] (row stride ld) into pool slots. */
int orc_kv_store(int32_t layout, uint8_t* pool, int64_t num_pages, const uint16_t* k,
                 int64_t ld, const int32_t* slots, int64_t n) {
    if (orc_bytes_per_token(layout) < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        uint8_t *code, *scale;
        if (!row_address(layout, pool, num_pages, slots[i], &code, &scale)) continue;
        float v[512];
        for (int c = 0; c < kHead; c++) v[c] = orc_bf16_to_f32(k[i * ld + c]);
        quant_row(layout, v, code, scale);
    }
    return 0;
}

/* Store with RoPE: rows whose position is outside [0, max_pos) are skipped. */
int orc_kv_store_rope(int32_t layout, uint8_t* pool, int64_t num_pages, const uint16_t* k,
                      int64_t ld, const int32_t* pos, const float* cos_sin, int64_t max_pos,
                      const int32_t* slots, int64_t n) {
    if (orc_bytes_per_token(layout) < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        uint8_t *code, *scale;
        if (!row_address(layout, pool, num_pages, slots[i], &code, &scale)) continue;
        if (pos[i] < 0 || pos[i] >= max_pos) continue;
        float v[512];
        for (int c = 0; c < kHead; c++) v[c] = orc_bf16_to_f32(k[i * ld + c]);
        rope_row(v, cos_sin + (int64_t)pos[i] * kRopeDim);
        quant_row(layout, v, code, scale);
    }
    return 0;
}

/* ---------------------------------------------------------------- K norm + RoPE */
/* The "fused K norm + RoPE" store of [P1]'s latency table; the page gives no formula.
 * Reading: RMS normalisation of the whole 512-channel bf16 row with a per-channel weight,
 * y_c = x_c * w_c / sqrt(mean_c(x_c^2) + eps), evaluated in float64 and rounded once to
 * bf16; then RoPE and the store as in orc_kv_store_rope. */
static void norm_row(float* v, const uint16_t* w_bf16, float eps) {
    double ss = 0.0;
    for (int c = 0; c < kHead; c++) ss += (double)v[c] * (double)v[c];
    double r = 1.0 / sqrt(ss / kHead + (double)eps);
    for (int c = 0; c < kHead; c++)
        v[c] = orc_bf16_to_f32(orc_bf16_from_double((double)v[c] * (double)orc_bf16_to_f32(w_bf16[c]) * r));
}

int orc_kv_store_norm_rope(int32_t layout, uint8_t* pool, int64_t num_pages, const uint16_t* k,
                           int64_t ld, const uint16_t* weight, float eps, const int32_t* pos,
                           const float* cos_sin, int64_t max_pos, const int32_t* slots, int64_t n) {
    if (orc_bytes_per_token(layout) < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        uint8_t *code, *scale;
        if (!row_address(layout, pool, num_pages, slots[i], &code, &scale)) continue;
        if (pos[i] < 0 || pos[i] >= max_pos) continue;
        float v[512];
        for (int c = 0; c < kHead; c++) v[c] = orc_bf16_to_f32(k[i * ld + c]);
        norm_row(v, weight, eps);
        rope_row(v, cos_sin + (int64_t)pos[i] * kRopeDim);
        quant_row(layout, v, code, scale);
    }
    return 0;
}

/* Normalised row only (for the pins): bf16 bits of y. */
int orc_norm_row(uint16_t* v_bf16, const uint16_t* weight, float eps) {
    float v[512];
    for (int c = 0; c < kHead; c++) v[c] = orc_bf16_to_f32(v_bf16[c]);
    norm_row(v, weight, eps);
    for (int c = 0; c < kHead; c++) v_bf16[c] = orc_bf16_from_double((double)v[c]);
    return 0;
}

/* ---------------------------------------------------------------- pooling */
/* Softmax pooling of window i ([P3] section 2): for every channel c, the weights are the
 * softmax over the r window rows of the scores in that channel, and the pooled value is
 * the weighted sum of the kv rows.  Windows are the contiguous, non-overlapping row
 * ranges [i*r, i*r + r).  The maximum is subtracted before exponentiation, as the online
 * form does; it cancels exactly in the ratio.  Evaluated in float64. */
static void pool_window(const float* kv, const float* score, int64_t ld, int ratio,
                        int64_t i, double* out) {
    for (int c = 0; c < kHead; c++) {
        double m = -INFINITY;
        for (int j = 0; j < ratio; j++) {
            double s = score[(i * ratio + j) * ld + c];
            if (s > m) m = s;
        }
        double num = 0.0, den = 0.0;
        for (int j = 0; j < ratio; j++) {
            double w = exp((double)score[(i * ratio + j) * ld + c] - m);
            den += w;
            num += w * (double)kv[(i * ratio + j) * ld + c];
        }
        out[c] = num / den;
    }
}

/* Pooled rows before RoPE: exact float64 values and their bf16 roundings. */
int orc_pool_rows(const float* kv, const float* score, int64_t ld, int32_t ratio, int64_t R,
                  double* out_f64, uint16_t* out_bf16) {
    if (ratio < 1) return -3;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; i++) {
        double p[512];
        pool_window(kv, score, ld, ratio, i, p);
        for (int c = 0; c < kHead; c++) {
            if (out_f64) out_f64[i * kHead + c] = p[c];
            if (out_bf16) out_bf16[i * kHead + c] = orc_bf16_from_double(p[c]);
        }
    }
    return 0;
}

/* Compressor: pool each window, round to bf16, RoPE at pos[i], quantise, store at
 * slots[i].  Rows with an out-of-pool slot or out-of-range position are skipped. */
int orc_kv_compress_store(int32_t layout, uint8_t* pool, int64_t num_pages, const float* kv,
                          const float* score, int64_t ld, int32_t ratio, const int32_t* pos,
                          const float* cos_sin, int64_t max_pos, const int32_t* slots,
                          int64_t R) {
    if (orc_bytes_per_token(layout) < 0) return -2;
    if (ratio < 1) return -3;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < R; i++) {
        uint8_t *code, *scale;
        if (!row_address(layout, pool, num_pages, slots[i], &code, &scale)) continue;
        if (pos[i] < 0 || pos[i] >= max_pos) continue;
        double p[512];
        float v[512];
        pool_window(kv, score, ld, ratio, i, p);
        for (int c = 0; c < kHead; c++) v[c] = orc_bf16_to_f32(orc_bf16_from_double(p[c]));
        rope_row(v, cos_sin + (int64_t)pos[i] * kRopeDim);
        quant_row(layout, v, code, scale);
    }
    return 0;
}

/* ---------------------------------------------------------------- dequant */
/* [P1] section 4: turn whole pages back into a bf16 workspace.  For each listed page, in
 * list order, and each of its 64 rows: value = decode(code) * decode(scale), formed in
 * float32 and rounded to bf16.  NaN codes or NaN scales give the quiet NaN 0x7FC0.
 * Page ids outside the pool leave their 64 output rows untouched. */
static uint16_t dequant_value(int32_t layout, uint8_t code, uint8_t scale) {
    double v, s;
    if (layout == ORC_LAYOUT_V41) {
        v = orc_e4m3_decode(code);
        if (scale == 0xFF || isnan(v)) return 0x7FC0;
        s = ldexp(1.0, (int)scale - 127);
    } else {
        v = orc_e2m1_decode(code);
        s = orc_e4m3_decode(scale);
        if (isnan(s)) return 0x7FC0;
    }
    float f = (float)(v * s); /* the exact product, rounded to float32 */
    return orc_bf16_from_double((double)f);
}

int orc_kv_dequant(int32_t layout, const uint8_t* pool, int64_t num_pages,
                   const int32_t* page_ids, int64_t P, uint16_t* out) {
    if (orc_bytes_per_token(layout) < 0) return -2;
    int64_t cr = orc_code_row_bytes(layout), sr = orc_scale_row_bytes(layout);
    int64_t pb = orc_page_bytes(layout);
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; p++) {
        int64_t page = page_ids[p];
        if (page < 0 || page >= num_pages) continue;
        const uint8_t* pg = pool + page * pb;
        for (int r = 0; r < kPageRows; r++) {
            const uint8_t* code = pg + r * cr;
            const uint8_t* scale = pg + kPageRows * cr + r * sr;
            uint16_t* o = out + (p * kPageRows + r) * kHead;
            for (int c = 0; c < kHead; c++) {
                uint8_t q;
                if (layout == ORC_LAYOUT_V41)
                    q = code[c];
                else
                    q = (c % 2 == 0) ? (code[c / 2] & 15) : (code[c / 2] >> 4);
                o[c] = dequant_value(layout, q, scale[c / kBlock]);
            }
        }
    }
    return 0;
}

/* Token-gather dequant: row i of the output is the dequantised row at slots[i] (the
 * per-token counterpart of [P1] section 4's page dequant); rows whose slot is outside the
 * pool are left untouched. */
int orc_kv_dequant_slots(int32_t layout, const uint8_t* pool, int64_t num_pages,
                         const int32_t* slots, int64_t n, uint16_t* out) {
    if (orc_bytes_per_token(layout) < 0) return -2;
    int64_t cr = orc_code_row_bytes(layout), sr = orc_scale_row_bytes(layout);
    int64_t pb = orc_page_bytes(layout);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        int64_t slot = slots[i];
        if (slot < 0 || slot >= num_pages * kPageRows) continue;
        const uint8_t* pg = pool + (slot / kPageRows) * pb;
        int64_t r = slot % kPageRows;
        const uint8_t* code = pg + r * cr;
        const uint8_t* scale = pg + kPageRows * cr + r * sr;
        for (int c = 0; c < kHead; c++) {
            uint8_t q;
            if (layout == ORC_LAYOUT_V41)
                q = code[c];
            else
                q = (c % 2 == 0) ? (code[c / 2] & 15) : (code[c / 2] >> 4);
            out[i * kHead + c] = dequant_value(layout, q, scale[c / kBlock]);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- full -> SWA slots */
/* [P2] section 1: the translation of full-pool slots into SWA-pool slots is done once per
 * step into a preallocated int32 buffer whose tail beyond n is zeroed; when n exceeds the
 * buffer the fill is refused (the caller then translates eagerly).  The map is an int32
 * table indexed by full slot; a full slot outside the table maps to -1 (skipped by the
 * stores). */
int orc_translate_slots(const int32_t* table, int64_t table_len, const int32_t* full,
                        int64_t n, int32_t* out, int64_t cap) {
    if (n > cap) return -4;
    for (int64_t i = 0; i < n; i++) {
        int64_t f = full[i];
        out[i] = (f >= 0 && f < table_len) ? table[f] : -1;
    }
    for (int64_t i = n; i < cap; i++) out[i] = 0;
    return 0;
}
