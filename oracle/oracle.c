/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the
 * quantized-decode hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library
 * under kv_quantization_amd/) may include, link or call this file; only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark do.
 * It shares no header, table or helper with the GPU code.
 *
 * Sources (web pages; each function names the section it follows):
 *   [KVQ]  boostr, src/ops/wgpu/shaders/cache/kv_cache_quant.wgsl
 *          sections "FP8 Per-Token Quantization/Dequantization",
 *          the declared per-tensor mode of its parameter block,
 *          "INT4 Per-Group Quantization/Dequantization",
 *          "INT8 Per-Token Quantization/Dequantization".
 *   [W8A8] metrale_model_layers, layers/ops/w8a8_decode.rs
 *          items W8a8Scale, W8a8Weight, W8a8Scratch, w8a8_act_quant,
 *          w8a8_act_quant_silu, w8a8_gemv.  The device kernels' source is not
 *          on that page, so the activation-quant formula here is a reading:
 *          absmax / 448 (the largest E4M3FN value) per row or per 128-group,
 *          the page's only scale floor 1e-8, and OCP E4M3FN encoding with
 *          round-to-nearest-even and saturation.
 *   [AWQ]  boostr, src/quant/wgpu/shaders/fused_int4_qkv.rs
 *          QKV_AWQ_SHIFTS, unpack_awq_qkv, fused_int4_qkv_{q,k,v}.
 *
 * Floating point: every quantizer step is the page's fp32 operation, done
 * one at a time in C float (built with -ffp-contract=off, no fast-math), with
 * rintf() for round-half-to-even.  OpenMP only splits independent tokens,
 * groups or rows across threads; it never changes an operation.
 *
 * Parity status: every exported function is pinned by the -m "not gpu" tests
 * (worked examples, closed forms, brute force, library cross-checks).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef int64_t i64;

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops that follow (timing only; no effect on
 * any result). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* [KVQ] INT8 per-token quantization.
 * For token t over its head_dim values: the absolute maximum, starting from
 * zero; scale = max(absmax / 127, 1e-8); each code is the value divided by the
 * scale, rounded half-to-even, clamped to [-128, 127]; one scale per token.  */
void oracle_kv_int8_quant(const float *x, int8_t *codes, float *scales,
                          i64 num_tokens, i64 head_dim) {
#pragma omp parallel for schedule(static)
    for (i64 t = 0; t < num_tokens; ++t) {
        const float *row = x + t * head_dim;
        float max_val = 0.0f;
        for (i64 d = 0; d < head_dim; ++d) max_val = fmaxf(max_val, fabsf(row[d]));
        float scale = fmaxf(max_val / 127.0f, 1e-8f);
        scales[t] = scale;
        for (i64 d = 0; d < head_dim; ++d) {
            float q = rintf(row[d] / scale);
            int c = (int)q;
            if (c < -128) c = -128;
            if (c > 127) c = 127;
            codes[t * head_dim + d] = (int8_t)c;
        }
    }
}

/* [KVQ] INT8 per-token dequantization: value = float(code) * scale[token]. */
void oracle_kv_int8_dequant(const int8_t *codes, const float *scales, float *y,
                            i64 num_tokens, i64 head_dim) {
#pragma omp parallel for schedule(static)
    for (i64 t = 0; t < num_tokens; ++t) {
        float scale = scales[t];
        for (i64 d = 0; d < head_dim; ++d)
            y[t * head_dim + d] = (float)codes[t * head_dim + d] * scale;
    }
}

/* [KVQ] INT8 per-tensor mode.  The page's shared parameter block declares a
 * mode (0 = per tensor, 1 = per token) but only per-token kernels are on it;
 * the reading taken here is the per-token rule with the absmax taken over the
 * whole tensor: one scale = max(absmax / 127, 1e-8) for all n values, codes
 * = clamp(rint(x / scale), -128, 127).  x is the flattened tensor. */
void oracle_kv_int8_quant_tensor(const float *x, int8_t *codes, float *scale, i64 n) {
    float max_val = 0.0f;
    for (i64 i = 0; i < n; ++i) max_val = fmaxf(max_val, fabsf(x[i]));
    float s = fmaxf(max_val / 127.0f, 1e-8f);
    *scale = s;
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) {
        int c = (int)rintf(x[i] / s);
        if (c < -128) c = -128;
        if (c > 127) c = 127;
        codes[i] = (int8_t)c;
    }
}

/* [KVQ] INT8 per-tensor dequantization: value = float(code) * scale. */
void oracle_kv_int8_dequant_tensor(const int8_t *codes, float scale, float *y, i64 n) {
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) y[i] = (float)codes[i] * scale;
}

/* [KVQ] the page's "FP8" per-token quantizer, transcribed from its own
 * section.  Its arithmetic is the /127 integer code of the INT8 section (not
 * an E4M3 encoding), kept as a separate function so a test can show the two
 * sections compute the same bytes. */
void oracle_kv_fp8_quant(const float *x, int8_t *codes, float *scales,
                         i64 num_tokens, i64 head_dim) {
    for (i64 t = 0; t < num_tokens; ++t) {
        float m = 0.0f;
        for (i64 d = 0; d < head_dim; ++d) {
            float a = fabsf(x[t * head_dim + d]);
            m = a > m ? a : m;
        }
        float s = m / 127.0f;
        if (s < 1e-8f) s = 1e-8f;
        scales[t] = s;
        for (i64 d = 0; d < head_dim; ++d) {
            i64 q = (i64)rintf(x[t * head_dim + d] / s);
            q = q < -128 ? -128 : (q > 127 ? 127 : q);
            codes[t * head_dim + d] = (int8_t)q;
        }
    }
}

/* [KVQ] "FP8" per-token dequantization: sign-extend the code, times scale. */
void oracle_kv_fp8_dequant(const int8_t *codes, const float *scales, float *y,
                           i64 num_tokens, i64 head_dim) {
    for (i64 t = 0; t < num_tokens; ++t)
        for (i64 d = 0; d < head_dim; ++d)
            y[t * head_dim + d] = (float)(int)codes[t * head_dim + d] * scales[t];
}

/* ------------------------------------------------------------------------ */
/* [KVQ] INT4 per-group asymmetric quantization.
 * Groups are group_size consecutive elements of the flattened
 * [num_tokens * head_dim] array.  Per group: min and max seeded with the first
 * element; scale = (max - min) / 15 (stored as computed, not floored);
 * zero = -min / max(scale, 1e-8); code = clamp(rint((x - min) / max(scale,
 * 1e-8)), 0, 15).  Two codes per byte: even element in the low nibble, odd in
 * the high nibble.  Zeros go to their own array (the page appends them after
 * the scales). */
void oracle_kv_int4_quant(const float *x, uint8_t *packed, float *scales,
                          float *zeros, i64 num_tokens, i64 head_dim,
                          i64 group_size) {
    i64 total_groups = num_tokens * head_dim / group_size;
#pragma omp parallel for schedule(static)
    for (i64 g = 0; g < total_groups; ++g) {
        i64 start = g * group_size;
        float min_val = x[start], max_val = x[start];
        for (i64 i = 0; i < group_size; ++i) {
            float v = x[start + i];
            min_val = fminf(min_val, v);
            max_val = fmaxf(max_val, v);
        }
        float scale = (max_val - min_val) / 15.0f;
        float floored = fmaxf(scale, 1e-8f);
        float zero = -min_val / floored;
        scales[g] = scale;
        zeros[g] = zero;
        for (i64 i = 0; i < group_size; i += 2) {
            int c[2];
            for (int h = 0; h < 2; ++h) {
                float diff = x[start + i + h] - min_val;
                float q = rintf(diff / floored);
                int v = (int)q;
                c[h] = v < 0 ? 0 : (v > 15 ? 15 : v);
            }
            packed[(start + i) / 2] = (uint8_t)(c[0] | (c[1] << 4));
        }
    }
}

/* [KVQ] INT4 per-group dequantization: value = code * scale - zero * scale,
 * two rounded products then one rounded subtraction (no fused multiply-add). */
void oracle_kv_int4_dequant(const uint8_t *packed, const float *scales,
                            const float *zeros, float *y, i64 num_tokens,
                            i64 head_dim, i64 group_size) {
    i64 total_groups = num_tokens * head_dim / group_size;
#pragma omp parallel for schedule(static)
    for (i64 g = 0; g < total_groups; ++g) {
        float scale = scales[g], zero = zeros[g];
        for (i64 i = 0; i < group_size; ++i) {
            i64 e = g * group_size + i;
            uint8_t b = packed[e / 2];
            unsigned q = (e % 2) ? (b >> 4) & 0xFu : b & 0xFu;
            float a = (float)q * scale;
            float zs = zero * scale;
            y[e] = a - zs;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Number formats.  bf16 and OCP E4M3FN are spelled out from their published
 * definitions (bf16 = top 16 bits of binary32; E4M3FN = 1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, largest
 * finite 448). */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float oracle_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u = f2u(f);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

float oracle_e4m3_decode(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    float mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexpf((float)m, -9);              /* m/8 * 2^-6 */
    else mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -mag : mag;
}

/* fp32 -> E4M3FN, round to nearest with ties to even, saturating to +-448,
 * sign kept (so -0 and tiny negatives give 0x80).  Finite input only.
 * Each intermediate below is exact (power-of-two scaling, Sterbenz), so the
 * only rounding is the final rintf. */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (a >= 448.0f) return sign | 0x7E;
    if (a < 0x1p-6f) {                                   /* subnormal range */
        int m = (int)rintf(a * 512.0f);                  /* steps of 2^-9; 8 -> 2^-6 */
        return sign | (uint8_t)m;
    }
    int e = ilogbf(a);                                   /* -6 .. 8 */
    float frac = ldexpf(a, -e) - 1.0f;                   /* [0, 1) */
    int m = (int)rintf(frac * 8.0f);                     /* 0 .. 8, 8 carries */
    int code = ((e + 7) << 3) + m;
    return sign | (uint8_t)code;
}

/* ------------------------------------------------------------------------ */
/* SiLU's exponential, pinned so that both sides reach the same fp32 bits.
 * Method: Cody & Waite argument reduction (W. J. Cody, W. Waite, Software
 * Manual for the Elementary Functions, 1980) with ln 2 split into a 16-bit
 * high part and an fp32 remainder, then the degree-7 Taylor polynomial of
 * e^r (coefficients 1/k! rounded to fp32) by Horner's rule with fused
 * multiply-adds, then a multiply by 2^n built in the exponent field.
 * Inputs above 88 give +inf, below -87 give +0; on [-87, 88] the reduced
 * result times 2^n is always a normal number. */
#define EXPK_L2E    0x1.715476p+0f     /* log2(e) rounded to fp32           */
#define EXPK_LN2_HI 0x1.62e4p-1f       /* ln 2 truncated to 15 fraction bits */
#define EXPK_LN2_LO 0x1.7f7d1cp-20f    /* fp32(ln 2 - EXPK_LN2_HI)          */

float oracle_exp(float y) {
    if (y > 88.0f) return INFINITY;
    if (y < -87.0f) return 0.0f;
    float t = y * EXPK_L2E;
    float n = rintf(t);
    float r = fmaf(-n, EXPK_LN2_HI, y);
    r = fmaf(-n, EXPK_LN2_LO, r);
    float p = 0x1.a01a02p-13f;                  /* 1/7! */
    p = fmaf(p, r, 0x1.6c16c2p-10f);            /* 1/6! */
    p = fmaf(p, r, 0x1.111112p-7f);             /* 1/5! */
    p = fmaf(p, r, 0x1.555556p-5f);             /* 1/4! */
    p = fmaf(p, r, 0x1.555556p-3f);             /* 1/3! */
    p = fmaf(p, r, 0.5f);                       /* 1/2! */
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int ni = (int)n;                            /* -126 .. 127 */
    float two_n = u2f((uint32_t)(ni + 127) << 23);
    return p * two_n;
}

/* silu(v) = v / (1 + e^-v), one rounded add and one IEEE division. */
float oracle_silu(float v) {
    float e = oracle_exp(-v);
    float den = 1.0f + e;
    return v / den;
}

/* ------------------------------------------------------------------------ */
/* [W8A8] activation quantization (w8a8_act_quant / w8a8_act_quant_silu).
 * x is bf16 [rows][ldx]; with silu the value is silu(x), and with up also
 * times up (same ldx).  kind 0 (per-row): one scale per row; kind 1 (g128):
 * one scale per 128 consecutive columns.  scale = max(amax / 448, 1e-8);
 * code = E4M3(value / scale).  q is [rows][k]; scales [rows] or
 * [rows][k/128]. */
static float act_value(const uint16_t *x, const uint16_t *up, i64 idx, int silu) {
    float v = oracle_bf16_to_f32(x[idx]);
    if (silu) v = oracle_silu(v);
    if (up) v = v * oracle_bf16_to_f32(up[idx]);
    return v;
}

void oracle_act_quant(int kind, int silu, const uint16_t *x, const uint16_t *up,
                      i64 ldx, i64 rows, i64 k, uint8_t *q, float *scales) {
    i64 span = kind == 0 ? k : 128;
    i64 nspan = k / span;
#pragma omp parallel for schedule(static)
    for (i64 r = 0; r < rows; ++r) {
        for (i64 g = 0; g < nspan; ++g) {
            float amax = 0.0f;
            for (i64 c = g * span; c < (g + 1) * span; ++c)
                amax = fmaxf(amax, fabsf(act_value(x, up, r * ldx + c, silu)));
            float s = fmaxf(amax / 448.0f, 1e-8f);
            scales[r * nspan + g] = s;
            for (i64 c = g * span; c < (g + 1) * span; ++c)
                q[r * k + c] = oracle_e4m3_encode(act_value(x, up, r * ldx + c, silu) / s);
        }
    }
}

/* Weight quantization to E4M3 with the same rule (offline preparation of the
 * synthetic weights; the page takes already-quantized Fp8Weight segments).
 * kind 0: one scale per weight row (w is [n][k]); kind 1: one scale per
 * 128x128 block, scales [ceil(n/128)][k/128]. */
void oracle_weight_quant(int kind, const float *w, i64 n, i64 k, uint8_t *q,
                         float *scales) {
    if (kind == 0) {
#pragma omp parallel for schedule(static)
        for (i64 j = 0; j < n; ++j) {
            float amax = 0.0f;
            for (i64 c = 0; c < k; ++c) amax = fmaxf(amax, fabsf(w[j * k + c]));
            float s = fmaxf(amax / 448.0f, 1e-8f);
            scales[j] = s;
            for (i64 c = 0; c < k; ++c) q[j * k + c] = oracle_e4m3_encode(w[j * k + c] / s);
        }
        return;
    }
    i64 nb = (n + 127) / 128, kb = k / 128;
#pragma omp parallel for schedule(static)
    for (i64 b = 0; b < nb * kb; ++b) {
        i64 jb = b / kb, cb = b % kb;
        i64 j1 = (jb + 1) * 128 < n ? (jb + 1) * 128 : n;
        float amax = 0.0f;
        for (i64 j = jb * 128; j < j1; ++j)
            for (i64 c = cb * 128; c < cb * 128 + 128; ++c)
                amax = fmaxf(amax, fabsf(w[j * k + c]));
        float s = fmaxf(amax / 448.0f, 1e-8f);
        scales[jb * kb + cb] = s;
        for (i64 j = jb * 128; j < j1; ++j)
            for (i64 c = cb * 128; c < cb * 128 + 128; ++c)
                q[j * k + c] = oracle_e4m3_encode(w[j * k + c] / s);
    }
}

/* ------------------------------------------------------------------------ */
/* [AWQ] nibble order: column j of an 8-column word sits at bit SHIFTS[j]. */
static const unsigned AWQ_SHIFTS[8] = {0, 16, 4, 20, 8, 24, 12, 28};

/* qweight [k][n/8] -> codes [k][n] (one byte per code). */
void oracle_awq_unpack(const uint32_t *qweight, uint8_t *codes, i64 k, i64 n) {
#pragma omp parallel for schedule(static)
    for (i64 r = 0; r < k; ++r)
        for (i64 j = 0; j < n; ++j)
            codes[r * n + j] = (uint8_t)((qweight[r * (n / 8) + j / 8] >> AWQ_SHIFTS[j % 8]) & 0xFu);
}

/* codes [k][n] (values 0..15) -> qweight [k][n/8], the inverse of unpack. */
void oracle_awq_pack(const uint8_t *codes, uint32_t *qweight, i64 k, i64 n) {
    for (i64 r = 0; r < k; ++r)
        for (i64 w = 0; w < n / 8; ++w) {
            uint32_t word = 0;
            for (int j = 0; j < 8; ++j)
                word |= (uint32_t)(codes[r * n + w * 8 + j] & 0xF) << AWQ_SHIFTS[j];
            qweight[r * (n / 8) + w] = word;
        }
}

/* [AWQ] dequantized weight, fp64: w[k][n] = (q - z[k/gs][n]) * s[k/gs][n].
 * The products the page sums (x * ((q - z) * s)) are then a plain fp64 matmul
 * in the Python layer. */
void oracle_awq_dequant_f64(const uint32_t *qweight, const float *scales,
                            const float *zeros, double *w, i64 k, i64 n,
                            i64 group_size) {
#pragma omp parallel for schedule(static)
    for (i64 r = 0; r < k; ++r) {
        i64 g = r / group_size;
        for (i64 j = 0; j < n; ++j) {
            unsigned q = (qweight[r * (n / 8) + j / 8] >> AWQ_SHIFTS[j % 8]) & 0xFu;
            w[r * n + j] = ((double)q - (double)zeros[g * n + j]) * (double)scales[g * n + j];
        }
    }
}

/* E4M3 codes [n][k] with scales -> fp64 values, for the W8A8 reference
 * product.  kind 0: scale[j] per row; kind 1 (weight 128x128 blocks):
 * scale[(j/128)*(k/128) + c/128]; kind 2 (activation 128-groups):
 * scale[j*(k/128) + c/128].  dec(code) has at most 4 significant bits, so
 * each product is exact in fp64. */
void oracle_e4m3_dequant_f64(int kind, const uint8_t *q, const float *scales,
                             double *out, i64 n, i64 k) {
    i64 kb = k / 128;
#pragma omp parallel for schedule(static)
    for (i64 j = 0; j < n; ++j)
        for (i64 c = 0; c < k; ++c) {
            float s = kind == 0 ? scales[j]
                    : kind == 1 ? scales[(j / 128) * kb + c / 128]
                                : scales[j * kb + c / 128];
            out[j * k + c] = (double)oracle_e4m3_decode(q[j * k + c]) * (double)s;
        }
}

/* ------------------------------------------------------------------------ */
/* Array forms of the scalar conversions above (same function per element). */
void oracle_e4m3_encode_array(const float *x, uint8_t *out, i64 n) {
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

void oracle_f32_to_bf16_array(const float *x, uint16_t *out, i64 n) {
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(x[i]);
}

void oracle_exp_array(const float *x, float *out, i64 n) {
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) out[i] = oracle_exp(x[i]);
}

void oracle_silu_array(const float *x, float *out, i64 n) {
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) out[i] = oracle_silu(x[i]);
}
