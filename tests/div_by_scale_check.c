/*
 * CPU check of the quotient the quantization kernels compute instead of an
 * IEEE division by the scale: y = RN(1/s) once per token, group or row, then
 * q = RN(v*y) and one fused correction RN(q + (v - q*s)*y), with a zero
 * input passed through unchanged (the kernels' div_by_scale).  Compared, in
 * fp32 with fmaf (correctly rounded) and no contraction, against the IEEE
 * quotient v/s over the (v, s) pairs the codecs produce:
 *
 *   INT8 per token:  s = max(RN(amax/127), 1e-8),  |v| <= amax
 *   E4M3 act quant:  s = max(RN(amax/448), 1e-8),  |v| <= amax
 *   INT4 per group:  s = max(RN(range/15), 1e-8),  0 <= v <= range
 *
 * on seeded random pairs (amax over the whole fp32 exponent range) plus the
 * boundaries where a code changes: the half-integer quotients of the INT8 and
 * INT4 codes, the midpoints between E4M3 values, E4M3's zero threshold 2^-10,
 * each with neighbouring fp32 values, the absmax element itself and signed
 * zeros.
 *
 * A pair passes when both quotients have the same bits, or when both are
 * below 2^-60 in magnitude with the same sign (every code is then zero:
 * rint gives 0, and E4M3 gives the zero of that sign).  Prints one summary
 * line; exit status 0 when every pair passes.
 *
 * Build: cc -O2 -ffp-contract=off div_by_scale_check.c -lm
 * Run:   ./a.out SEED PAIRS_PER_DIVISOR
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t rng_state;

/* splitmix64 (Steele, Lea, Flood: "Fast splittable pseudorandom number
 * generators", 2014) */
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static float bits_to_f(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t f_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* the kernels' sequence, operation for operation (built with
 * -DWITHOUT_CORRECTION it stops at the product, which the check must reject) */
static float quotient_via_reciprocal(float v, float s, float y) {
    const float q = v * y;
#ifdef WITHOUT_CORRECTION
    const float r = q;
    (void)s;
#else
    const float r = fmaf(fmaf(-q, s, v), y, q);
#endif
    return v == 0.0f ? v : r;
}

static unsigned long long pairs, equal, tiny, bad;
static double max_tiny;

static void check(float v, float s) {
    const float y = 1.0f / s;
    const float qi = v / s;
    const float qr = quotient_via_reciprocal(v, s, y);
    ++pairs;
    if (f_to_bits(qi) == f_to_bits(qr)) {
        ++equal;
        return;
    }
    const float lim = 0x1p-60f;
    if (fabsf(qi) < lim && fabsf(qr) < lim && signbit(qi) == signbit(qr) && rintf(qi) == rintf(qr)) {
        ++tiny;
        if (fabs((double)qi) > max_tiny) max_tiny = fabs((double)qi);
        return;
    }
    if (bad < 10)
        fprintf(stderr, "mismatch: v=%a s=%a ieee=%a reciprocal=%a\n", (double)v, (double)s, (double)qi,
                (double)qr);
    ++bad;
}

/* v = RN(t * s) and its fp32 neighbours: quotients on either side of t
 * (skipped where t * s is past the largest float: no input is) */
static void around(float t, float s) {
    float v = t * s;
    if (!isfinite(v) || !isfinite(nextafterf(v, INFINITY))) return;
    float lo = v, hi = v;
    check(v, s);
    for (int i = 0; i < 3; ++i) {
        lo = nextafterf(lo, -INFINITY);
        hi = nextafterf(hi, INFINITY);
        check(lo, s);
        check(hi, s);
    }
}

/* positive E4M3FN values (bias 7, no infinities, 448 the largest) */
static int e4m3_values(float *out) {
    int n = 0;
    for (int e = 0; e < 16; ++e)
        for (int m = 0; m < 8; ++m) {
            if (e == 15 && m == 7) continue;   /* NaN */
            out[n++] = e == 0 ? ldexpf((float)m / 8.0f, -6) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
        }
    return n;
}

static float random_amax(void) {
    /* every normal exponent, random mantissa */
    const uint32_t e = 1 + (uint32_t)(next_u64() % 254);
    return bits_to_f((e << 23) | (uint32_t)(next_u64() & 0x7FFFFF));
}

int main(int argc, char **argv) {
    rng_state = argc > 1 ? strtoull(argv[1], NULL, 10) : 1;
    const unsigned long long per = argc > 2 ? strtoull(argv[2], NULL, 10) : 1000000ull;
    const float divisors[3] = {127.0f, 448.0f, 15.0f};
    float e4[128];
    const int ne4 = e4m3_values(e4);

    for (int d = 0; d < 3; ++d) {
        const float D = divisors[d];
        for (unsigned long long i = 0; i < per; ++i) {
            const float amax = random_amax();
            const float s = fmaxf(amax / D, 1e-8f);
            /* |v| <= amax, random magnitude and sign */
            const float u = (float)((next_u64() >> 40) * 0x1p-24);
            float v = amax * u;
            if (d != 2 && (next_u64() & 1)) v = -v;
            check(v, s);
            if ((i & 1023) == 0) {
                check(amax, s);        /* the absmax element */
                check(-amax, s);
                check(0.0f, s);
                check(-0.0f, s);
            }
            if ((i & 4095) == 0) {
                /* code boundaries for this scale */
                if (d == 1) {
                    for (int j = 0; j + 1 < ne4; ++j) around(0.5f * (e4[j] + e4[j + 1]), s);
                    around(0x1p-10f, s);
                } else {
                    const int top = d == 0 ? 128 : 15;
                    for (int k = 0; k < top; ++k) around((float)k + 0.5f, s);
                }
            }
        }
        /* the floored scale and the largest scales, exhaustively over code boundaries */
        const float edge_s[4] = {1e-8f, fmaxf(0x1p-100f / D, 1e-8f), 0x1.fffffep127f / D, 1.0f};
        for (int j = 0; j < 4; ++j)
            for (int k = 0; k < 128; ++k) around((float)k + 0.5f, edge_s[j]);
    }
    printf("pairs=%llu equal=%llu tiny=%llu bad=%llu max_tiny=%a\n", pairs, equal, tiny, bad, max_tiny);
    return bad == 0 ? 0 : 1;
}
