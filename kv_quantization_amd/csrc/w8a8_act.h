// Activation arithmetic of the W8A8 quantizers (metrale_model_layers
// w8a8_decode.rs, w8a8_act_quant and w8a8_act_quant_silu; the formula is the
// reading stated in kvq.h), shared by the stand-alone quantizer kernels and
// the GEMV that quantizes its own activations, so both produce the same codes.
#ifndef KVQ_W8A8_ACT_H
#define KVQ_W8A8_ACT_H

#include "kvq_common.h"

namespace kvq {

// SiLU's exponential with a fixed operation sequence (so both this library
// and an independent implementation of the same method agree bit for bit):
// Cody & Waite argument reduction, e^y = 2^n * e^r with n = rint(y*log2 e),
// r = y - n*ln2 in two fused steps (ln 2 = HI + LO, HI keeping 15 fraction
// bits so n*HI is exact), then the degree-7 Taylor polynomial of e^r with
// coefficients 1/k! rounded to fp32, by Horner's rule with fused
// multiply-adds, and a multiply by 2^n built in the exponent field.  Above 88
// the result is +inf and below -87 it is +0; between them 2^n stays normal.
__device__ __forceinline__ float silu_exp(float y) {
    if (y > 88.0f) return __builtin_inff();
    if (y < -87.0f) return 0.0f;
    const float n = __builtin_rintf(y * 0x1.715476p+0f);        // log2(e) in fp32
    float r = __builtin_fmaf(-n, 0x1.62e4p-1f, y);                // ln2 high part
    r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);                   // ln2 - high, in fp32
    float p = 0x1.a01a02p-13f;                                    // 1/5040
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);                    // 1/720
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);                     // 1/120
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);                     // 1/24
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);                     // 1/6
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return p * __int_as_float(((int)n + 127) << 23);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + silu_exp(-v)); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four fp32 values -> four E4M3FN codes, byte i = code of value i.  The
// hardware conversion rounds to nearest even but turns magnitudes that round
// past 448 into the NaN code, so inputs are first clamped to [-448, 448]
// (v_med3_f32; it keeps the sign and every in-range value).
__device__ __forceinline__ float sat448(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), r, true);
    return (uint32_t)r;
}

__device__ __forceinline__ float act_scale(float amax) { return fmaxf(amax / 448.0f, 1e-8f); }

// The 8 activation values held by 16 bytes of bf16 x (and of up): f32(x),
// silu(f32(x)) or silu(f32(x)) * f32(up).
template <bool SILU, bool UP>
__device__ __forceinline__ void act8(const u32x4 &w, const u32x4 &u, float v[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
    if (SILU) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = silu(v[i]);
    }
    if (UP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = v[2 * i] * bf16_lo(u[i]);
            v[2 * i + 1] = v[2 * i + 1] * bf16_hi(u[i]);
        }
    }
}

// 8 consecutive activation values from 16-byte loads of x (and up).
template <bool SILU, bool UP>
__device__ __forceinline__ void load8_bf16(const u32x4 *x, const u32x4 *up, uint32_t idx, float v[8]) {
    const u32x4 w = x[idx];
    const u32x4 u = UP ? up[idx] : w;
    act8<SILU, UP>(w, u, v);
}

__device__ __forceinline__ float absmax8(const float v[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    return m;
}

// y = 1/s (see div_by_scale)
__device__ __forceinline__ u32x2 encode8(const float v[8], float s, float y) {
    u32x2 r;
    r.x = e4m3x4(div_by_scale(v[0], s, y), div_by_scale(v[1], s, y), div_by_scale(v[2], s, y),
                 div_by_scale(v[3], s, y));
    r.y = e4m3x4(div_by_scale(v[4], s, y), div_by_scale(v[5], s, y), div_by_scale(v[6], s, y),
                 div_by_scale(v[7], s, y));
    return r;
}

}  // namespace kvq

#endif
