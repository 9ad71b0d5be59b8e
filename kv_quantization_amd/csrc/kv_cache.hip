// KV-cache quantization for gfx950: symmetric per-token INT8 and asymmetric
// per-group INT4, quantize and dequantize.
//
// Follows boostr kv_cache_quant.wgsl, sections "INT8 Per-Token
// Quantization/Dequantization" (the "FP8 Per-Token" sections compute the same
// code) and "INT4 Per-Group Quantization/Dequantization".  The page runs one
// thread per token or group with strided, uncoalesced loops; here a team of
// lanes owns a token (INT8) or group (INT4): each lane holds 4 consecutive
// fp32 values from one 16-byte load, so a wave64 load instruction reads 1 KiB
// of contiguous memory, the absmax/min/max is a butterfly over the team, and
// each lane writes its packed codes with one 4-byte (INT8) or 2-byte (INT4)
// store.  Shapes the teams cannot tile fall back to one wave per unit.
//
// Numerics match the page's fp32 arithmetic: the scale itself is an IEEE
// division; each element's quotient x / scale comes from the scale's
// reciprocal (once per token or group), a product and one fused correction
// (div_by_scale), which yields the correctly rounded IEEE quotient for every
// pair these codecs form (a CPU test checks the sequence against IEEE
// division), so the codes are those of a division; round-half-to-even via
// v_rndne_f32; no other fused multiply-add (the library is built with
// -ffp-contract=off).
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr int kBlock = 256;           // 4 waves
constexpr int kWavesPerBlock = kBlock / kWave;
// 16-byte loads per lane per wave.  Small waves measured faster: the loads
// of many short waves spread over the whole kernel instead of one burst.
constexpr int kQuantUnroll = 2;
constexpr int kDequantUnroll = 2;

// y = 1/s (see div_by_scale)
__device__ __forceinline__ uint32_t int8_code(float v, float s, float y) {
    int c = (int)__builtin_rintf(div_by_scale(v, s, y));
    c = c < -128 ? -128 : (c > 127 ? 127 : c);
    return (uint32_t)c & 0xFFu;
}

__device__ __forceinline__ float int8_scale(float amax) { return fmaxf(amax / 127.0f, 1e-8f); }

// Element I/O.  DT 0: fp32 values in memory; 1: fp16; 2: bf16.  Values are
// fp32 in registers: 16-bit inputs widen exactly, so the arithmetic is that
// of the fp32 codec on the same numbers; 16-bit outputs round the fp32
// result to nearest even.  Index i4 counts groups of 4 consecutive values.
template <int DT>
__device__ __forceinline__ float from16(uint32_t h) {
    if (DT == 1) return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    return __uint_as_float(h << 16);
}
template <int DT>
__device__ __forceinline__ uint32_t to16(float f) {
    if (DT == 1) return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
template <int DT>
__device__ __forceinline__ f32x4 load4(const void *p, uint64_t i4) {
    if (DT == 0) return __builtin_nontemporal_load(static_cast<const f32x4 *>(p) + i4);
    const u32x2 w = __builtin_nontemporal_load(static_cast<const u32x2 *>(p) + i4);
    return f32x4{from16<DT>(w.x & 0xFFFFu), from16<DT>(w.x >> 16), from16<DT>(w.y & 0xFFFFu), from16<DT>(w.y >> 16)};
}
template <int DT>
__device__ __forceinline__ float load1(const void *p, uint64_t i) {
    if (DT == 0) return static_cast<const float *>(p)[i];
    return from16<DT>(static_cast<const uint16_t *>(p)[i]);
}
template <int DT>
__device__ __forceinline__ void store4(void *p, uint64_t i4, f32x4 v) {
    if (DT == 0) {
        __builtin_nontemporal_store(v, static_cast<f32x4 *>(p) + i4);
    } else {
        const u32x2 w = {to16<DT>(v.x) | (to16<DT>(v.y) << 16), to16<DT>(v.z) | (to16<DT>(v.w) << 16)};
        __builtin_nontemporal_store(w, static_cast<u32x2 *>(p) + i4);
    }
}
template <int DT>
__device__ __forceinline__ void store1(void *p, uint64_t i, float v) {
    if (DT == 0) static_cast<float *>(p)[i] = v;
    else static_cast<uint16_t *>(p)[i] = (uint16_t)to16<DT>(v);
}

// y = 1/sf (see div_by_scale)
__device__ __forceinline__ uint32_t int4_code(float v, float mn, float sf, float y) {
    float d = v - mn;
    int c = (int)__builtin_rintf(div_by_scale(d, sf, y));
    c = c < 0 ? 0 : (c > 15 ? 15 : c);
    return (uint32_t)c;
}

__device__ __forceinline__ float abs_max4(f32x4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ uint64_t global_wave() {
    return (uint64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
}

// ------------------------------------------------------------ INT8 ------

// L lanes per token (head_dim = 4L); a wave covers U*(64/L) tokens.
template <int L, int U, int DT>
__global__ __launch_bounds__(kBlock) void int8_quant_team(const void *__restrict__ x,
                                                          uint32_t *__restrict__ codes,
                                                          float *__restrict__ scales,
                                                          uint64_t num_tokens) {
    constexpr int TPI = kWave / L;
    const int lane = lane_id();
    const int sub = lane / L, li = lane % L;
    const uint64_t t0 = global_wave() * (U * TPI) + sub;
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t t = t0 + (uint64_t)u * TPI;
        v[u] = t < num_tokens ? load4<DT>(x, t * L + li) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t t = t0 + (uint64_t)u * TPI;
        const float s = int8_scale(team_absmax<L>(abs_max4(v[u])));
        const float y = 1.0f / s;
        const uint32_t packed = int8_code(v[u].x, s, y) | (int8_code(v[u].y, s, y) << 8) |
                                (int8_code(v[u].z, s, y) << 16) | (int8_code(v[u].w, s, y) << 24);
        if (t < num_tokens) {
            codes[t * L + li] = packed;
            if (li == 0) scales[t] = s;
        }
    }
}

// Any head_dim: one wave per token.
template <int DT>
__global__ __launch_bounds__(kBlock) void int8_quant_wave(const void *__restrict__ x,
                                                          int8_t *__restrict__ codes,
                                                          float *__restrict__ scales,
                                                          uint64_t num_tokens, uint32_t head_dim) {
    const uint64_t t = global_wave();
    if (t >= num_tokens) return;
    const uint64_t row = t * head_dim;
    float m = 0.0f;
    for (uint32_t d = lane_id(); d < head_dim; d += kWave) m = fmaxf(m, fabsf(load1<DT>(x, row + d)));
    const float s = int8_scale(team_absmax<kWave>(m));
    if (lane_id() == 0) scales[t] = s;
    for (uint32_t d = lane_id(); d < head_dim; d += kWave)
        codes[row + d] = (int8_t)(uint8_t)int8_code(load1<DT>(x, row + d), s, 1.0f / s);
}

template <int L, int U, int DT>
__global__ __launch_bounds__(kBlock) void int8_dequant_team(const uint32_t *__restrict__ codes,
                                                            const float *__restrict__ scales,
                                                            void *__restrict__ y,
                                                            uint64_t num_tokens) {
    constexpr int TPI = kWave / L;
    const int lane = lane_id();
    const int sub = lane / L, li = lane % L;
    const uint64_t t0 = global_wave() * (U * TPI) + sub;
    uint32_t w[U];
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t t = t0 + (uint64_t)u * TPI;
        const bool ok = t < num_tokens;
        w[u] = ok ? __builtin_nontemporal_load(&codes[t * L + li]) : 0u;
        s[u] = ok ? scales[t] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t t = t0 + (uint64_t)u * TPI;
        f32x4 o;
        o.x = (float)(int8_t)(w[u]) * s[u];
        o.y = (float)(int8_t)(w[u] >> 8) * s[u];
        o.z = (float)(int8_t)(w[u] >> 16) * s[u];
        o.w = (float)(int8_t)(w[u] >> 24) * s[u];
        if (t < num_tokens) store4<DT>(y, t * L + li, o);
    }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void int8_dequant_wave(const int8_t *__restrict__ codes,
                                                            const float *__restrict__ scales,
                                                            void *__restrict__ y,
                                                            uint64_t num_tokens, uint32_t head_dim) {
    const uint64_t t = global_wave();
    if (t >= num_tokens) return;
    const float s = scales[t];
    for (uint32_t d = lane_id(); d < head_dim; d += kWave)
        store1<DT>(y, t * head_dim + d, (float)codes[t * head_dim + d] * s);
}

// ------------------------------------------------------ INT8 per tensor --
//
// The declared per-tensor mode: one scale from the absmax of the whole
// tensor.  Pass 1: each of up to kTensorBlocks workgroups takes a
// grid-strided share of the flattened tensor and writes its absmax to the
// caller's workspace.  Pass 2: each workgroup issues the loads of its slice,
// then reduces all partials (the max is exact in any order, so every
// workgroup gets the same scale), and encodes its slice; the second read of
// the tensor is served by the MALL for tensors that fit it.  Values past the
// last multiple of 4 are handled one per thread by the last workgroup.
constexpr uint32_t kTensorBlocks = 512;
static_assert(KVQ_INT8_TENSOR_WORKSPACE_BYTES >= KVQ_WORKSPACE_COUNTER_BYTES + kTensorBlocks * 4, "workspace size");
constexpr int kTensorUnroll = 4;

__global__ __launch_bounds__(kBlock) void int8_tensor_absmax(const float *__restrict__ x, uint64_t n,
                                                             float *__restrict__ partials) {
    __shared__ float red[kWavesPerBlock];
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
    const uint64_t n4 = n / 4;
    const uint64_t stride = (uint64_t)gridDim.x * kBlock;
    uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    float m = 0.0f;
    for (; i + (kTensorUnroll - 1) * stride < n4; i += kTensorUnroll * stride) {
        f32x4 v[kTensorUnroll];
#pragma unroll
        for (int u = 0; u < kTensorUnroll; ++u) v[u] = x4[i + u * stride];
#pragma unroll
        for (int u = 0; u < kTensorUnroll; ++u) m = fmaxf(m, abs_max4(v[u]));
    }
    for (; i < n4; i += stride) m = fmaxf(m, abs_max4(x4[i]));
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x < n - n4 * 4) m = fmaxf(m, fabsf(x[n4 * 4 + threadIdx.x]));
    m = team_absmax<kWave>(m);
    if (lane_id() == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) partials[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(kBlock) void int8_tensor_quant(const float *__restrict__ x, uint64_t n,
                                                            const float *__restrict__ partials, uint32_t np,
                                                            int8_t *__restrict__ codes, float *__restrict__ scale) {
    __shared__ float red[kWavesPerBlock];
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
    uint32_t *c4 = reinterpret_cast<uint32_t *>(codes);
    const uint64_t n4 = n / 4;
    const uint64_t i0 = (uint64_t)blockIdx.x * (kBlock * kTensorUnroll) + threadIdx.x;
    f32x4 v[kTensorUnroll];
#pragma unroll
    for (int u = 0; u < kTensorUnroll; ++u) {
        const uint64_t i = i0 + (uint64_t)u * kBlock;
        v[u] = i < n4 ? __builtin_nontemporal_load(&x4[i]) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m = 0.0f;
    for (uint32_t p = threadIdx.x; p < np; p += kBlock) m = fmaxf(m, partials[p]);
    m = team_absmax<kWave>(m);
    if (lane_id() == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    const float s = int8_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    const float y = 1.0f / s;
#pragma unroll
    for (int u = 0; u < kTensorUnroll; ++u) {
        const uint64_t i = i0 + (uint64_t)u * kBlock;
        if (i < n4)
            c4[i] = int8_code(v[u].x, s, y) | (int8_code(v[u].y, s, y) << 8) | (int8_code(v[u].z, s, y) << 16) |
                    (int8_code(v[u].w, s, y) << 24);
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x < n - n4 * 4) {
        const uint64_t e = n4 * 4 + threadIdx.x;
        codes[e] = (int8_t)(uint8_t)int8_code(x[e], s, y);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
}

__global__ __launch_bounds__(kBlock) void int8_tensor_dequant(const int8_t *__restrict__ codes,
                                                              const float *__restrict__ scale,
                                                              float *__restrict__ y, uint64_t n) {
    const uint32_t *c4 = reinterpret_cast<const uint32_t *>(codes);
    f32x4 *y4 = reinterpret_cast<f32x4 *>(y);
    const uint64_t n4 = n / 4;
    const float s = *scale;
    const uint64_t i0 = (uint64_t)blockIdx.x * (kBlock * kTensorUnroll) + threadIdx.x;
    uint32_t w[kTensorUnroll];
#pragma unroll
    for (int u = 0; u < kTensorUnroll; ++u) {
        const uint64_t i = i0 + (uint64_t)u * kBlock;
        w[u] = i < n4 ? __builtin_nontemporal_load(&c4[i]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kTensorUnroll; ++u) {
        const uint64_t i = i0 + (uint64_t)u * kBlock;
        f32x4 o;
        o.x = (float)(int8_t)(w[u]) * s;
        o.y = (float)(int8_t)(w[u] >> 8) * s;
        o.z = (float)(int8_t)(w[u] >> 16) * s;
        o.w = (float)(int8_t)(w[u] >> 24) * s;
        if (i < n4) __builtin_nontemporal_store(o, &y4[i]);
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x < n - n4 * 4) {
        const uint64_t e = n4 * 4 + threadIdx.x;
        y[e] = (float)codes[e] * s;
    }
}

// ------------------------------------------------------------ INT4 ------

// L lanes per group (group_size = 4L); a wave covers U*(64/L) groups.
template <int L, int U, int DT>
__global__ __launch_bounds__(kBlock) void int4_quant_team(const void *__restrict__ x,
                                                          uint16_t *__restrict__ packed,
                                                          float *__restrict__ scales,
                                                          float *__restrict__ zeros,
                                                          uint64_t num_groups) {
    constexpr int GPI = kWave / L;
    const int lane = lane_id();
    const int sub = lane / L, li = lane % L;
    const uint64_t g0 = global_wave() * (U * GPI) + sub;
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t g = g0 + (uint64_t)u * GPI;
        v[u] = g < num_groups ? load4<DT>(x, g * L + li) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t g = g0 + (uint64_t)u * GPI;
        const float mn = team_min<L>(fminf(fminf(v[u].x, v[u].y), fminf(v[u].z, v[u].w)));
        const float mx = team_max<L>(fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
        const float s = (mx - mn) / 15.0f;
        const float sf = fmaxf(s, 1e-8f);
        const float z = -mn / sf;
        const float y = 1.0f / sf;
        const uint32_t p = int4_code(v[u].x, mn, sf, y) | (int4_code(v[u].y, mn, sf, y) << 4) |
                           (int4_code(v[u].z, mn, sf, y) << 8) | (int4_code(v[u].w, mn, sf, y) << 12);
        if (g < num_groups) {
            packed[g * L + li] = (uint16_t)p;
            if (li == 0) {
                scales[g] = s;
                zeros[g] = z;
            }
        }
    }
}

// Any even group_size: one wave per group, one byte (two codes) per step.
template <int DT>
__global__ __launch_bounds__(kBlock) void int4_quant_wave(const void *__restrict__ x,
                                                          uint8_t *__restrict__ packed,
                                                          float *__restrict__ scales,
                                                          float *__restrict__ zeros,
                                                          uint64_t num_groups, uint32_t group_size) {
    const uint64_t g = global_wave();
    if (g >= num_groups) return;
    const uint64_t g0 = g * group_size;
    float mn = load1<DT>(x, g0), mx = mn;
    for (uint32_t i = lane_id(); i < group_size; i += kWave) {
        const float v = load1<DT>(x, g0 + i);
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
    mn = team_min<kWave>(mn);
    mx = team_max<kWave>(mx);
    const float s = (mx - mn) / 15.0f;
    const float sf = fmaxf(s, 1e-8f);
    const float z = -mn / sf;
    if (lane_id() == 0) {
        scales[g] = s;
        zeros[g] = z;
    }
    uint8_t *out = packed + g * (group_size / 2);
    for (uint32_t p = lane_id(); p < group_size / 2; p += kWave)
        out[p] = (uint8_t)(int4_code(load1<DT>(x, g0 + 2 * p), mn, sf, 1.0f / sf) |
                           (int4_code(load1<DT>(x, g0 + 2 * p + 1), mn, sf, 1.0f / sf) << 4));
}

template <int L, int U, int DT>
__global__ __launch_bounds__(kBlock) void int4_dequant_team(const uint16_t *__restrict__ packed,
                                                            const float *__restrict__ scales,
                                                            const float *__restrict__ zeros,
                                                            void *__restrict__ y,
                                                            uint64_t num_groups) {
    constexpr int GPI = kWave / L;
    const int lane = lane_id();
    const int sub = lane / L, li = lane % L;
    const uint64_t g0 = global_wave() * (U * GPI) + sub;
    uint32_t w[U];
    float s[U], z[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t g = g0 + (uint64_t)u * GPI;
        const bool ok = g < num_groups;
        w[u] = ok ? packed[g * L + li] : 0u;
        s[u] = ok ? scales[g] : 0.0f;
        z[u] = ok ? zeros[g] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t g = g0 + (uint64_t)u * GPI;
        const float zs = z[u] * s[u];
        f32x4 o;
        o.x = (float)(w[u] & 15u) * s[u] - zs;
        o.y = (float)((w[u] >> 4) & 15u) * s[u] - zs;
        o.z = (float)((w[u] >> 8) & 15u) * s[u] - zs;
        o.w = (float)((w[u] >> 12) & 15u) * s[u] - zs;
        if (g < num_groups) store4<DT>(y, g * L + li, o);
    }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void int4_dequant_wave(const uint8_t *__restrict__ packed,
                                                            const float *__restrict__ scales,
                                                            const float *__restrict__ zeros,
                                                            void *__restrict__ y,
                                                            uint64_t num_groups, uint32_t group_size) {
    const uint64_t g = global_wave();
    if (g >= num_groups) return;
    const float s = scales[g];
    const float zs = zeros[g] * s;
    const uint8_t *in = packed + g * (group_size / 2);
    const uint64_t o0 = g * group_size;
    for (uint32_t p = lane_id(); p < group_size / 2; p += kWave) {
        const uint32_t b = in[p];
        store1<DT>(y, o0 + 2 * p, (float)(b & 15u) * s - zs);
        store1<DT>(y, o0 + 2 * p + 1, (float)(b >> 4) * s - zs);
    }
}

// ------------------------------------------------------------ host ------

inline unsigned blocks_for(uint64_t units, uint64_t units_per_block) {
    return (unsigned)((units + units_per_block - 1) / units_per_block);
}

// Team width for a row of `elems` fp32 values split 4 per lane, or 0.
inline int team_lanes(uint64_t elems) {
    if (elems % 4) return 0;
    const uint64_t l = elems / 4;
    return (l >= 1 && l <= 64 && (l & (l - 1)) == 0) ? (int)l : 0;
}

#define KVQ_TEAM_SWITCH(L, CALL)              \
    switch (L) {                              \
        case 1: { constexpr int LL = 1; CALL; } break;   \
        case 2: { constexpr int LL = 2; CALL; } break;   \
        case 4: { constexpr int LL = 4; CALL; } break;   \
        case 8: { constexpr int LL = 8; CALL; } break;   \
        case 16: { constexpr int LL = 16; CALL; } break; \
        case 32: { constexpr int LL = 32; CALL; } break; \
        default: { constexpr int LL = 64; CALL; } break; \
    }

int check_kv_common(const char *fn, const void *a, const void *b, const void *c,
                    uint32_t num_tokens, uint32_t head_dim) {
    if (!a || !b || !c) return fail(KVQ_E_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(a) || !aligned16(b) || !aligned16(c))
        return fail(KVQ_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
    if (num_tokens == 0 || head_dim == 0)
        return fail(KVQ_E_INVALID, "%s: num_tokens=%u head_dim=%u (want both >= 1)", fn, num_tokens, head_dim);
    return KVQ_OK;
}

int check_int4(const char *fn, const void *a, const void *b, const void *c, const void *d,
               uint32_t num_tokens, uint32_t head_dim, uint32_t group_size) {
    int st = check_kv_common(fn, a, b, c, num_tokens, head_dim);
    if (st) return st;
    if (!d) return fail(KVQ_E_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(d)) return fail(KVQ_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
    const uint64_t total = (uint64_t)num_tokens * head_dim;
    if (group_size < 2 || group_size % 2 || total % group_size)
        return fail(KVQ_E_INVALID,
                    "%s: group_size=%u must be even, >= 2 and divide num_tokens*head_dim=%llu", fn,
                    group_size, (unsigned long long)total);
    return KVQ_OK;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

namespace kvq {
namespace {

int check_dtype(const char *fn, int dt) {
    if (dt != KVQ_DT_F32 && dt != KVQ_DT_F16 && dt != KVQ_DT_BF16)
        return fail(KVQ_E_INVALID, "%s: dtype %d is not fp32 (0), fp16 (1) or bf16 (2)", fn, dt);
    return KVQ_OK;
}

#define KVQ_DT_SWITCH(DTV, CALL)                                  \
    switch (DTV) {                                                \
        case KVQ_DT_F32: { constexpr int D_ = 0; CALL; } break;   \
        case KVQ_DT_F16: { constexpr int D_ = 1; CALL; } break;   \
        default: { constexpr int D_ = 2; CALL; } break;           \
    }

int int8_quant(const char *fn, const void *x, int dt, int8_t *codes, float *scales, uint32_t num_tokens,
               uint32_t head_dim, hipStream_t s) {
    int st = check_kv_common(fn, x, codes, scales, num_tokens, head_dim);
    if (!st) st = check_dtype(fn, dt);
    if (st) return st;
    const int L = team_lanes(head_dim);
    if (L) {
        const uint64_t per_block = (uint64_t)kWavesPerBlock * kQuantUnroll * (kWave / L);
        KVQ_DT_SWITCH(dt, KVQ_TEAM_SWITCH(L, (int8_quant_team<LL, kQuantUnroll, D_><<<blocks_for(num_tokens, per_block),
                                                                                       kBlock, 0, s>>>(
                                                 x, (uint32_t *)codes, scales, num_tokens))));
    } else {
        KVQ_DT_SWITCH(dt, (int8_quant_wave<D_><<<blocks_for(num_tokens, kWavesPerBlock), kBlock, 0, s>>>(
                              x, codes, scales, num_tokens, head_dim)));
    }
    return launch_status(fn);
}

int int8_dequant(const char *fn, const int8_t *codes, const float *scales, void *y, int dt, uint32_t num_tokens,
                 uint32_t head_dim, hipStream_t s) {
    int st = check_kv_common(fn, codes, scales, y, num_tokens, head_dim);
    if (!st) st = check_dtype(fn, dt);
    if (st) return st;
    const int L = team_lanes(head_dim);
    if (L) {
        const uint64_t per_block = (uint64_t)kWavesPerBlock * kDequantUnroll * (kWave / L);
        KVQ_DT_SWITCH(dt, KVQ_TEAM_SWITCH(L, (int8_dequant_team<LL, kDequantUnroll, D_><<<
                                                 blocks_for(num_tokens, per_block), kBlock, 0, s>>>(
                                                 (const uint32_t *)codes, scales, y, num_tokens))));
    } else {
        KVQ_DT_SWITCH(dt, (int8_dequant_wave<D_><<<blocks_for(num_tokens, kWavesPerBlock), kBlock, 0, s>>>(
                              codes, scales, y, num_tokens, head_dim)));
    }
    return launch_status(fn);
}

int int4_quant(const char *fn, const void *x, int dt, uint8_t *packed, float *scales, float *zeros,
               uint32_t num_tokens, uint32_t head_dim, uint32_t group_size, hipStream_t s) {
    int st = check_int4(fn, x, packed, scales, zeros, num_tokens, head_dim, group_size);
    if (!st) st = check_dtype(fn, dt);
    if (st) return st;
    const uint64_t groups = (uint64_t)num_tokens * head_dim / group_size;
    const int L = team_lanes(group_size);
    if (L) {
        const uint64_t per_block = (uint64_t)kWavesPerBlock * kQuantUnroll * (kWave / L);
        KVQ_DT_SWITCH(dt, KVQ_TEAM_SWITCH(L, (int4_quant_team<LL, kQuantUnroll, D_><<<blocks_for(groups, per_block),
                                                                                       kBlock, 0, s>>>(
                                                 x, (uint16_t *)packed, scales, zeros, groups))));
    } else {
        KVQ_DT_SWITCH(dt, (int4_quant_wave<D_><<<blocks_for(groups, kWavesPerBlock), kBlock, 0, s>>>(
                              x, packed, scales, zeros, groups, group_size)));
    }
    return launch_status(fn);
}

int int4_dequant(const char *fn, const uint8_t *packed, const float *scales, const float *zeros, void *y, int dt,
                 uint32_t num_tokens, uint32_t head_dim, uint32_t group_size, hipStream_t s) {
    int st = check_int4(fn, packed, scales, zeros, y, num_tokens, head_dim, group_size);
    if (!st) st = check_dtype(fn, dt);
    if (st) return st;
    const uint64_t groups = (uint64_t)num_tokens * head_dim / group_size;
    const int L = team_lanes(group_size);
    if (L) {
        const uint64_t per_block = (uint64_t)kWavesPerBlock * kDequantUnroll * (kWave / L);
        KVQ_DT_SWITCH(dt, KVQ_TEAM_SWITCH(L, (int4_dequant_team<LL, kDequantUnroll, D_><<<
                                                 blocks_for(groups, per_block), kBlock, 0, s>>>(
                                                 (const uint16_t *)packed, scales, zeros, y, groups))));
    } else {
        KVQ_DT_SWITCH(dt, (int4_dequant_wave<D_><<<blocks_for(groups, kWavesPerBlock), kBlock, 0, s>>>(
                              packed, scales, zeros, y, groups, group_size)));
    }
    return launch_status(fn);
}

}  // namespace
}  // namespace kvq

extern "C" int kvq_quant_int8_token(const float *x, int8_t *codes, float *scales, uint32_t num_tokens,
                                    uint32_t head_dim, void *stream) {
    return int8_quant("kvq_quant_int8_token", x, KVQ_DT_F32, codes, scales, num_tokens, head_dim, as_stream(stream));
}

extern "C" int kvq_dequant_int8_token(const int8_t *codes, const float *scales, float *y, uint32_t num_tokens,
                                      uint32_t head_dim, void *stream) {
    return int8_dequant("kvq_dequant_int8_token", codes, scales, y, KVQ_DT_F32, num_tokens, head_dim,
                        as_stream(stream));
}

extern "C" int kvq_quant_fp8_token(const float *x, int8_t *codes, float *scales, uint32_t num_tokens,
                                   uint32_t head_dim, void *stream) {
    return kvq_quant_int8_token(x, codes, scales, num_tokens, head_dim, stream);
}

extern "C" int kvq_dequant_fp8_token(const int8_t *codes, const float *scales, float *y, uint32_t num_tokens,
                                     uint32_t head_dim, void *stream) {
    return kvq_dequant_int8_token(codes, scales, y, num_tokens, head_dim, stream);
}

extern "C" int kvq_quant_int4_group(const float *x, uint8_t *packed, float *scales, float *zeros,
                                    uint32_t num_tokens, uint32_t head_dim, uint32_t group_size, void *stream) {
    return int4_quant("kvq_quant_int4_group", x, KVQ_DT_F32, packed, scales, zeros, num_tokens, head_dim,
                      group_size, as_stream(stream));
}

extern "C" int kvq_dequant_int4_group(const uint8_t *packed, const float *scales, const float *zeros, float *y,
                                      uint32_t num_tokens, uint32_t head_dim, uint32_t group_size, void *stream) {
    return int4_dequant("kvq_dequant_int4_group", packed, scales, zeros, y, KVQ_DT_F32, num_tokens, head_dim,
                        group_size, as_stream(stream));
}

extern "C" int kvq_quant_int8_token_dt(const void *x, int x_dtype, int8_t *codes, float *scales,
                                       uint32_t num_tokens, uint32_t head_dim, void *stream) {
    return int8_quant("kvq_quant_int8_token_dt", x, x_dtype, codes, scales, num_tokens, head_dim, as_stream(stream));
}

extern "C" int kvq_dequant_int8_token_dt(const int8_t *codes, const float *scales, void *y, int y_dtype,
                                         uint32_t num_tokens, uint32_t head_dim, void *stream) {
    return int8_dequant("kvq_dequant_int8_token_dt", codes, scales, y, y_dtype, num_tokens, head_dim,
                        as_stream(stream));
}

extern "C" int kvq_quant_int4_group_dt(const void *x, int x_dtype, uint8_t *packed, float *scales, float *zeros,
                                       uint32_t num_tokens, uint32_t head_dim, uint32_t group_size, void *stream) {
    return int4_quant("kvq_quant_int4_group_dt", x, x_dtype, packed, scales, zeros, num_tokens, head_dim,
                      group_size, as_stream(stream));
}

extern "C" int kvq_dequant_int4_group_dt(const uint8_t *packed, const float *scales, const float *zeros, void *y,
                                         int y_dtype, uint32_t num_tokens, uint32_t head_dim, uint32_t group_size,
                                         void *stream) {
    return int4_dequant("kvq_dequant_int4_group_dt", packed, scales, zeros, y, y_dtype, num_tokens, head_dim,
                        group_size, as_stream(stream));
}

extern "C" int kvq_quant_int8_tensor(const float *x, int8_t *codes, float *scale, uint32_t num_tokens,
                                     uint32_t head_dim, void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "kvq_quant_int8_tensor";
    int st = check_kv_common(fn, x, codes, scale, num_tokens, head_dim);
    if (st) return st;
    if (!workspace || !aligned16(workspace) || workspace_bytes < KVQ_INT8_TENSOR_WORKSPACE_BYTES)
        return fail(KVQ_E_INVALID, "%s: needs a 16-byte aligned workspace of >= %u bytes (got %zu)", fn,
                    KVQ_INT8_TENSOR_WORKSPACE_BYTES, workspace ? workspace_bytes : (size_t)0);
    const uint64_t n = (uint64_t)num_tokens * head_dim;
    const uint64_t n4 = n / 4;
    uint64_t np = (n4 + kBlock - 1) / kBlock;
    np = np < 1 ? 1 : (np > kTensorBlocks ? kTensorBlocks : np);
    float *partials = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + KVQ_WORKSPACE_COUNTER_BYTES);
    hipStream_t s = as_stream(stream);
    int8_tensor_absmax<<<(unsigned)np, kBlock, 0, s>>>(x, n, partials);
    st = launch_status(fn);
    if (st) return st;
    const uint64_t blocks = n4 ? (n4 + kBlock * kTensorUnroll - 1) / (kBlock * kTensorUnroll) : 1;
    if (blocks > 0x7FFFFFFFull) return fail(KVQ_E_INVALID, "%s: tensor too large", fn);
    int8_tensor_quant<<<(unsigned)blocks, kBlock, 0, s>>>(x, n, partials, (uint32_t)np, codes, scale);
    return launch_status(fn);
}

extern "C" int kvq_dequant_int8_tensor(const int8_t *codes, const float *scale, float *y, uint32_t num_tokens,
                                       uint32_t head_dim, void *stream) {
    const char *fn = "kvq_dequant_int8_tensor";
    int st = check_kv_common(fn, codes, scale, y, num_tokens, head_dim);
    if (st) return st;
    const uint64_t n = (uint64_t)num_tokens * head_dim;
    const uint64_t n4 = n / 4;
    const uint64_t blocks = n4 ? (n4 + kBlock * kTensorUnroll - 1) / (kBlock * kTensorUnroll) : 1;
    if (blocks > 0x7FFFFFFFull) return fail(KVQ_E_INVALID, "%s: tensor too large", fn);
    int8_tensor_dequant<<<(unsigned)blocks, kBlock, 0, as_stream(stream)>>>(codes, scale, y, n);
    return launch_status(fn);
}
