// W8A8 FP8 quantizers for gfx950: activation quantization (per row or per
// 128-column group, optional SiLU and SiLU*up), offline weight quantization
// (per row or per 128x128 block) and a plain fp32 -> E4M3 cast.
//
// Follows metrale_model_layers w8a8_decode.rs, items w8a8_act_quant,
// w8a8_act_quant_silu, W8a8Scale and W8a8Scratch.  The page launches one
// 256-thread workgroup per activation row and names the device kernels
// (w8a8_act_quant_row / _g128 / _silu_row / _silu_g128) without their source;
// the arithmetic here is the reading stated in kvq.h: scale = max(amax / 448,
// 1e-8) with 448 the largest OCP E4M3FN value and 1e-8 the floor the
// kv_cache_quant page uses, code = E4M3(value / scale) rounded to nearest
// even.  The encoding runs on gfx950's v_cvt_pk_fp8_f32 (OCP E4M3FN, round to
// nearest even in the default mode); the per-group kernel keeps a 128-column
// group in one 16-lane team so the absmax is a 4-step butterfly and every
// lane writes 8 codes with one 8-byte store.
#include "kvq_common.h"
#include "w8a8_act.h"

namespace kvq {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ void load8_f32(const f32x4 *x, uint32_t idx, float v[8]) {
    const f32x4 a = x[2 * idx], b = x[2 * idx + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Max over the 256 threads of the block; every thread gets the result.
__device__ __forceinline__ float block_max(float v, float *red) {
    v = team_absmax<kWave>(v);
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return v;
}

// ------------------------------------------------------------- kernels ---

// One workgroup per row; the row's codes depend on one scale.  Rows of up to
// kRowCached * 8 * 256 columns stay in registers between the block-wide
// absmax and the encoding (one read of the row); longer rows are read again
// (from L2) in a second pass.
constexpr int kRowCached = 4;   // 8-value chunks per thread kept in registers
template <bool SILU, bool UP>
__global__ __launch_bounds__(kBlock) void act_quant_row(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ up, uint32_t ldx,
                                                        uint32_t k, uint8_t *__restrict__ q,
                                                        float *__restrict__ scales) {
    __shared__ float red[4];
    const uint32_t r = blockIdx.x;
    const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + (size_t)r * ldx);
    const u32x4 *ur = UP ? reinterpret_cast<const u32x4 *>(up + (size_t)r * ldx) : nullptr;
    u32x2 *qr = reinterpret_cast<u32x2 *>(q + (size_t)r * k);
    const uint32_t nc = k / 8;
    float m = 0.0f;
    if (nc <= (uint32_t)kBlock * kRowCached) {
        float v[kRowCached][8];
#pragma unroll
        for (int j = 0; j < kRowCached; ++j) {
            const uint32_t c = threadIdx.x + j * kBlock;
            if (c < nc) {
                load8_bf16<SILU, UP>(xr, ur, c, v[j]);
                m = fmaxf(m, absmax8(v[j]));
            }
        }
        const float s = act_scale(block_max(m, red));
        const float y = 1.0f / s;
#pragma unroll
        for (int j = 0; j < kRowCached; ++j) {
            const uint32_t c = threadIdx.x + j * kBlock;
            if (c < nc) qr[c] = encode8(v[j], s, y);
        }
        if (threadIdx.x == 0) scales[r] = s;
        return;
    }
    float v[8];
    for (uint32_t c = threadIdx.x; c < nc; c += kBlock) {
        load8_bf16<SILU, UP>(xr, ur, c, v);
        m = fmaxf(m, absmax8(v));
    }
    const float s = act_scale(block_max(m, red));
    const float y = 1.0f / s;
    for (uint32_t c = threadIdx.x; c < nc; c += kBlock) {
        load8_bf16<SILU, UP>(xr, ur, c, v);
        qr[c] = encode8(v, s, y);
    }
    if (threadIdx.x == 0) scales[r] = s;
}

// 16 lanes per 128-column group, 16 groups per workgroup; grid (ceil(k/2048), rows).
template <bool SILU, bool UP>
__global__ __launch_bounds__(kBlock) void act_quant_g128(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ up, uint32_t ldx,
                                                         uint32_t k, uint8_t *__restrict__ q,
                                                         float *__restrict__ scales) {
    const uint32_t r = blockIdx.y;
    const uint32_t li = threadIdx.x & 15;
    const uint32_t col = blockIdx.x * 2048u + (threadIdx.x >> 4) * 128u + li * 8u;
    const bool ok = col < k;   // k % 128 == 0: a team is wholly in or out
    const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + (size_t)r * ldx);
    const u32x4 *ur = UP ? reinterpret_cast<const u32x4 *>(up + (size_t)r * ldx) : nullptr;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (ok) load8_bf16<SILU, UP>(xr, ur, col / 8, v);
    const float s = act_scale(team_absmax<16>(absmax8(v)));
    const float y = 1.0f / s;
    if (ok) {
        *reinterpret_cast<u32x2 *>(q + (size_t)r * k + col) = encode8(v, s, y);
        if (li == 0) scales[(size_t)r * (k / 128) + col / 128] = s;
    }
}

// Weight rows (fp32): one workgroup per row.
__global__ __launch_bounds__(kBlock) void weight_quant_row(const float *__restrict__ w, uint32_t k,
                                                           uint8_t *__restrict__ q, float *__restrict__ scales) {
    __shared__ float red[4];
    const uint32_t j = blockIdx.x;
    const f32x4 *wr = reinterpret_cast<const f32x4 *>(w + (size_t)j * k);
    u32x2 *qr = reinterpret_cast<u32x2 *>(q + (size_t)j * k);
    float v[8];
    float m = 0.0f;
    for (uint32_t c = threadIdx.x; c < k / 8; c += kBlock) {
        load8_f32(wr, c, v);
        m = fmaxf(m, absmax8(v));
    }
    const float s = act_scale(block_max(m, red));
    const float y = 1.0f / s;
    for (uint32_t c = threadIdx.x; c < k / 8; c += kBlock) {
        load8_f32(wr, c, v);
        qr[c] = encode8(v, s, y);
    }
    if (threadIdx.x == 0) scales[j] = s;
}

// One 128x128 block per workgroup; grid (k/128, ceil(n/128)).  Thread t owns
// columns 4*(t%32)..+3 of rows t/32 + 8*i (i < 16) that exist.
__global__ __launch_bounds__(kBlock) void weight_quant_blk128(const float *__restrict__ w, uint32_t n,
                                                              uint32_t k, uint8_t *__restrict__ q,
                                                              float *__restrict__ scales) {
    __shared__ float red[4];
    const uint32_t cb = blockIdx.x, jb = blockIdx.y;
    const uint32_t c = cb * 128u + (threadIdx.x & 31u) * 4u;
    f32x4 v[16];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t j = jb * 128u + (threadIdx.x >> 5) + 8u * i;
        v[i] = j < n ? *reinterpret_cast<const f32x4 *>(w + (size_t)j * k + c) : f32x4{0.f, 0.f, 0.f, 0.f};
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    const float s = act_scale(block_max(m, red));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t j = jb * 128u + (threadIdx.x >> 5) + 8u * i;
        if (j < n)
            *reinterpret_cast<uint32_t *>(q + (size_t)j * k + c) =
                e4m3x4(v[i].x / s, v[i].y / s, v[i].z / s, v[i].w / s);
    }
    if (threadIdx.x == 0) scales[(size_t)jb * (k / 128) + cb] = s;
}

__global__ __launch_bounds__(kBlock) void cast_e4m3(const float *__restrict__ x, uint8_t *__restrict__ q,
                                                    uint64_t n) {
    const uint64_t i4 = (uint64_t)blockIdx.x * kBlock + threadIdx.x;   // index of a group of 4
    const uint64_t i = i4 * 4;
    if (i + 4 <= n) {
        const f32x4 v = reinterpret_cast<const f32x4 *>(x)[i4];
        reinterpret_cast<uint32_t *>(q)[i4] = e4m3x4(v.x, v.y, v.z, v.w);
    } else if (i < n) {
        for (uint64_t e = i; e < n; ++e) q[e] = (uint8_t)(e4m3x4(x[e], 0.0f, 0.0f, 0.0f) & 0xFFu);
    }
}

// ---------------------------------------------------------------- host ---

}  // namespace

int act_quant_launch(w8a8_scale_t kind, int silu, const uint16_t *x, const uint16_t *up, uint32_t ldx,
                     uint32_t rows, uint32_t k, uint8_t *q, float *a_scales, hipStream_t s) {
    const bool g = kind == W8A8_BLK128;
    const dim3 grid = g ? dim3((k + 2047) / 2048, rows) : dim3(rows);
#define KVQ_ACT(S, U)                                                                               \
    do {                                                                                            \
        if (g) act_quant_g128<S, U><<<grid, kBlock, 0, s>>>(x, up, ldx, k, q, a_scales);            \
        else act_quant_row<S, U><<<grid, kBlock, 0, s>>>(x, up, ldx, k, q, a_scales);               \
    } while (0)
    if (!silu) KVQ_ACT(false, false);
    else if (!up) KVQ_ACT(true, false);
    else KVQ_ACT(true, true);
#undef KVQ_ACT
    return launch_status("w8a8_act_quant");
}

int check_act_quant(const char *fn, w8a8_scale_t kind, int silu, const uint16_t *x, const uint16_t *up,
                    uint32_t ldx, uint32_t rows, uint32_t k, const uint8_t *q, const float *a_scales) {
    if (kind != W8A8_ROWSCALE && kind != W8A8_BLK128)
        return fail(KVQ_E_INVALID, "%s: scale kind %d is not per-row (0) or 128x128 block (1)", fn, (int)kind);
    if (rows < 1 || rows > W8A8_MAX_ROWS)
        return fail(KVQ_E_INVALID, "%s: %u rows (want 1..=%u)", fn, rows, W8A8_MAX_ROWS);
    if (k == 0 || k % W8A8_K_UNIT || ldx < k || ldx % 8)
        return fail(KVQ_E_INVALID, "%s: K=%u, ldx=%u (want K %% 128 == 0, K > 0, ldx >= K, ldx %% 8 == 0)", fn, k,
                    ldx);
    if (!silu && up) return fail(KVQ_E_INVALID, "%s: up is only used with silu", fn);
    int st = check_ptrs(fn, {x, q, a_scales});
    if (st) return st;
    if (up && !aligned16(up)) return fail(KVQ_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
    return KVQ_OK;
}

}  // namespace kvq

using namespace kvq;

extern "C" int w8a8_act_quant(w8a8_scale_t kind, int silu, const uint16_t *x, const uint16_t *up, uint32_t ldx,
                              uint32_t rows, uint32_t k, uint8_t *q, float *a_scales, void *stream) {
    int st = check_act_quant("w8a8_act_quant", kind, silu, x, up, ldx, rows, k, q, a_scales);
    if (st) return st;
    return act_quant_launch(kind, silu, x, up, ldx, rows, k, q, a_scales, as_stream(stream));
}

extern "C" int w8a8_scratch_bytes(w8a8_scale_t kind, uint32_t rows, uint32_t k, size_t *q_bytes,
                                  size_t *scale_bytes) {
    if (!q_bytes || !scale_bytes) return fail(KVQ_E_INVALID, "w8a8_scratch_bytes: null output pointer");
    if (kind != W8A8_ROWSCALE && kind != W8A8_BLK128)
        return fail(KVQ_E_INVALID, "w8a8_scratch_bytes: scale kind %d is not 0 or 1", (int)kind);
    *q_bytes = (size_t)rows * k;
    const size_t per_row = kind == W8A8_ROWSCALE ? 1 : ((k + W8A8_K_UNIT - 1) / W8A8_K_UNIT ?: 1);
    *scale_bytes = (size_t)rows * per_row * 4;
    return KVQ_OK;
}

extern "C" int w8a8_weight_quant(w8a8_scale_t kind, const float *w, uint32_t n, uint32_t k, uint8_t *q,
                                 float *scales, void *stream) {
    const char *fn = "w8a8_weight_quant";
    if (kind != W8A8_ROWSCALE && kind != W8A8_BLK128)
        return fail(KVQ_E_INVALID, "%s: scale kind %d is not 0 or 1", fn, (int)kind);
    if (n == 0 || k == 0 || k % W8A8_K_UNIT)
        return fail(KVQ_E_INVALID, "%s: n=%u K=%u (want n > 0, K a positive multiple of 128)", fn, n, k);
    int st = check_ptrs(fn, {w, q, scales});
    if (st) return st;
    hipStream_t s = as_stream(stream);
    if (kind == W8A8_ROWSCALE) weight_quant_row<<<n, kBlock, 0, s>>>(w, k, q, scales);
    else weight_quant_blk128<<<dim3(k / 128, (n + 127) / 128), kBlock, 0, s>>>(w, n, k, q, scales);
    return launch_status(fn);
}

extern "C" int kvq_f32_to_e4m3(const float *x, uint8_t *q, uint64_t n, void *stream) {
    const char *fn = "kvq_f32_to_e4m3";
    if (n == 0) return fail(KVQ_E_INVALID, "%s: n == 0", fn);
    int st = check_ptrs(fn, {x, q});
    if (st) return st;
    const uint64_t groups = (n + 3) / 4;
    const uint64_t blocks = (groups + kBlock - 1) / kBlock;
    if (blocks > 0x7FFFFFFFull) return fail(KVQ_E_INVALID, "%s: n=%llu too large", fn, (unsigned long long)n);
    cast_e4m3<<<(unsigned)blocks, kBlock, 0, as_stream(stream)>>>(x, q, n);
    return launch_status(fn);
}
