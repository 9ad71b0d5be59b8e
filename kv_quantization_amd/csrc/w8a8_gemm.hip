// W8A8 FP8 GEMV/GEMM for gfx950: out = bf16(sum_k dec(qa) * sa * dec(W) * sw)
// over 1..3 concatenated E4M3 weight segments, per-row or 128x128-block scales.
//
// Follows metrale_model_layers w8a8_decode.rs: W8a8Weight (segments, their
// boundaries and alignment), w8a8_gemv (validation, per-row vs Block128
// kernels, bf16 output with leading dimension ldc) and w8a8_proj.  The page's
// device kernels are not shown; it launches ceil(N/16) workgroups of 256
// threads over <=128-row chunks, re-streaming the weights per chunk.  Here
// every call is one launch over all (<=256) rows:
//
//   * rows <= 64  "skinny": a workgroup owns 16 output columns; its 4 waves
//     split K, each streaming 16 weight rows with 16-byte loads straight into
//     MFMA operands (v_mfma_scale_f32_16x16x128_f8f6f4, unit E8M0 scales, so
//     one instruction is one 128-wide scale block) and the activation rows
//     as the other operand; partial sums meet in LDS.
//   * rows > 64   "tiled": 64x64 output tiles, activation and weight tiles
//     staged through padded LDS rows (conflict-free 16-byte reads), double
//     buffered so the next K block's global loads overlap the MFMAs.
//
// Operand layout: for a 16x16x128 fp8 MFMA, lane l supplies row (l % 16) of
// A (or column (l % 16) of B) and 32 bytes of K.  Lane l carries K bytes
// [16*(l/16), +16) and [64 + 16*(l/16), +16) of the 128-wide block, the same
// for A and B, so the sum over K is complete and one load instruction reads
// 64 contiguous bytes of each row.  The result tile has column (l % 16) and
// rows 4*(l/16) + i in register i.
//
// Block scales: each MFMA covers exactly one 128-wide K block, so its fresh
// result is multiplied by sa[m][kb] * sw[jb][kb] in fp32 and added to the
// accumulator (fp32 accumulation throughout; products of two E4M3 values are
// exact in the MFMA).
#include "kvq_common.h"

namespace kvq {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBlock = 256;

struct Segs {
    const uint8_t *w[3];
    const float *s[3];
    uint32_t start[3];   // first global column of each segment
    uint32_t n[3];       // rows of each segment
    uint32_t count;
    uint32_t ntotal;
};

// Segment holding global column j (segments are contiguous and ordered).
__device__ __forceinline__ int seg_of(const Segs &S, uint32_t j) {
    return (S.count > 1 && j >= S.start[1]) ? ((S.count > 2 && j >= S.start[2]) ? 2 : 1) : 0;
}

__device__ __forceinline__ i32x8 load_frag(const uint8_t *p) {
    // 16 bytes at p and 16 bytes at p + 64 (see the operand layout above)
    const u32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    const u32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + 64));
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

__device__ __forceinline__ i32x8 load_frag_cached(const uint8_t *p) {
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 64);
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x4 &c) {
    // format codes 0/0 = E4M3 for both operands; E8M0 scale 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ------------------------------------------------------------- skinny ---

// MT 16-row tiles of activations (rows <= 16*MT); KIND 0 per-row, 1 block.
template <int MT, int KIND>
__global__ __launch_bounds__(kBlock) void w8a8_skinny(const uint8_t *__restrict__ q, const float *__restrict__ sa,
                                                      uint32_t rows, uint32_t K, Segs S, uint16_t *__restrict__ out,
                                                      uint32_t ldc) {
    __shared__ f32x4 red[4][MT][kWave];
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const uint32_t n0 = blockIdx.x * 16u;
    const int sg = seg_of(S, n0);
    const uint32_t jloc0 = n0 - S.start[sg];
    const uint32_t jrow = jloc0 + r16;
    const bool jok = jrow < S.n[sg];
    const uint8_t *wrow = S.w[sg] + (size_t)(jok ? jrow : 0) * K + g * 16;
    const uint32_t nkb = K / 128;
    const uint32_t kb0 = wv * nkb / 4, kb1 = (wv + 1) * nkb / 4;

    const uint8_t *arow[MT];
    bool aok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint32_t m = mt * 16 + r16;
        aok[mt] = m < rows;
        arow[mt] = q + (size_t)(aok[mt] ? m : 0) * K + g * 16;
    }
    // per-lane output rows of the result tile (for block scales)
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const i32x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint32_t kbs = K / 128;

    constexpr int U = MT >= 3 ? 2 : 4;
    uint32_t kb = kb0;
    for (; kb + U <= kb1; kb += U) {
        i32x8 b[U], a[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            b[u] = jok ? load_frag(wrow + (size_t)(kb + u) * 128) : zero8;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                a[u][mt] = aok[mt] ? load_frag_cached(arow[mt] + (size_t)(kb + u) * 128) : zero8;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (KIND == 0) {
                    acc[mt] = mfma_fp8(a[u][mt], b[u], acc[mt]);
                } else {
                    const f32x4 p = mfma_fp8(a[u][mt], b[u], f32x4{0.f, 0.f, 0.f, 0.f});
                    const float swb = S.s[sg][(size_t)(jloc0 / 128) * kbs + kb + u];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t m = mt * 16 + 4 * g + i;
                        const float sab = m < rows ? sa[(size_t)m * kbs + kb + u] : 0.0f;
                        acc[mt][i] = __builtin_fmaf(p[i], sab * swb, acc[mt][i]);
                    }
                }
            }
        }
    }
    for (; kb < kb1; ++kb) {
        const i32x8 b = jok ? load_frag(wrow + (size_t)kb * 128) : zero8;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const i32x8 a = aok[mt] ? load_frag_cached(arow[mt] + (size_t)kb * 128) : zero8;
            if (KIND == 0) {
                acc[mt] = mfma_fp8(a, b, acc[mt]);
            } else {
                const f32x4 p = mfma_fp8(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
                const float swb = S.s[sg][(size_t)(jloc0 / 128) * kbs + kb];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t m = mt * 16 + 4 * g + i;
                    const float sab = m < rows ? sa[(size_t)m * kbs + kb] : 0.0f;
                    acc[mt][i] = __builtin_fmaf(p[i], sab * swb, acc[mt][i]);
                }
            }
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wv][mt][lane] = acc[mt];
    __syncthreads();
    if (wv < MT) {
        const int mt = wv;
        const f32x4 t = red[0][mt][lane] + red[1][mt][lane] + red[2][mt][lane] + red[3][mt][lane];
        const uint32_t j = n0 + r16;
        if (jok) {
            const float sw = KIND == 0 ? S.s[sg][jrow] : 1.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t m = mt * 16 + 4 * g + i;
                if (m < rows) {
                    const float y = KIND == 0 ? t[i] * sa[m] * sw : t[i];
                    out[(size_t)m * ldc + j] = bf16_rne(y);
                }
            }
        }
    }
}

// -------------------------------------------------------------- tiled ---

constexpr int kTile = 64;                 // output tile 64 x 64
constexpr int kLdsRow = 144;              // 128 bytes of K + 16 bytes pad

// KIND 0 per-row, 1 block scales.  grid (ceil(N/64), ceil(rows/64)).
template <int KIND>
__global__ __launch_bounds__(kBlock) void w8a8_tiled(const uint8_t *__restrict__ q, const float *__restrict__ sa,
                                                     uint32_t rows, uint32_t K, Segs S, uint16_t *__restrict__ out,
                                                     uint32_t ldc) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kTile * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kTile * kLdsRow];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;            // wave's 32x32 sub-tile
    const int r16 = lane & 15, g = lane >> 4;
    const uint32_t n0 = blockIdx.x * kTile, m0 = blockIdx.y * kTile;
    const uint32_t nkb = K / 128;

    // global -> LDS assignment: thread t moves 16-byte chunks c = t and t+256
    // of each 64 x 128-byte tile: row c/8, column chunk c%8.
    const uint8_t *ga[2];
    const uint8_t *gb[2];
    bool oka[2], okb[2];
    int ldsoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = tid + h * kBlock;
        const int row = c >> 3, col = (c & 7) * 16;
        ldsoff[h] = row * kLdsRow + col;
        const uint32_t m = m0 + row;
        oka[h] = m < rows;
        ga[h] = q + (size_t)(oka[h] ? m : 0) * K + col;
        const uint32_t j = n0 + row;
        okb[h] = j < S.ntotal;
        const int sg = seg_of(S, okb[h] ? j : 0);
        const uint32_t jl = (okb[h] ? j : 0) - S.start[sg];
        okb[h] = okb[h] && jl < S.n[sg];
        gb[h] = S.w[sg] + (size_t)(okb[h] ? jl : 0) * K + col;
    }
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    u32x4 ra[2], rb[2];
    auto gload = [&](uint32_t kb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            ra[h] = oka[h] ? *reinterpret_cast<const u32x4 *>(ga[h] + (size_t)kb * 128) : z4;
            rb[h] = okb[h] ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(gb[h] + (size_t)kb * 128))
                           : z4;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            *reinterpret_cast<u32x4 *>(&lds_a[buf][ldsoff[h]]) = ra[h];
            *reinterpret_cast<u32x4 *>(&lds_b[buf][ldsoff[h]]) = rb[h];
        }
    };

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // block-scale bookkeeping: the 64-column tile lies in one 128-row band
    // of one segment (BLK128 segments start at multiples of 128)
    const int sg_blk = seg_of(S, n0);
    const float *swp = S.s[sg_blk] + (size_t)((n0 - S.start[sg_blk]) / 128) * nkb;

    gload(0);
    lstore(0);
    __syncthreads();
    for (uint32_t kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nkb) gload(kb + 1);
        i32x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint8_t *pa = &lds_a[buf][(wm * 32 + i * 16 + r16) * kLdsRow + g * 16];
            const uint8_t *pb = &lds_b[buf][(wn * 32 + i * 16 + r16) * kLdsRow + g * 16];
            const u32x4 alo = *reinterpret_cast<const u32x4 *>(pa), ahi = *reinterpret_cast<const u32x4 *>(pa + 64);
            const u32x4 blo = *reinterpret_cast<const u32x4 *>(pb), bhi = *reinterpret_cast<const u32x4 *>(pb + 64);
            a[i] = i32x8{(int)alo[0], (int)alo[1], (int)alo[2], (int)alo[3], (int)ahi[0], (int)ahi[1], (int)ahi[2],
                         (int)ahi[3]};
            b[i] = i32x8{(int)blo[0], (int)blo[1], (int)blo[2], (int)blo[3], (int)bhi[0], (int)bhi[1], (int)bhi[2],
                         (int)bhi[3]};
        }
        if (KIND == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma_fp8(a[i], b[j], acc[i][j]);
        } else {
            const float swb = swp[kb];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float sab[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t m = m0 + wm * 32 + i * 16 + 4 * g + e;
                    sab[e] = (m < rows ? sa[(size_t)m * nkb + kb] : 0.0f) * swb;
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const f32x4 p = mfma_fp8(a[i], b[j], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(p[e], sab[e], acc[i][j][e]);
                }
            }
        }
        if (kb + 1 < nkb) {
            lstore(buf ^ 1);
            __syncthreads();
        }
    }

    // epilogue
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t col = n0 + wn * 32 + j * 16 + r16;
        if (col >= S.ntotal) continue;
        const int sg = seg_of(S, col);
        const uint32_t jl = col - S.start[sg];
        if (jl >= S.n[sg]) continue;
        const float sw = KIND == 0 ? S.s[sg][jl] : 1.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t m = m0 + wm * 32 + i * 16 + 4 * g + e;
                if (m < rows) {
                    const float y = KIND == 0 ? acc[i][j][e] * sa[m] * sw : acc[i][j][e];
                    out[(size_t)m * ldc + col] = bf16_rne(y);
                }
            }
        }
    }
}

// --------------------------------------------------------------- host ---

int check_gemv(const char *fn, w8a8_scale_t kind, const uint8_t *q, const float *a_scales, uint32_t rows, uint32_t k,
               const w8a8_segment_t *segs, uint32_t nseg, const uint16_t *out, uint32_t ldc, Segs *S) {
    if (kind != W8A8_ROWSCALE && kind != W8A8_BLK128)
        return fail(KVQ_E_INVALID, "%s: scale kind %d is not per-row (0) or 128x128 block (1)", fn, (int)kind);
    if (rows < 1 || rows > W8A8_MAX_ROWS)
        return fail(KVQ_E_INVALID, "%s: %u rows (want 1..=%u)", fn, rows, W8A8_MAX_ROWS);
    if (k == 0 || k % W8A8_K_UNIT)
        return fail(KVQ_E_INVALID, "%s: K=%u is not a positive multiple of %u", fn, k, W8A8_K_UNIT);
    if (!segs || nseg < 1 || nseg > 3) return fail(KVQ_E_INVALID, "%s: %u segments, want 1..=3", fn, segs ? nseg : 0);
    const uint32_t align = kind == W8A8_ROWSCALE ? 16 : 128;
    uint64_t total = 0;
    for (uint32_t i = 0; i < nseg; ++i) {
        if (segs[i].n == 0 || !segs[i].w || !segs[i].scale)
            return fail(KVQ_E_INVALID, "%s: segment %u is empty", fn, i);
        if (!aligned16(segs[i].w) || !aligned16(segs[i].scale))
            return fail(KVQ_E_INVALID, "%s: segment %u pointers must be 16-byte aligned", fn, i);
        if (i + 1 < nseg && segs[i].n % align)
            return fail(KVQ_E_INVALID, "%s: segment %u has %u rows, not a multiple of %u", fn, i, segs[i].n, align);
        S->w[i] = segs[i].w;
        S->s[i] = segs[i].scale;
        S->start[i] = (uint32_t)total;
        S->n[i] = segs[i].n;
        total += segs[i].n;
    }
    if (total > 0xFFFFFFF0ull) return fail(KVQ_E_INVALID, "%s: total N too large", fn);
    for (uint32_t i = nseg; i < 3; ++i) {
        S->w[i] = segs[0].w;
        S->s[i] = segs[0].scale;
        S->start[i] = (uint32_t)total;
        S->n[i] = 0;
    }
    S->count = nseg;
    S->ntotal = (uint32_t)total;
    if (ldc < total) return fail(KVQ_E_INVALID, "%s: ldc=%u < N=%u", fn, ldc, (uint32_t)total);
    if (!q || !a_scales || !out) return fail(KVQ_E_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(q) || !aligned16(a_scales) || !aligned16(out))
        return fail(KVQ_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
    return KVQ_OK;
}

int gemv_launch(w8a8_scale_t kind, const uint8_t *q, const float *a_scales, uint32_t rows, uint32_t k, const Segs &S,
                uint16_t *out, uint32_t ldc, hipStream_t s) {
    if (rows <= 64) {
        const unsigned grid = (S.ntotal + 15) / 16;
        const int mt = (rows + 15) / 16;
#define KVQ_SKINNY(MT)                                                                                        \
    do {                                                                                                      \
        if (kind == W8A8_ROWSCALE) w8a8_skinny<MT, 0><<<grid, kBlock, 0, s>>>(q, a_scales, rows, k, S, out, ldc); \
        else w8a8_skinny<MT, 1><<<grid, kBlock, 0, s>>>(q, a_scales, rows, k, S, out, ldc);                  \
    } while (0)
        switch (mt) {
            case 1: KVQ_SKINNY(1); break;
            case 2: KVQ_SKINNY(2); break;
            case 3: KVQ_SKINNY(3); break;
            default: KVQ_SKINNY(4); break;
        }
#undef KVQ_SKINNY
    } else {
        const dim3 grid((S.ntotal + kTile - 1) / kTile, (rows + kTile - 1) / kTile);
        if (kind == W8A8_ROWSCALE) w8a8_tiled<0><<<grid, kBlock, 0, s>>>(q, a_scales, rows, k, S, out, ldc);
        else w8a8_tiled<1><<<grid, kBlock, 0, s>>>(q, a_scales, rows, k, S, out, ldc);
    }
    return launch_status("w8a8_gemv");
}

}  // namespace

int act_quant_launch(w8a8_scale_t kind, int silu, const uint16_t *x, const uint16_t *up, uint32_t ldx,
                     uint32_t rows, uint32_t k, uint8_t *q, float *a_scales, hipStream_t s);
int check_act_quant(const char *fn, w8a8_scale_t kind, int silu, const uint16_t *x, const uint16_t *up,
                    uint32_t ldx, uint32_t rows, uint32_t k, const uint8_t *q, const float *a_scales);

}  // namespace kvq

using namespace kvq;

extern "C" int w8a8_gemv(w8a8_scale_t kind, const uint8_t *q, const float *a_scales, uint32_t rows, uint32_t k,
                         const w8a8_segment_t *segs, uint32_t nseg, uint16_t *out, uint32_t ldc, void *workspace,
                         size_t workspace_bytes, void *stream) {
    (void)workspace;
    (void)workspace_bytes;
    Segs S;
    int st = check_gemv("w8a8_gemv", kind, q, a_scales, rows, k, segs, nseg, out, ldc, &S);
    if (st) return st;
    return gemv_launch(kind, q, a_scales, rows, k, S, out, ldc, as_stream(stream));
}

extern "C" int w8a8_gemv_workspace_bytes(w8a8_scale_t kind, uint32_t rows, uint32_t k, uint32_t n_total,
                                         size_t *bytes) {
    (void)kind; (void)rows; (void)k; (void)n_total;
    if (!bytes) return fail(KVQ_E_INVALID, "w8a8_gemv_workspace_bytes: null output pointer");
    *bytes = 0;
    return KVQ_OK;
}

extern "C" int w8a8_proj(w8a8_scale_t kind, int silu, const uint16_t *x, const uint16_t *up, uint32_t ldx,
                         uint32_t rows, uint32_t k, const w8a8_segment_t *segs, uint32_t nseg, uint16_t *out,
                         uint32_t ldc, uint8_t *q, float *a_scales, void *workspace, size_t workspace_bytes,
                         void *stream) {
    int st = check_act_quant("w8a8_proj", kind, silu, x, up, ldx, rows, k, q, a_scales);
    if (st) return st;
    Segs S;
    st = check_gemv("w8a8_proj", kind, q, a_scales, rows, k, segs, nseg, out, ldc, &S);
    if (st) return st;
    st = act_quant_launch(kind, silu, x, up, ldx, rows, k, q, a_scales, as_stream(stream));
    if (st) return st;
    (void)workspace;
    (void)workspace_bytes;
    return gemv_launch(kind, q, a_scales, rows, k, S, out, ldc, as_stream(stream));
}
