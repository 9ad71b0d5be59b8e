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
//   * rows <= 32  "skinny": a workgroup owns a few 16-column tiles (a pair of
//     workgroups shares three, so 6144 columns make 256 equal workgroups);
//     its waves split K, each streaming 16 weight rows per tile with 16-byte
//     loads straight into MFMA operands (v_mfma_scale_f32_16x16x128_f8f6f4,
//     unit E8M0 scales, so one instruction is one 128-wide scale block) and
//     the activation rows as the other operand; partial sums meet in LDS.
//     Up to 8 rows the same kernel can quantize the bf16 activations itself
//     (the single-launch projection).
//   * rows > 32   "wide": all rows x 128 columns per workgroup over a slice
//     of K; 4 loader waves fill LDS rings (3 to 6 stages of the activation
//     and weight tiles) with direct global->LDS loads while 8 waves multiply,
//     one barrier per K step; split-K partials are added by a second kernel.
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
#include "w8a8_act.h"

namespace kvq {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

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

// Cache-policy operand of the buffer intrinsics for streamed weights: nt
// (non-temporal), as the nontemporal global loads below.
constexpr int kAuxNt = 2;

// Column tile nt (16 output columns) of this workgroup and the lanes (weight
// rows r16 in [rlo, rhi)) it loads.  Plain: NT consecutive tiles.  Balanced
// (BAL, NT == 2): a pair of workgroups shares three tiles, the first taking
// tile 3p and rows 0-7 of tile 3p+1, the second rows 8-15 of tile 3p+1 and
// tile 3p+2, so 384 tiles make 256 equal workgroups (one per CU) instead of
// 384 (half the CUs with twice the bytes); the MFMA lanes of the other half
// tile read zeros.
template <int NT, bool BAL>
__device__ __forceinline__ void col_tile(int nt, uint32_t &tile, uint32_t &rlo, uint32_t &rhi) {
    if (!BAL) {
        tile = blockIdx.x * NT + nt;
        rlo = 0;
        rhi = 16;
    } else {
        static_assert(!BAL || NT == 2, "balanced tiling pairs two column tiles");
        const uint32_t h = blockIdx.x & 1u;
        tile = 3u * (blockIdx.x >> 1) + h + nt;
        rlo = (h == 1 && nt == 0) ? 8u : 0u;
        rhi = (h == 0 && nt == 1) ? 8u : 16u;
    }
}

template <int NT, bool BAL>
inline unsigned col_grid(uint32_t ntotal) {
    const uint32_t tiles = (ntotal + 15) / 16;
    return BAL ? 2 * ((tiles + 2) / 3) : (tiles + NT - 1) / NT;
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

// rows <= 32: a workgroup owns NT 16-column tiles; its W waves split K, each
// streaming the weight rows of its slice with 16-byte loads straight into
// MFMA operands (U K blocks in flight per lane) and the activation rows (L2)
// as the other operand; partial sums meet in LDS.  MT 16-row tiles of
// activations (rows <= 16*MT); KIND 0 per-row, 1 block scales.  NT > 1 reuses
// each activation fragment for several column tiles.
template <int MT, int NT, int W, int U, int KIND, bool BAL>
__global__ __launch_bounds__(W * kWave) void w8a8_skinny(const uint8_t *__restrict__ q,
                                                          const float *__restrict__ sa, uint32_t rows, uint32_t K,
                                                          Segs S, uint16_t *__restrict__ out, uint32_t ldc) {
    __shared__ f32x4 red[W][MT * NT][kWave];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const uint32_t nkb = K / 128;
    const uint32_t kb0 = wv * nkb / W, kb1 = (wv + 1) * nkb / W;

    int sg[NT];
    uint32_t jloc0[NT], jrow[NT], n0s[NT];
    bool jok[NT];
    const uint8_t *wrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        uint32_t tile, rlo, rhi;
        col_tile<NT, BAL>(nt, tile, rlo, rhi);
        const uint32_t n0 = tile * 16u;
        n0s[nt] = n0;
        const uint32_t nn = n0 < S.ntotal ? n0 : 0;
        sg[nt] = seg_of(S, nn);
        jloc0[nt] = nn - S.start[sg[nt]];
        jrow[nt] = jloc0[nt] + r16;
        jok[nt] = n0 < S.ntotal && jrow[nt] < S.n[sg[nt]] && (uint32_t)r16 >= rlo && (uint32_t)r16 < rhi;
        wrow[nt] = S.w[sg[nt]] + (size_t)(jok[nt] ? jrow[nt] : 0) * K + g * 16;
    }
    const uint8_t *arow[MT];
    bool aok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint32_t m = mt * 16 + r16;
        aok[mt] = m < rows;
        arow[mt] = q + (size_t)(aok[mt] ? m : 0) * K + g * 16;
    }
    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const i32x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

    auto step = [&](uint32_t kb, const i32x8 *b, const i32x8 *a) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (KIND == 0) {
                    acc[mt][nt] = mfma_fp8(a[mt], b[nt], acc[mt][nt]);
                } else {
                    const f32x4 p = mfma_fp8(a[mt], b[nt], f32x4{0.f, 0.f, 0.f, 0.f});
                    const float swb = S.s[sg[nt]][(size_t)(jloc0[nt] / 128) * nkb + kb];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t m = mt * 16 + 4 * g + i;
                        const float sab = m < rows ? sa[(size_t)m * nkb + kb] : 0.0f;
                        acc[mt][nt][i] = __builtin_fmaf(p[i], sab * swb, acc[mt][nt][i]);
                    }
                }
            }
        }
    };
    uint32_t kb = kb0;
    for (; kb + U <= kb1; kb += U) {
        i32x8 b[U][NT], a[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) b[u][nt] = jok[nt] ? load_frag(wrow[nt] + (size_t)(kb + u) * 128) : zero8;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                a[u][mt] = aok[mt] ? load_frag_cached(arow[mt] + (size_t)(kb + u) * 128) : zero8;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) step(kb + u, b[u], a[u]);
    }
    for (; kb < kb1; ++kb) {
        i32x8 b[NT], a[MT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) b[nt] = jok[nt] ? load_frag(wrow[nt] + (size_t)kb * 128) : zero8;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) a[mt] = aok[mt] ? load_frag_cached(arow[mt] + (size_t)kb * 128) : zero8;
        step(kb, b, a);
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[wv][mt * NT + nt][lane] = acc[mt][nt];
    __syncthreads();
    for (int t = wv; t < MT * NT; t += W) {
        const int mt = t / NT, nt = t % NT;
        f32x4 v = red[0][t][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += red[w][t][lane];
        if (jok[nt]) {
            const uint32_t j = n0s[nt] + r16;
            const float sw = KIND == 0 ? S.s[sg[nt]][jrow[nt]] : 1.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t m = mt * 16 + 4 * g + i;
                if (m < rows) {
                    const float y = KIND == 0 ? v[i] * sa[m] * sw : v[i];
                    out[(size_t)m * ldc + j] = bf16_rne(y);
                }
            }
        }
    }
}

// launch for rows <= 32
template <int MT, int NT, int W, int U, bool BAL = false>
void skinny_launch(w8a8_scale_t kind, const uint8_t *q, const float *a_scales, uint32_t rows, uint32_t k,
                   const Segs &S, uint16_t *out, uint32_t ldc, hipStream_t s) {
    const unsigned grid = col_grid<NT, BAL>(S.ntotal);
    if (kind == W8A8_ROWSCALE)
        w8a8_skinny<MT, NT, W, U, 0, BAL><<<grid, W * kWave, 0, s>>>(q, a_scales, rows, k, S, out, ldc);
    else
        w8a8_skinny<MT, NT, W, U, 1, BAL><<<grid, W * kWave, 0, s>>>(q, a_scales, rows, k, S, out, ldc);
}

// --------------------------------------------------------- fused proj ---
//
// rows <= kFusedRows: w8a8_proj in one launch.  The skinny GEMV above, with
// each workgroup quantizing the activations it needs itself: it reads the
// bf16 rows (from L2 after the first touch), computes the scales and codes
// with the same arithmetic as the stand-alone quantizer, and hands the codes
// to the MFMAs through a per-wave LDS area.  Workgroup 0 also writes codes
// and scales to the caller's scratch, as the two-launch form does.  K split,
// operand layout and accumulation order are those of w8a8_skinny<1, NT, 4,
// U>, so the output equals that of act_quant + gemv bit for bit.
//
// Per wave and chunk of U K blocks: activation loads first, then the weight
// loads, so the in-order load counter lets the encoding run while the weights
// are still in flight.  Per-row scales need the whole row's absmax, i.e. a
// workgroup barrier after every wave has its part; the host keeps per-row
// calls to one chunk per wave (K <= W * U * 128), where that barrier sits
// between the first loads and the first MFMAs.  Block scales are local to
// one 128-column group (a 16-lane team) and any K works.
constexpr uint32_t kFusedRows = 8;

// R: activation rows the kernel is built for (rows <= R); W waves split K.
template <int NT, int R, int W, int U, int KIND, bool SILU, bool UP, bool BAL>
__global__ __launch_bounds__(W * kWave) void w8a8_fused(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ up, uint32_t ldx, uint32_t rows, uint32_t K, Segs S,
    uint16_t *__restrict__ out, uint32_t ldc, uint8_t *__restrict__ qout, float *__restrict__ saout) {
    constexpr int XJ = U / 4;          // 16-byte activation loads per row per chunk (64 lanes x 8 values)
    constexpr int RS = U * 128 + 16;   // byte stride of a staged code row (padded against bank conflicts)
    static_assert(U % 4 == 0, "a chunk is a whole number of 4-block wave loads");
    __shared__ __attribute__((aligned(16))) uint8_t lq[W][R][RS];
    __shared__ float lgs[W][R][U];
    __shared__ float lamax[W][R];
    __shared__ float ls[R], ly[R];
    __shared__ f32x4 red[W][NT][kWave];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const uint32_t nkb = K / 128;
    const uint32_t kb0 = wv * nkb / W, kb1 = (wv + 1) * nkb / W;
    const bool writer = blockIdx.x == 0;

    // weights through buffer resources (one per column tile; a tile lies in
    // one segment), activations through one over the rows used
    int sg[NT];
    uint32_t jloc0[NT], jrow[NT], woff[NT], n0s[NT];
    bool jok[NT];
    rsrc_t rw[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        uint32_t tile, rlo, rhi;
        col_tile<NT, BAL>(nt, tile, rlo, rhi);
        const uint32_t n0 = tile * 16u;
        n0s[nt] = n0;
        const uint32_t nn = n0 < S.ntotal ? n0 : 0;
        sg[nt] = seg_of(S, nn);
        jloc0[nt] = nn - pick(sg[nt], S.start[0], S.start[1], S.start[2]);
        jrow[nt] = jloc0[nt] + r16;
        const uint32_t segn = pick(sg[nt], S.n[0], S.n[1], S.n[2]);
        jok[nt] = n0 < S.ntotal && jrow[nt] < segn && (uint32_t)r16 >= rlo && (uint32_t)r16 < rhi;
        rw[nt] = make_rsrc(pick(sg[nt], S.w[0], S.w[1], S.w[2]), segn * K);
        woff[nt] = jok[nt] ? jrow[nt] * K + g * 16 : kOffNone;
    }
    const uint32_t xbytes = ((rows - 1) * ldx + K) * 2;
    const rsrc_t rx = make_rsrc(x, xbytes);
    const rsrc_t ru = make_rsrc(UP ? up : x, xbytes);
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const i32x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

    // lane's 8 activation values of load j: block 4j + g of the chunk,
    // columns 8*r16 .. +7; rows >= rows and blocks past the chunk read zeros
    u32x4 xw[R][XJ], xu[R][XJ];
    i32x8 b[U][NT];
    auto load_chunk = [&](uint32_t kbc, uint32_t nb) {
#pragma unroll
        for (int m = 0; m < R; ++m) {
#pragma unroll
            for (int j = 0; j < XJ; ++j) {
                const bool ok = (uint32_t)m < rows && (uint32_t)(4 * j + g) < nb;
                const uint32_t off = ok ? (m * ldx + kbc * 128 + j * 512 + lane * 8) * 2 : kOffNone;
                xw[m][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
                if (UP) xu[m][j] = __builtin_amdgcn_raw_buffer_load_b128(ru, off, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const uint32_t off = (uint32_t)u < nb ? woff[nt] + (kbc + u) * 128 : kOffNone;
                const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rw[nt], off, 0, kAuxNt);
                const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(rw[nt], off, 64, kAuxNt);
                b[u][nt] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
        }
        // issue every load before any use: the first wait on an activation
        // must not hold back the weight loads behind it
        __builtin_amdgcn_sched_barrier(0);
    };

    // (an empty slice loads nothing and leaves zeros)
    load_chunk(kb0, kb1 - kb0 < (uint32_t)U ? kb1 - kb0 : (uint32_t)U);

    if (KIND == 0) {
        // row absmax: this wave's part, then across the waves (one chunk per wave)
        float am[R];
#pragma unroll
        for (int m = 0; m < R; ++m) {
            am[m] = 0.0f;
#pragma unroll
            for (int j = 0; j < XJ; ++j) {
                float v[8];
                act8<SILU, UP>(xw[m][j], xu[m][j], v);
                am[m] = fmaxf(am[m], absmax8(v));
            }
        }
#pragma unroll
        for (int m = 0; m < R; ++m) am[m] = team_absmax<kWave>(am[m]);
        if (lane == 0) {
#pragma unroll
            for (int m = 0; m < R; ++m) lamax[wv][m] = am[m];
        }
        // barriers over LDS only: the weight loads stay in flight
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (threadIdx.x < R) {
            float am = lamax[0][threadIdx.x];
#pragma unroll
            for (int w = 1; w < W; ++w) am = fmaxf(am, lamax[w][threadIdx.x]);
            const float s = act_scale(am);
            ls[threadIdx.x] = s;
            ly[threadIdx.x] = 1.0f / s;
            if (writer && threadIdx.x < rows) saout[threadIdx.x] = s;
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    for (uint32_t kbc = kb0; kbc < kb1; kbc += U) {
        const uint32_t nb = kb1 - kbc < (uint32_t)U ? kb1 - kbc : (uint32_t)U;
        if (kbc != kb0) load_chunk(kbc, nb);
        // codes (and block scales) of the chunk -> this wave's LDS rows
#pragma unroll
        for (int m = 0; m < R; ++m) {
            if ((uint32_t)m >= rows) break;
            const float srow = KIND == 0 ? ls[m] : 0.0f;
            const float yrow = KIND == 0 ? ly[m] : 0.0f;
#pragma unroll
            for (int j = 0; j < XJ; ++j) {
                const uint32_t blk = 4 * j + g;
                const bool ok = blk < nb;
                float v[8];
                act8<SILU, UP>(xw[m][j], xu[m][j], v);
                const float s = KIND == 0 ? srow : act_scale(team_absmax<16>(absmax8(v)));
                const float y = KIND == 0 ? yrow : 1.0f / s;
                const u32x2 c = encode8(v, s, y);
                if (ok) {
                    *reinterpret_cast<u32x2 *>(&lq[wv][m][blk * 128 + r16 * 8]) = c;
                    if (KIND == 1 && r16 == 0) lgs[wv][m][blk] = s;
                    if (writer) {
                        *reinterpret_cast<u32x2 *>(qout + (size_t)m * K + (size_t)(kbc + blk) * 128 + r16 * 8) = c;
                        if (KIND == 1 && r16 == 0) saout[(size_t)m * nkb + kbc + blk] = s;
                    }
                }
            }
        }
        // the LDS writes above were made by other lanes of this wave; a wave's
        // LDS operations complete in order, so only code motion must be stopped
        asm volatile("" ::: "memory");
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if ((uint32_t)u >= nb) break;
            i32x8 a = zero8;
            if ((uint32_t)r16 < rows) {
                const u32x4 lo = *reinterpret_cast<const u32x4 *>(&lq[wv][r16][u * 128 + g * 16]);
                const u32x4 hi = *reinterpret_cast<const u32x4 *>(&lq[wv][r16][u * 128 + 64 + g * 16]);
                a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
                a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (KIND == 0) {
                    acc[nt] = mfma_fp8(a, b[u][nt], acc[nt]);
                } else {
                    const f32x4 p = mfma_fp8(a, b[u][nt], f32x4{0.f, 0.f, 0.f, 0.f});
                    const float swb = S.s[sg[nt]][(size_t)(jloc0[nt] / 128) * nkb + kbc + u];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t m = 4 * g + i;
                        const float sab = m < rows ? lgs[wv][m][u] : 0.0f;
                        acc[nt][i] = __builtin_fmaf(p[i], sab * swb, acc[nt][i]);
                    }
                }
            }
        }
        // the next chunk overwrites this wave's LDS rows
        asm volatile("" ::: "memory");
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[wv][nt][lane] = acc[nt];
    __syncthreads();
    for (int nt = wv; nt < NT; nt += W) {
        f32x4 v = red[0][nt][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += red[w][nt][lane];
        if (jok[nt]) {
            const uint32_t j = n0s[nt] + r16;
            const float sw = KIND == 0 ? S.s[sg[nt]][jrow[nt]] : 1.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t m = 4 * g + i;
                if (m < rows) {
                    const float y = KIND == 0 ? v[i] * ls[m] * sw : v[i];
                    out[(size_t)m * ldc + j] = bf16_rne(y);
                }
            }
        }
    }
}

// Shapes {NT, W, U} shared by the skinny GEMV and the fused projection for
// the same row counts (same K split, so both forms give the same bits): up
// to 8 rows, two column tiles per workgroup in the balanced pairing, 8 K
// slices of 4 blocks (more waves to hide the loads, and half of each wave's
// share of the activation encoding compared with 4 slices of 8).
// W * U is kFusedMaxBlocksRow: with per-row scales K may have that many
// 128-blocks (one chunk per wave).
constexpr uint32_t kFusedMaxBlocksRow = 32;

// Whether w8a8_proj runs as one launch (see the fused kernel's comment).
bool fused_ok(w8a8_scale_t kind, uint32_t rows, uint32_t k, uint32_t ldx) {
    return rows <= kFusedRows && (kind == W8A8_BLK128 || k / 128 <= kFusedMaxBlocksRow) &&
           ((uint64_t)(rows - 1) * ldx + k) * 2 < 0x80000000ull;
}

template <int NT, int R, int W, int U, bool BAL, int KIND, bool SILU, bool UP>
void fused_launch3(const uint16_t *x, const uint16_t *up, uint32_t ldx, uint32_t rows, uint32_t k, const Segs &S,
                   uint16_t *out, uint32_t ldc, uint8_t *q, float *a_scales, hipStream_t s) {
    static_assert(W * U == (int)kFusedMaxBlocksRow, "per-row scales: one chunk per wave");
    w8a8_fused<NT, R, W, U, KIND, SILU, UP, BAL><<<col_grid<NT, BAL>(S.ntotal), W * kWave, 0, s>>>(
        x, up, ldx, rows, k, S, out, ldc, q, a_scales);
}

template <int NT, int R, int W, int U, bool BAL>
void fused_launch(w8a8_scale_t kind, int silu, const uint16_t *x, const uint16_t *up, uint32_t ldx, uint32_t rows,
                  uint32_t k, const Segs &S, uint16_t *out, uint32_t ldc, uint8_t *q, float *a_scales,
                  hipStream_t s) {
#define KVQ_FUSED(KIND)                                                                                        \
    do {                                                                                                       \
        if (!silu)                                                                                             \
            fused_launch3<NT, R, W, U, BAL, KIND, false, false>(x, up, ldx, rows, k, S, out, ldc, q, a_scales, s); \
        else if (!up)                                                                                          \
            fused_launch3<NT, R, W, U, BAL, KIND, true, false>(x, up, ldx, rows, k, S, out, ldc, q, a_scales, s);  \
        else                                                                                                   \
            fused_launch3<NT, R, W, U, BAL, KIND, true, true>(x, up, ldx, rows, k, S, out, ldc, q, a_scales, s);   \
    } while (0)
    if (kind == W8A8_ROWSCALE) KVQ_FUSED(0);
    else KVQ_FUSED(1);
#undef KVQ_FUSED
}

// --------------------------------------------------------------- wide ---
//
// rows > 32: one workgroup owns all (<= 256) activation rows and 128 output
// columns over one slice of K (split-K), so the weight tile is read from HBM
// once per call and the activation tile (re-read by every column tile) comes
// from L2.  8 multiplying waves in a 4 (rows) x 2 (64 columns) grid, two per
// SIMD, so one wave's scaling arithmetic overlaps the other's matrix
// instructions, and 4 loader waves: two stream the activation tile (and its
// block scales), two the weight tile, each into its own LDS ring with direct
// DMA loads (lane i's 16 bytes land at LDS base + 16*i).  The activation ring
// has 3-4 stages (its tiles come from L2), the weight ring what LDS leaves,
// up to a cap of 4-8 by tile size (its tiles come from HBM with the longer
// latency, but more weight loads in flight slow the CU's L2 hits).  A loader waits for
// its own loads of the next K step (vmcnt), then every wave meets at one
// barrier per K step; a multiplying wave reads the next activation fragment
// before the matrix instructions of the current one.  Rows are stored with
// their eight 16-byte chunks XOR-swizzled by (row & 7), which keeps both the
// load pattern and the MFMA operand reads (ds_read_b128) free of bank
// conflicts.  The loads are buffer loads from wave-uniform bases (the
// per-lane offsets never change; rows past the end of the activations or of
// a weight segment read as zero); a 128-column tile that straddles two weight
// segments (possible only with per-row scales) uses per-lane global addresses
// instead.  With split-K the fp32 partial tiles go to the workspace and
// w8a8_reduce adds them in split order (deterministic), applies per-row
// scales and writes bf16.

constexpr int kWideN = 128;
constexpr int kWideWM = 4;                                 // multiplying waves along rows (x 2 along columns)
constexpr int kWideWaves = 2 * kWideWM;                    // waves that multiply
constexpr int kWideMaxMTW = 256 / (16 * kWideWM);         // 16-row tiles per wave at 256 rows
constexpr int kWideLoaders = 4;                            // waves that only load (2 per stream)
constexpr int kWideThreads = (kWideWaves + kWideLoaders) * kWave;


template <int MTW, int KIND, bool SX4>
struct WideCfg {
    static constexpr int WM = kWideWM;                   // multiplying waves along rows
    static constexpr int BM = 16 * MTW * WM;             // rows per workgroup
    static constexpr int A_BYTES = BM * 128;
    static constexpr int B_BYTES = kWideN * 128;
    // Producer / consumer: waves 0-7 only read LDS and multiply; waves 8-9
    // load the activation tiles (and block scales), waves 10-11 the weight
    // tiles.  A wave that issues a load waits while the address unit's queue
    // is full, and in-order issue then holds back its matrix instructions
    // too; loader waves take that wait instead.  Each loader's vector-memory
    // counter tracks one stream, so the weight ring can run further ahead
    // than the activation ring (a wave can only wait for its loads in issue
    // order).
    static constexpr int LW = kWideLoaders / 2;                   // loader waves per stream
    static constexpr int A_INSTR = A_BYTES / 1024 / LW;           // 1 KiB loads per A loader per stage
    static constexpr int B_INSTR = B_BYTES / 1024 / LW;           // per B loader per stage
    static constexpr int SA_ROWS = BM / LW;                       // activation-scale rows per A loader
    // scale loads per A loader per chunk: SX4 one 16-byte load per row (a
    // row's 4 scales), else one 4-byte load per scale.  The vector L1 takes
    // a direct-to-LDS instruction at a time per wave whatever its width, so
    // the 16-byte form issues a quarter of the instructions.
    static constexpr int SC_INSTR = SX4 ? (SA_ROWS + 63) / 64 : (SA_ROWS * 4 + 63) / 64;
    static constexpr int SC_BYTES = (BM + 1) * 16;                // one chunk: [BM rows + sw][4 K blocks]
    // Ring depths: the activation tiles come from L2 (every column tile
    // reads them), the weight tiles from HBM with its longer latency; the
    // weight ring takes what LDS is left, up to a cap.  Weight loads in
    // flight beyond what keeps the CU's share of HBM busy only slow the
    // activation loads (L2 hits) of the same CU, so the small tiles keep
    // fewer weight stages and more activation stages (measured per tile
    // size).  The double-buffered scale chunks are refilled 8 K blocks
    // apart, so SA <= 5.
    static constexpr int SA = MTW <= 2 ? 4 : 3;
    static constexpr int SB_CAP = MTW == 1 ? 4 : (MTW == 2 ? 6 : 8);
    static constexpr int LDS_MAX = 160 * 1024 - 2 * SC_BYTES - 1024;
    static constexpr int SB_FIT = (LDS_MAX - SA * A_BYTES) / B_BYTES;
    static constexpr int SB = SB_FIT > SB_CAP ? SB_CAP : SB_FIT;
    static_assert(A_INSTR >= 1 && B_INSTR >= 1 && SA_ROWS % 8 == 0, "tile shape");
    static_assert(SB >= 3 && SA <= 5, "ring depths");
    static_assert((SB - 2) * B_INSTR + 15 < 64 && (SA - 2) * (A_INSTR + SC_INSTR + 1) + 15 < 64, "vmcnt range");
    static_assert(SC_INSTR + 1 <= 15, "scale loads per chunk");
};

// s_waitcnt vmcnt(base + extra) for a run-time extra in [0, 15] (larger
// extras wait for more loads than needed: slower, never wrong)
template <int BASE>
__device__ __forceinline__ void wait_vm_plus(uint32_t extra) {
    switch (extra) {
        case 0: wait_vm<BASE>(); break;
        case 1: wait_vm<BASE + 1>(); break;
        case 2: wait_vm<BASE + 2>(); break;
        case 3: wait_vm<BASE + 3>(); break;
        case 4: wait_vm<BASE + 4>(); break;
        case 5: wait_vm<BASE + 5>(); break;
        case 6: wait_vm<BASE + 6>(); break;
        case 7: wait_vm<BASE + 7>(); break;
        case 8: wait_vm<BASE + 8>(); break;
        case 9: wait_vm<BASE + 9>(); break;
        case 10: wait_vm<BASE + 10>(); break;
        case 11: wait_vm<BASE + 11>(); break;
        case 12: wait_vm<BASE + 12>(); break;
        case 13: wait_vm<BASE + 13>(); break;
        case 14: wait_vm<BASE + 14>(); break;
        default: wait_vm<BASE + 15>(); break;
    }
}

// wait until at most `later` stages of N loads (plus `extra`) are in flight
template <int N, int MAXL>
__device__ __forceinline__ void wait_stages(int later, uint32_t extra) {
    if constexpr (MAXL >= 6) {
        if (later == 6) { wait_vm_plus<6 * N>(extra); return; }
    }
    if constexpr (MAXL >= 5) {
        if (later == 5) { wait_vm_plus<5 * N>(extra); return; }
    }
    if constexpr (MAXL >= 4) {
        if (later == 4) { wait_vm_plus<4 * N>(extra); return; }
    }
    if constexpr (MAXL >= 3) {
        if (later == 3) { wait_vm_plus<3 * N>(extra); return; }
    }
    if constexpr (MAXL >= 2) {
        if (later == 2) { wait_vm_plus<2 * N>(extra); return; }
    }
    if (later == 1) { wait_vm_plus<N>(extra); return; }
    wait_vm_plus<0>(extra);
}


template <int MTW, int KIND, bool UNI, bool SX4>
__global__ __launch_bounds__(kWideThreads) void w8a8_wide(const uint8_t *__restrict__ q, const float *__restrict__ sa,
                                                          uint32_t rows, uint32_t K, Segs S,
                                                          uint16_t *__restrict__ out, uint32_t ldc, uint32_t splits,
                                                          uint32_t ntiles, float *__restrict__ partials) {
    using C = WideCfg<MTW, KIND, SX4>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_a[C::SA * C::A_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_b[C::SB * C::B_BYTES];
    // block scales (KIND 1), double-buffered in chunks of 4 K blocks
    __shared__ __attribute__((aligned(16))) float lds_sc[KIND == 1 ? 2 : 1][KIND == 1 ? C::SC_BYTES / 4 : 4];
    const int lane = lane_id();
    const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wv >> 1, wn = wv & 1;
    const int r16 = lane & 15, g = lane >> 4;
    // wave-uniform roles: multiply (0-7), load activations (8-9), load weights (10-11)
    const bool mul_wave = wv < (uint32_t)kWideWaves;
    const bool a_wave = !mul_wave && wv < (uint32_t)(kWideWaves + C::LW);
    const bool b_wave = !mul_wave && !a_wave;
    const uint32_t lw = a_wave ? wv - kWideWaves : (b_wave ? wv - kWideWaves - C::LW : 0);
    // consecutive workgroups take the K slices of one column tile: with the
    // usual round-robin dispatch over the 8 XCDs each XCD then works on few
    // K slices, so fewer copies of the activation tile sit in its L2
    const uint32_t split = blockIdx.x % splits, tile = blockIdx.x / splits;
    const uint32_t n0 = tile * kWideN;
    const uint32_t nkb = K / 128;
    const uint32_t kb0 = (uint32_t)((uint64_t)split * nkb / splits);
    const uint32_t kb1 = (uint32_t)((uint64_t)(split + 1) * nkb / splits);
    const int nks = (int)(kb1 - kb0);

    const int sg0 = seg_of(S, n0);
    const uint32_t seg_start = sg0 == 0 ? S.start[0] : (sg0 == 1 ? S.start[1] : S.start[2]);

    if (!mul_wave) {
        // ------------------------------------------------------ loaders --
        // Load j of loader wave w fills 1 KiB of its tile: rows
        // 8*(w*INSTR + j) .. +8; lane i writes LDS chunk slot i%8 of row
        // (that + i/8), which holds logical chunk (i%8) ^ (row & 7).
        const uint32_t a0 = __builtin_amdgcn_readfirstlane(lds_offset(lds_a));
        const uint32_t b0 = __builtin_amdgcn_readfirstlane(lds_offset(lds_b));
        const uint32_t sc0 = __builtin_amdgcn_readfirstlane(lds_offset(&lds_sc[0][0]));
        // number of scale loads an A loader adds to activation stage it
        auto sc_count = [&](int it) -> uint32_t {
            if (KIND != 1 || it >= nks || (it != 0 && ((kb0 + it) & 3) != 0)) return 0;
            return C::SC_INSTR + (lw == 0 ? 1 : 0);
        };
        if (a_wave) {
            const u32x4 ra = buffer_rsrc(q, rows * K);
            uint32_t aoff[C::A_INSTR];
#pragma unroll
            for (int j = 0; j < C::A_INSTR; ++j) {
                const uint32_t row = 8 * (lw * C::A_INSTR + j) + (lane >> 3);
                aoff[j] = row * K + (((lane & 7) ^ (row & 7)) << 4);   // rows >= `rows` read zeros
            }
            // Block scales travel in chunks of 4 K blocks (kb = 4c .. 4c+3),
            // loaded with the first activation stage that needs them: lane i
            // of load j of A loader w takes sa[row][4c + i%4] for row
            // w*SA_ROWS + 16j + i/4 (rows past the end and K blocks past the
            // array read zero), so a chunk holds [row][4] floats; A loader 0
            // also loads sw[band][4c .. 4c+3] of this 128-column band behind
            // the rows.  Scales are re-read from HBM once per 4 K blocks, not
            // per stage: a per-row 4-byte read touches a whole cache line.
            const u32x4 rsa = buffer_rsrc(sa, KIND == 1 ? rows * nkb * 4 : 4);
            u32x4 rsw = rsa;
            if (KIND == 1) {
                const float *sseg = sg0 == 0 ? S.s[0] : (sg0 == 1 ? S.s[1] : S.s[2]);
                rsw = buffer_rsrc(sseg + (size_t)((n0 - seg_start) / 128) * nkb, nkb * 4);
            }
            uint32_t scoff[C::SC_INSTR];
#pragma unroll
            for (int j = 0; j < C::SC_INSTR; ++j)
                scoff[j] = SX4 ? (lw * C::SA_ROWS + 64 * j + lane) * nkb * 4
                               : ((lw * C::SA_ROWS + 16 * j + (lane >> 2)) * nkb + (lane & 3)) * 4;
            auto issue_a = [&](int it) {
                const uint32_t kb = kb0 + it;
                const uint32_t abase = a0 + (uint32_t)(it % C::SA) * C::A_BYTES;
                const uint32_t soff = __builtin_amdgcn_readfirstlane(kb * 128);
#pragma unroll
                for (int j = 0; j < C::A_INSTR; ++j)
                    lds_buf16(ra, aoff[j], soff, abase + (lw * C::A_INSTR + j) * 1024);
                if (sc_count(it)) {
                    // the chunk offset goes into the per-lane offset, which the
                    // buffer range check covers
                    const uint32_t c4 = (kb & ~3u) * 4;
                    const uint32_t slot = sc0 + ((kb >> 2) & 1) * C::SC_BYTES;
#pragma unroll
                    for (int j = 0; j < C::SC_INSTR; ++j) {
                        if (SX4) {
                            // lane i: row lw*SA_ROWS + 64j + i, its 4 scales
                            // (16-byte aligned: nkb is a multiple of 4)
                            const uint32_t dst = slot + (lw * C::SA_ROWS + 64 * j) * 16;
                            if (64 * j + lane < C::SA_ROWS) lds_buf16(rsa, scoff[j] + c4, 0, dst);
                        } else {
                            const uint32_t dst = slot + (lw * C::SA_ROWS + 16 * j) * 16;
                            if (16 * j + (lane >> 2) < C::SA_ROWS) lds_buf4(rsa, scoff[j] + c4, 0, dst);
                        }
                    }
                    if (lw == 0 && lane < 4) lds_buf4(rsw, lane * 4 + c4, 0, slot + C::BM * 16);
                }
            };
            // this wave's loads of K step `next` complete; later steps may stay in flight
            auto wait_a = [&](int next) {
                if (next >= nks) return;
                int later = nks - 1 - next;
                if (later > C::SA - 2) later = C::SA - 2;
                uint32_t extra = 0;
                for (int j = 1; j <= later; ++j) extra += sc_count(next + j);
                wait_stages<C::A_INSTR, C::SA - 2>(later, extra);
            };
            for (int i = 0; i < C::SA - 1 && i < nks; ++i) issue_a(i);
            wait_a(0);
            asm volatile("s_barrier" ::: "memory");
            for (int it = 0; it < nks; ++it) {
                if (it + C::SA - 1 < nks) issue_a(it + C::SA - 1);
                wait_a(it + 1);
                asm volatile("s_barrier" ::: "memory");
            }
        } else {
            const uint8_t *wseg = sg0 == 0 ? S.w[0] : (sg0 == 1 ? S.w[1] : S.w[2]);
            const uint32_t seg_n = sg0 == 0 ? S.n[0] : (sg0 == 1 ? S.n[1] : S.n[2]);
            const u32x4 rb = buffer_rsrc(wseg, seg_n * K);
            uint32_t boff[C::B_INSTR];
            const uint8_t *bsrc[C::B_INSTR];
#pragma unroll
            for (int j = 0; j < C::B_INSTR; ++j) {
                const uint32_t row = 8 * (lw * C::B_INSTR + j) + (lane >> 3);
                const uint32_t chunk = ((lane & 7) ^ (row & 7)) << 4;
                boff[j] = (n0 - seg_start + row) * K + chunk;          // past the segment: zeros
                if (!UNI) {
                    uint32_t jg = n0 + row;
                    int sg = seg_of(S, jg < S.ntotal ? jg : 0);
                    uint32_t jl = (jg < S.ntotal ? jg : 0) - S.start[sg];
                    if (jl >= S.n[sg]) { sg = 0; jl = 0; }           // past the end: any valid row
                    bsrc[j] = S.w[sg] + (size_t)jl * K + chunk;
                }
            }
            auto issue_b = [&](int it) {
                const uint32_t kb = kb0 + it;
                const uint32_t bbase = b0 + (uint32_t)(it % C::SB) * C::B_BYTES;
                const uint32_t soff = __builtin_amdgcn_readfirstlane(kb * 128);
#pragma unroll
                for (int j = 0; j < C::B_INSTR; ++j) {
                    if (UNI) lds_buf16(rb, boff[j], soff, bbase + (lw * C::B_INSTR + j) * 1024);
                    else lds_glb16(bsrc[j] + (size_t)kb * 128, bbase + (lw * C::B_INSTR + j) * 1024);
                }
            };
            auto wait_b = [&](int next) {
                if (next >= nks) return;
                int later = nks - 1 - next;
                if (later > C::SB - 2) later = C::SB - 2;
                wait_stages<C::B_INSTR, C::SB - 2>(later, 0);
            };
            for (int i = 0; i < C::SB - 1 && i < nks; ++i) issue_b(i);
            wait_b(0);
            asm volatile("s_barrier" ::: "memory");
            for (int it = 0; it < nks; ++it) {
                if (it + C::SB - 1 < nks) issue_b(it + C::SB - 1);
                wait_b(it + 1);
                asm volatile("s_barrier" ::: "memory");
            }
        }
        return;
    }

    // ------------------------------------------------------- multiply ---
    // Step it reads the slots of step it: filled before the barrier that
    // ended step it-1 (its loaders waited for them), and refilled only after
    // the barrier that ends step it.  lgkmcnt(0) before each barrier makes
    // this wave's LDS reads of the step complete first.  The asm barrier
    // keeps LDS accesses on their side of it.
    f32x4 acc[MTW][4];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    asm volatile("s_barrier" ::: "memory");
    for (int it = 0; it < nks; ++it) {
        const uint32_t kbi = kb0 + it;
        const float *scs = &lds_sc[KIND == 1 ? (kbi >> 2) & 1 : 0][kbi & 3];   // [row * 4] of this K block
        const uint8_t *abase = lds_a + (it % C::SA) * C::A_BYTES;
        const uint8_t *bbase = lds_b + (it % C::SB) * C::B_BYTES;
        // operand fragments: the weight fragments of the step and the first
        // activation fragment are read together; activation fragment mt+1
        // is read before the matrix instructions of fragment mt, so its LDS
        // latency runs under them instead of between the groups
        auto frag = [&](const uint8_t *base, int row) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + row * 128 + ((g ^ (row & 7)) << 4));
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + row * 128 + (((g + 4) ^ (row & 7)) << 4));
            return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        };
        auto scales = [&](int mt) {
            // rows 4g..4g+3 of this M tile, times the weight block scale
            const int r0 = wm * 16 * MTW + mt * 16 + 4 * g;
            const float swk = scs[C::BM * 4];
            return f32x4{scs[r0 * 4], scs[r0 * 4 + 4], scs[r0 * 4 + 8], scs[r0 * 4 + 12]} * swk;
        };
        i32x8 b[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) b[nt] = frag(bbase, wn * 64 + nt * 16 + r16);
        i32x8 a_cur = frag(abase, wm * 16 * MTW + r16);
        f32x4 sc_cur = KIND == 1 ? scales(0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) {
            i32x8 a_next = a_cur;
            f32x4 sc_next = sc_cur;
            if (mt + 1 < MTW) {
                a_next = frag(abase, wm * 16 * MTW + (mt + 1) * 16 + r16);
                if (KIND == 1) sc_next = scales(mt + 1);
            }
            if (KIND == 0) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_fp8(a_cur, b[nt], acc[mt][nt]);
            } else {
                f32x4 p[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) p[nt] = mfma_fp8(a_cur, b[nt], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[mt][nt][e] = __builtin_fmaf(p[nt][e], sc_cur[e], acc[mt][nt][e]);
            }
            a_cur = a_next;
            sc_cur = sc_next;
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }


    // ---- epilogue: bf16 output (no split), or the fp32 partial tile in the
    // accumulators' own layout: per (tile, split) [wm][mt][wn][nt][lane] of
    // f32x4 (lane (r16, g) holds column r16 of its 16x16 block and rows
    // 4g..4g+3), so every wave writes whole 1 KiB blocks with 16-byte stores.
    // Rows past `rows` and columns past the weights hold zero sums.
    if (splits > 1) {
        f32x4 *part = reinterpret_cast<f32x4 *>(partials) + (size_t)blockIdx.x * (kWideWM * MTW * 2 * 4 * kWave);
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                part[(((wm * MTW + mt) * 2 + wn) * 4 + nt) * kWave + lane] = acc[mt][nt];
        return;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const uint32_t col = n0 + wn * 64 + nt * 16 + r16;
        if (col >= S.ntotal) continue;
        const int sg = seg_of(S, col);
        const uint32_t jl = col - S.start[sg];
        if (jl >= S.n[sg]) continue;
        const float sw = KIND == 0 ? S.s[sg][jl] : 1.0f;
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t m = wm * 16 * MTW + mt * 16 + 4 * g + e;
                if (m >= rows) continue;
                const float y = KIND == 0 ? acc[mt][nt][e] * sa[m] * sw : acc[mt][nt][e];
                out[(size_t)m * ldc + col] = bf16_rne(y);
            }
        }
    }
}

// Sum the split-K partial tiles in split order (deterministic), scale (per-row
// kind), round to bf16.  One workgroup per (column tile, wave block
// (wm, mt, wn)): thread (nt, lane) adds the splits' f32x4 at its place of the
// partial layout (up to 8 loads in flight) and writes rows 4g..4g+3 of column
// r16 of block nt.
template <int KIND, int MTW>
__global__ __launch_bounds__(256) void w8a8_reduce(const f32x4 *__restrict__ partials, uint32_t splits,
                                                   const float *__restrict__ sa, uint32_t rows, Segs S,
                                                   uint16_t *__restrict__ out, uint32_t ldc) {
    constexpr int UNITS = kWideWM * MTW * 2;
    const uint32_t tile = blockIdx.x / UNITS, u = blockIdx.x % UNITS;
    const int wm = u / (MTW * 2), mt = (u / 2) % MTW, wn = u % 2;
    const int nt = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const size_t per_split = (size_t)UNITS * 4 * kWave;
    const f32x4 *p = partials + (size_t)tile * splits * per_split + ((size_t)u * 4 + nt) * kWave + lane;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (uint32_t s0 = 0; s0 < splits; s0 += 8) {
        f32x4 t[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (s0 + q < splits) t[q] = __builtin_nontemporal_load(p + (size_t)(s0 + q) * per_split);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (s0 + q < splits) v += t[q];
    }
    const uint32_t col = tile * kWideN + wn * 64 + nt * 16 + r16;
    if (col >= S.ntotal) return;
    const int sg = seg_of(S, col);
    const uint32_t jl = col - S.start[sg];
    if (jl >= S.n[sg]) return;
    const float sw = KIND == 0 ? S.s[sg][jl] : 1.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t m = wm * 16 * MTW + mt * 16 + 4 * g + e;
        if (m < rows) out[(size_t)m * ldc + col] = bf16_rne(KIND == 0 ? v[e] * sa[m] * sw : v[e]);
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
        if ((uint64_t)segs[i].n * k >= 0x80000000ull)
            return fail(KVQ_E_INVALID, "%s: segment %u is larger than 2 GiB", fn, i);
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
    if ((uint64_t)rows * k >= 0x80000000ull) return fail(KVQ_E_INVALID, "%s: activation block is larger than 2 GiB", fn);
    if (!q || !a_scales || !out) return fail(KVQ_E_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(q) || !aligned16(a_scales) || !aligned16(out))
        return fail(KVQ_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
    return KVQ_OK;
}

struct WidePlan {
    uint32_t mtw, ntiles, splits;
    size_t counter_bytes;    // the workspace's counter area, left untouched
    size_t ws_bytes;
};

// rows > 32: all rows per workgroup (MTW = ceil(rows/64) 16-row tiles per
// wave, 4 waves along rows), 128-column tiles, and enough K slices to give
// ~256 workgroups.
WidePlan wide_plan(uint32_t rows, uint32_t k, uint32_t ntotal) {
    WidePlan p;
    p.mtw = (rows + 16 * kWideWM - 1) / (16 * kWideWM);
    p.ntiles = (ntotal + kWideN - 1) / kWideN;
    const uint32_t nkb = k / 128;
    uint32_t sp = 256 / (p.ntiles ? p.ntiles : 1);
    if (sp > nkb) sp = nkb;
    if (sp < 1) sp = 1;
    p.splits = sp;
    p.counter_bytes = sp > 1 ? KVQ_WORKSPACE_COUNTER_BYTES : 0;   // partials go behind the counters
    // partial tiles: per (column tile, split) 4 x MTW x 2 x 4 blocks of 64 f32x4
    p.ws_bytes = sp > 1 ? p.counter_bytes + (size_t)p.ntiles * sp * (kWideWM * p.mtw * 2 * 4 * kWave) * 16 : 0;
    return p;
}

int gemv_launch(w8a8_scale_t kind, const uint8_t *q, const float *a_scales, uint32_t rows, uint32_t k, const Segs &S,
                uint16_t *out, uint32_t ldc, void *workspace, size_t workspace_bytes, hipStream_t s) {
    if (rows <= 32) {
        // {MT, NT, W, U}: up to 8 rows as the fused projection (see there); up
        // to 16 rows two column tiles per activation fragment (half the
        // activation re-reads), 4 K slices; 32 rows 8 K slices of 4 blocks
        if (rows <= 4) skinny_launch<1, 2, 8, 4, true>(kind, q, a_scales, rows, k, S, out, ldc, s);
        else if (rows <= 8) skinny_launch<1, 2, 8, 4, true>(kind, q, a_scales, rows, k, S, out, ldc, s);
        else if (rows <= 16) skinny_launch<1, 2, 4, 8, true>(kind, q, a_scales, rows, k, S, out, ldc, s);
        else skinny_launch<2, 2, 8, 4, true>(kind, q, a_scales, rows, k, S, out, ldc, s);
        return launch_status("w8a8_gemv");
    }
    WidePlan pl = wide_plan(rows, k, S.ntotal);
    float *partials = nullptr;
    if (pl.splits > 1) {
        if (workspace && workspace_bytes >= pl.ws_bytes && aligned16(workspace))
            partials = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pl.counter_bytes);
        else
            pl.splits = 1;
    }
    const unsigned grid = pl.ntiles * pl.splits;
    // tiles never straddle segments when every non-last segment is a multiple of 128 rows
    bool uni = true;
    for (uint32_t i = 0; i + 1 < S.count; ++i) uni = uni && (S.n[i] % kWideN == 0);
    // block-scale rows start 16-byte aligned when K is a multiple of 512
    const bool sx4 = (k / 128) % 4 == 0;
#define KVQ_WIDE3(MTW, KIND, UNI, SX4) \
    w8a8_wide<MTW, KIND, UNI, SX4><<<grid, kWideThreads, 0, s>>>(q, a_scales, rows, k, S, out, ldc, pl.splits, \
                                                                  pl.ntiles, partials)
#define KVQ_WIDE(MTW)                                                  \
    do {                                                               \
        if (kind == W8A8_BLK128 && sx4) KVQ_WIDE3(MTW, 1, true, true); \
        else if (kind == W8A8_BLK128) KVQ_WIDE3(MTW, 1, true, false);  \
        else if (uni) KVQ_WIDE3(MTW, 0, true, false);                  \
        else KVQ_WIDE3(MTW, 0, false, false);                          \
    } while (0)
    switch (pl.mtw) {
        case 1: KVQ_WIDE(1); break;
        case 2: KVQ_WIDE(2); break;
        case 3: KVQ_WIDE(3); break;
        case 4: KVQ_WIDE(4); break;
        default:
            if constexpr (kWideMaxMTW > 4) {
                switch (pl.mtw) {
                    case 5: KVQ_WIDE(5 < kWideMaxMTW ? 5 : kWideMaxMTW); break;
                    case 6: KVQ_WIDE(6 < kWideMaxMTW ? 6 : kWideMaxMTW); break;
                    case 7: KVQ_WIDE(7 < kWideMaxMTW ? 7 : kWideMaxMTW); break;
                    default: KVQ_WIDE(kWideMaxMTW); break;
                }
            }
            break;
    }
#undef KVQ_WIDE3
#undef KVQ_WIDE
    int st = launch_status("w8a8_gemv");
    if (st || pl.splits == 1) return st;
    const unsigned rgrid = pl.ntiles * (kWideWM * pl.mtw * 2);
    const f32x4 *pt = reinterpret_cast<const f32x4 *>(partials);
#define KVQ_RED(MTW)                                                                                          \
    do {                                                                                                      \
        if (kind == W8A8_ROWSCALE) w8a8_reduce<0, MTW><<<rgrid, 256, 0, s>>>(pt, pl.splits, a_scales, rows, S, out, ldc); \
        else w8a8_reduce<1, MTW><<<rgrid, 256, 0, s>>>(pt, pl.splits, a_scales, rows, S, out, ldc);           \
    } while (0)
    switch (pl.mtw) {
        case 1: KVQ_RED(1); break;
        case 2: KVQ_RED(2); break;
        case 3: KVQ_RED(3); break;
        case 4: KVQ_RED(4); break;
        default:
            if constexpr (kWideMaxMTW > 4) {
                switch (pl.mtw) {
                    case 5: KVQ_RED(5 < kWideMaxMTW ? 5 : kWideMaxMTW); break;
                    case 6: KVQ_RED(6 < kWideMaxMTW ? 6 : kWideMaxMTW); break;
                    case 7: KVQ_RED(7 < kWideMaxMTW ? 7 : kWideMaxMTW); break;
                    default: KVQ_RED(kWideMaxMTW); break;
                }
            }
            break;
    }
#undef KVQ_RED
    return launch_status("w8a8_gemv (split-K reduction)");
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
    Segs S;
    int st = check_gemv("w8a8_gemv", kind, q, a_scales, rows, k, segs, nseg, out, ldc, &S);
    if (st) return st;
    return gemv_launch(kind, q, a_scales, rows, k, S, out, ldc, workspace, workspace_bytes, as_stream(stream));
}

extern "C" int w8a8_gemv_workspace_bytes(w8a8_scale_t kind, uint32_t rows, uint32_t k, uint32_t n_total,
                                         size_t *bytes) {
    (void)kind;
    if (!bytes) return fail(KVQ_E_INVALID, "w8a8_gemv_workspace_bytes: null output pointer");
    *bytes = (rows > 32 && rows <= W8A8_MAX_ROWS && k >= 128) ? wide_plan(rows, k, n_total).ws_bytes : 0;
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
    if (fused_ok(kind, rows, k, ldx)) {
        // one launch: the GEMV quantizes the activations itself (and fills q, a_scales)
        if (rows <= 4)
            fused_launch<2, 4, 8, 4, true>(kind, silu, x, up, ldx, rows, k, S, out, ldc, q, a_scales, as_stream(stream));
        else
            fused_launch<2, 8, 8, 4, true>(kind, silu, x, up, ldx, rows, k, S, out, ldc, q, a_scales, as_stream(stream));
        return launch_status("w8a8_proj");
    }
    st = act_quant_launch(kind, silu, x, up, ldx, rows, k, q, a_scales, as_stream(stream));
    if (st) return st;
    return gemv_launch(kind, q, a_scales, rows, k, S, out, ldc, workspace, workspace_bytes, as_stream(stream));
}
