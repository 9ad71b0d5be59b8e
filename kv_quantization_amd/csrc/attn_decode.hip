// Decode attention over the quantized KV cache: one new token per query head.
//
// The pages define the cache (INT8 with one scale per token row, INT4 with a
// scale and zero per group) and its dequantization, not the attention that
// reads it; this is that consumer, textbook scaled-dot-product attention
// with grouped queries.  Query head h reads KV head h / G (G = Hq / Hkv
// consecutive query heads per KV head):
//
//   s_t = scale * (q_h . k_t)   k_t = code * k_scale[t]  (INT8)
//                               k_t = code * s - z * s   (INT4, per group)
//   p   = softmax(s)            (running max subtracted)
//   o_h = sum_t p_t v_t         v_t dequantized the same way
//
// The scales multiply the integer dot products (INT4: s * (sum q c - z sum
// q) per group) and the softmax weights (INT4: sum_t (p s) c - sum_t (p s
// z)); no dequantized copy of the cache is made, each cache byte is read once.
//
// Work: one workgroup per (KV head, chunk of tokens).  256 threads walk the
// chunk in blocks of 128 tokens with an online softmax (running max and
// sum; the partial output is rescaled when the max grows).  Per block:
//   1. scores: 8 lanes per token, each with 16 dims of the key row (one
//      16-byte load) and the same 16 dims of the G query rows in registers;
//      the 8 partial dot products are summed with DPP lane moves (all 8
//      lanes end with the same bits) and go to LDS;
//   2. softmax: per head the block max and sum over 128 tokens (two waves,
//      DPP then LDS), the new running max and rescale factor, and
//      p * v_scale to LDS;
//   3. values: thread (group of 16 tokens, 4 dims) adds p * v_scale * code
//      over its tokens into registers (4-byte loads of value codes, issued
//      with the key loads when the block starts).
// At the end the 8 token groups are added in LDS in a fixed order.  With
// several chunks per head, each workgroup writes (output, max, sum) of its
// chunk behind the workspace's counter area and a second kernel merges the
// chunks in chunk order (measured: merging inside the attention kernel by
// the last workgroup of a head, after device-scope stores and a counter,
// cost 8 us of a 14 us call; the kernel boundary is cheaper).
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr int kAttnBlk = 128;     // tokens per block
constexpr int kTpw = kAttnBlk / 4;    // scores: tokens per wave
constexpr int kWpb = kAttnBlk / 64;   // softmax: waves over one head's tokens
constexpr int kHg = 4 / kWpb;         // softmax: head groups (heads j with j % kHg == group)

constexpr int kAttnThreads = 256;
constexpr uint32_t kAttnTargetWgs = 256;
constexpr uint32_t kAttnMaxBpc = 2;         // blocks walked by one workgroup at most (when the workspace allows)

// The cache: INT8 codes [rows][D] with one scale per row (NG == 0), or INT4
// codes packed two per byte [rows][D/2] (even element in the low nibble)
// with NG groups of D/NG values per row, a scale and a zero per group
// (value = code * scale - zero * scale).  rows = T * Hkv, row = t * Hkv + head.
struct KvCache {
    const uint8_t *kc, *vc;
    const float *ks, *vs;   // [rows] (INT8) or [rows][NG] (INT4)
    const float *kz, *vz;   // INT4 zeros [rows][NG]
};

// Sequence b of a batch: its first cache token and its token count.  With
// seq_start NULL (one sequence) that is 0 and T; else seq_start[b] and
// seq_start[b+1] - seq_start[b], capped at tmax (device data the host never
// sees: a bad entry only makes the reads leave the cache, and those read
// zeros).
struct Seq {
    uint32_t base, len;
};

__device__ __forceinline__ Seq seq_of(const uint32_t *seq_start, uint32_t b, uint32_t T, uint32_t tmax) {
    if (!seq_start) return Seq{0u, T};
    const uint32_t s0 = seq_start[b], s1 = seq_start[b + 1];
    const uint32_t n = s1 > s0 ? s1 - s0 : 0u;
    return Seq{s0, n < tmax ? n : tmax};
}

// T: tokens in the cache (with a batch, the rows of all sequences); grid:
// batch x KV head x chunk.
template <int D, int GM, int NG>
__global__ __launch_bounds__(kAttnThreads) void attn_decode(const float *__restrict__ q, uint32_t G, uint32_t hkv,
                                                            uint32_t T, const uint32_t *__restrict__ seq_start,
                                                            uint32_t tmax, KvCache C, float sm_scale,
                                                            uint32_t nchunks, uint32_t bpc, float *__restrict__ out,
                                                            float *__restrict__ partials) {
    constexpr int LPT = D / 16;               // scores: lanes per token (16 dims each)
    constexpr int TPI = kWave / LPT;          // scores: tokens per wave load
    constexpr int SLOTS = kTpw / TPI;         // scores: loads per lane per block
    constexpr int TPR = D / 4;                // values: threads per token row (4 dims each)
    constexpr int NTG = kAttnThreads / TPR;   // values: token groups
    constexpr int TPG = kAttnBlk / NTG;       // values: tokens per group
    static_assert(D == 64 || D == 128 || D == 256, "head_dim");
    constexpr bool I4 = NG > 0;
    constexpr int NGS = I4 ? NG : 1;                 // scale slots per row
    constexpr uint32_t RB = I4 ? D / 2 : D;          // code bytes per row
    __shared__ float s_w[kAttnBlk][GM];              // scores; INT8: then p * v_scale
    __shared__ float s_wz[I4 ? kAttnBlk : 1][GM][I4 ? 2 * NGS : 1];   // INT4: p * s, p * s * z per group
    __shared__ float s_red[kWpb][GM][2];             // per wave of a head group: block max, block sum
    __shared__ float s_o[NTG][GM][D];                // the token groups' outputs

    const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint32_t per_b = hkv * nchunks;
    const uint32_t b = blockIdx.x / per_b, g = (blockIdx.x % per_b) / nchunks, c = blockIdx.x % nchunks;
    const Seq sq = seq_of(seq_start, b, T, tmax);
    const uint32_t hq = hkv * G;
    q += (size_t)b * hq * D;
    out += (size_t)b * hq * D;
    const uint32_t nblk = (sq.len + kAttnBlk - 1) / kAttnBlk;
    const uint32_t blk0 = c * bpc, blk1 = blk0 + bpc < nblk ? blk0 + bpc : nblk;
    if (blk0 >= nblk) {
        // no tokens in this chunk: the merge reads only chunks that have
        // some; an empty sequence without chunks gets zeros
        if (nchunks == 1)
            for (uint32_t i = threadIdx.x; i < G * D; i += kAttnThreads) out[(size_t)g * G * D + i] = 0.f;
        return;
    }

    // query rows of this head group, the 16 dims of this lane's key slice
    // (INT4: they lie in group l8 / (16 / (D / NG)) ... one group, since a
    // group holds a multiple of 16 values)
    const uint32_t l8 = lane % LPT, tk = lane / LPT;
    // (buffer loads: padding heads read zeros without a branch, so the
    // cache loads below are issued before the query arrives)
    float qr[GM][16], qsum[GM];
    const rsrc_t rq = make_rsrc(q, hq * D * 4);
#pragma unroll
    for (int j = 0; j < GM; ++j) {
        const uint32_t qo = (uint32_t)j < G ? ((g * G + j) * D + 16 * l8) * 4 : kOffNone;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qo, 16 * e4, 0));
            qr[j][4 * e4] = v.x; qr[j][4 * e4 + 1] = v.y; qr[j][4 * e4 + 2] = v.z; qr[j][4 * e4 + 3] = v.w;
        }
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) sq += qr[j][e];
        qsum[j] = sq;
    }
    const uint32_t kgrp = I4 ? (16 * l8) / (D / NGS) : 0;   // INT4 group of this lane's key dims

    const uint32_t rows = T * hkv;
    const rsrc_t rk = make_rsrc(C.kc, rows * RB), rv = make_rsrc(C.vc, rows * RB);
    const rsrc_t rks = make_rsrc(C.ks, rows * NGS * 4), rvs = make_rsrc(C.vs, rows * NGS * 4);
    const rsrc_t rkz = make_rsrc(I4 ? C.kz : C.ks, rows * NGS * 4), rvz = make_rsrc(I4 ? C.vz : C.vs, rows * NGS * 4);
    const uint32_t tg = tid / TPR, e4 = tid % TPR;        // values: token group, 4-dim slice
    const uint32_t vgrp = I4 ? (4 * e4) / (D / NGS) : 0;  // INT4 group of this thread's value dims
    const uint32_t tt = tid % kAttnBlk, hp = tid / kAttnBlk;   // softmax: token, head group

    float o[GM][4], oz[GM];
    float m_run[GM], l_run[GM];
#pragma unroll
    for (int j = 0; j < GM; ++j) {
        m_run[j] = -__builtin_inff();
        l_run[j] = 0.f;
        oz[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[j][e] = 0.f;
    }

    for (uint32_t blk = blk0; blk < blk1; ++blk) {
        const uint32_t t0 = blk * kAttnBlk;
        // -- loads of the block (out-of-range tokens read zeros)
        u32x4 kraw[SLOTS];
        float ksc[SLOTS], kzr[SLOTS];
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const uint32_t t = t0 + wv * kTpw + i * TPI + tk;
            const uint32_t row = (sq.base + t) * hkv + g;
            if (I4) {
                const u32x2 w2 = __builtin_amdgcn_raw_buffer_load_b64(rk, t < sq.len ? row * RB + 8 * l8 : kOffNone, 0, 0);
                kraw[i] = u32x4{w2.x, w2.y, 0u, 0u};
                const uint32_t so = t < sq.len ? (row * NGS + kgrp) * 4 : kOffNone;
                ksc[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, so, 0, 0));
                kzr[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rkz, so, 0, 0));
            } else {
                kraw[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, t < sq.len ? row * RB + 16 * l8 : kOffNone, 0, 0);
                ksc[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, t < sq.len ? row * 4 : kOffNone, 0, 0));
                kzr[i] = 0.f;
            }
        }
        uint32_t vraw[TPG];
#pragma unroll
        for (int u = 0; u < TPG; ++u) {
            const uint32_t t = t0 + tg * TPG + u;
            const uint32_t row = (sq.base + t) * hkv + g;
            if (I4)
                vraw[u] = __builtin_amdgcn_raw_buffer_load_b16(rv, t < sq.len ? row * RB + 2 * e4 : kOffNone, 0, 0);
            else
                vraw[u] = __builtin_amdgcn_raw_buffer_load_b32(rv, t < sq.len ? row * RB + 4 * e4 : kOffNone, 0, 0);
        }
        const uint32_t tv = t0 + tt;
        const uint32_t vrow = (sq.base + tv) * hkv + g;
        float vsc[NGS], vzr[NGS];
#pragma unroll
        for (int k = 0; k < NGS; ++k) {
            const uint32_t so = tv < sq.len ? (vrow * NGS + k) * 4 : kOffNone;
            vsc[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvs, so, 0, 0));
            vzr[k] = I4 ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvz, so, 0, 0)) : 0.f;
        }

        // -- 1. scores
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            float x[16];
            if (I4) {
#pragma unroll
                for (int w = 0; w < 2; ++w)
#pragma unroll
                    for (int b = 0; b < 8; ++b) x[8 * w + b] = (float)((kraw[i][w] >> (4 * b)) & 0xFu);
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w)
#pragma unroll
                    for (int b = 0; b < 4; ++b) x[4 * w + b] = (float)(int8_t)(kraw[i][w] >> (8 * b));
            }
            const uint32_t lt = wv * kTpw + i * TPI + tk;
            const bool valid = t0 + lt < sq.len;
#pragma unroll
            for (int j = 0; j < GM; ++j) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) d = __builtin_fmaf(qr[j][e], x[e], d);
                // INT8: scale the row's integer dot product once after the
                // sum; INT4: each lane's 16 values share one group
                if (I4) d = ksc[i] * __builtin_fmaf(-kzr[i], qsum[j], d);
                d = team_sum<LPT>(d);
                const float s = valid ? (I4 ? d : d * ksc[i]) * sm_scale : -__builtin_inff();
                if (l8 == 0) s_w[lt][j] = s;
            }
        }
        __syncthreads();

        // -- 2. softmax of the block: thread (token tt, head group hp) owns heads hp, hp + kHg, ...
        const uint32_t half = (tid / 64) % kWpb;
#pragma unroll
        for (int j = 0; j < GM; ++j) {
            if ((uint32_t)(j % kHg) != hp) continue;
            const float bm = team_max<64>(s_w[tt][j]);
            if (lane == 0) s_red[half][j][0] = bm;
        }
        __syncthreads();
        float alpha[GM];
#pragma unroll
        for (int j = 0; j < GM; ++j) {
            float bm = s_red[0][j][0];
#pragma unroll
            for (int w = 1; w < kWpb; ++w) bm = fmaxf(bm, s_red[w][j][0]);
            const float mn = fmaxf(m_run[j], bm);
            alpha[j] = expf(m_run[j] - mn);   // 0 for the first block (m_run = -inf)
            m_run[j] = mn;
        }
#pragma unroll
        for (int j = 0; j < GM; ++j) {
            if ((uint32_t)(j % kHg) != hp) continue;
            const float p = expf(s_w[tt][j] - m_run[j]);   // 0 for tokens past the end
            if (I4) {
#pragma unroll
                for (int k = 0; k < NGS; ++k) {
                    const float ps = p * vsc[k];
                    s_wz[I4 ? tt : 0][j][2 * k] = ps;
                    s_wz[I4 ? tt : 0][j][I4 ? 2 * k + 1 : 0] = ps * vzr[k];
                }
            } else {
                s_w[tt][j] = p * vsc[0];
            }
            const float bs = team_sum<64>(p);
            if (lane == 0) s_red[half][j][1] = bs;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < GM; ++j) {
            float bs = s_red[0][j][1];
#pragma unroll
            for (int w = 1; w < kWpb; ++w) bs += s_red[w][j][1];
            l_run[j] = l_run[j] * alpha[j] + bs;
        }

        // -- 3. values: INT8 sum_t (p v_scale) code; INT4 sum_t (p s) code - sum_t (p s z)
#pragma unroll
        for (int j = 0; j < GM; ++j) {
            oz[j] *= alpha[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[j][e] *= alpha[j];
        }
#pragma unroll
        for (int u = 0; u < TPG; ++u) {
            float cv[4];
            if (I4) {
#pragma unroll
                for (int b = 0; b < 4; ++b) cv[b] = (float)((vraw[u] >> (4 * b)) & 0xFu);
            } else {
#pragma unroll
                for (int b = 0; b < 4; ++b) cv[b] = (float)(int8_t)(vraw[u] >> (8 * b));
            }
#pragma unroll
            for (int j = 0; j < GM; ++j) {
                float w;
                if (I4) {
                    w = s_wz[I4 ? tg * TPG + u : 0][j][2 * vgrp];
                    oz[j] += s_wz[I4 ? tg * TPG + u : 0][j][I4 ? 2 * vgrp + 1 : 0];
                } else {
                    w = s_w[tg * TPG + u][j];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) o[j][e] = __builtin_fmaf(w, cv[e], o[j][e]);
            }
        }
        __syncthreads();   // s_w, s_wz and s_red are rewritten by the next block
    }

    // -- the 8 token groups, added in order
#pragma unroll
    for (int j = 0; j < GM; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_o[tg][j][4 * e4 + e] = o[j][e] - oz[j];
    __syncthreads();
    constexpr int kOut = GM * D;   // outputs of the head group
    float ov[(kOut + kAttnThreads - 1) / kAttnThreads];
#pragma unroll
    for (int r = 0; r * kAttnThreads < kOut; ++r) {
        const uint32_t idx = tid + r * kAttnThreads;
        float a = 0.f;
        if (idx < (uint32_t)kOut) {
            const uint32_t j = idx / D, d = idx % D;
#pragma unroll
            for (int x = 0; x < NTG; ++x) a += s_o[x][j][d];
        }
        ov[r] = a;
    }

    if (nchunks == 1) {
#pragma unroll
        for (int r = 0; r * kAttnThreads < kOut; ++r) {
            const uint32_t idx = tid + r * kAttnThreads;
            const uint32_t j = idx / D, d = idx % D;
            if (idx < (uint32_t)kOut && j < G) {
                float l = 0.f;
#pragma unroll
                for (int jj = 0; jj < GM; ++jj) l = (uint32_t)jj == j ? l_run[jj] : l;
                out[(size_t)(g * G + j) * D + d] = ov[r] / l;
            }
        }
        return;
    }

    // -- several chunks: (output, max, sum, 2 pad) of this chunk as a record
    // [sequence][head][chunk][GM][D + 4] behind the workspace's counter area; the
    // merge kernel that follows on the stream combines them
    constexpr uint32_t kRecD = D + 4;
    float *rec = partials + (((size_t)b * hkv + g) * nchunks + c) * GM * kRecD;
#pragma unroll
    for (int r = 0; r * kAttnThreads < kOut; ++r) {
        const uint32_t idx = tid + r * kAttnThreads;
        if (idx < (uint32_t)kOut) {
            const uint32_t j = idx / D, d = idx % D;
            rec[j * kRecD + d] = ov[r];
            if (d == 0) {
                float m = 0.f, l = 0.f;
#pragma unroll
                for (int jj = 0; jj < GM; ++jj) {
                    m = (uint32_t)jj == j ? m_run[jj] : m;
                    l = (uint32_t)jj == j ? l_run[jj] : l;
                }
                rec[j * kRecD + D] = m;
                rec[j * kRecD + D + 1] = l;
            }
        }
    }
}

// Merge of the chunk records: one workgroup per query head (KV head g, head
// j of its group), one thread per output dim.  All output values of a batch
// of 64 chunks are loaded at once; lane u of each wave takes chunk u's max
// and sum, and fixed-order DPP reductions give the batch max, the chunk
// weights exp(m_c - M) and the weighted sum of the sums, so the chunks are
// added in order and the result does not depend on launch timing.
template <int D, int GM>
__global__ __launch_bounds__(D) void attn_merge(const float *__restrict__ partials, uint32_t G, uint32_t hkv,
                                                uint32_t T, const uint32_t *__restrict__ seq_start, uint32_t tmax,
                                                uint32_t nchunks_max, uint32_t bpc, float *__restrict__ out) {
    constexpr uint32_t kRecD = D + 4;
    const uint32_t per_b = hkv * G;
    const uint32_t b = blockIdx.x / per_b, g = (blockIdx.x % per_b) / G, j = blockIdx.x % G;
    const uint32_t d = threadIdx.x, lane = d & 63;
    out += (size_t)b * per_b * D;
    // the chunks that hold tokens of this sequence
    const Seq sq = seq_of(seq_start, b, T, tmax);
    const uint32_t nblk = (sq.len + kAttnBlk - 1) / kAttnBlk;
    const uint32_t nchunks = (nblk + bpc - 1) / bpc;
    if (nchunks == 0) {
        out[((size_t)g * G + j) * D + d] = 0.f;
        return;
    }
    // this head's records: chunk c at (c * GM + j) * kRecD floats (buffer
    // loads: chunks past the end read zeros without a branch)
    const rsrc_t rp = make_rsrc(partials + ((size_t)b * hkv + g) * nchunks_max * GM * kRecD,
                                nchunks * GM * kRecD * 4);
    float M = -__builtin_inff(), L = 0.f, O = 0.f;
    for (uint32_t c0 = 0; c0 < nchunks; c0 += 64) {
        float ov[64];
#pragma unroll
        for (int u = 0; u < 64; ++u) {
            const uint32_t off = c0 + u < nchunks ? (((c0 + u) * GM + j) * kRecD + d) * 4 : kOffNone;
            ov[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, off, 0, 0));
        }
        const bool in = c0 + lane < nchunks;
        const uint32_t ro = in ? (((c0 + lane) * GM + j) * kRecD + D) * 4 : kOffNone;
        const float mc = in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, ro, 0, 0)) : -__builtin_inff();
        const float lc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, ro, 4, 0));
        const float mn = fmaxf(M, team_max<64>(mc));
        const float a = expf(M - mn);   // rescales earlier batches (0 for the first)
        const float bw = in ? expf(mc - mn) : 0.f;
        L = L * a + team_sum<64>(bw * lc);
        O *= a;
#pragma unroll
        for (int u = 0; u < 64; ++u) O = __builtin_fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(bw), u)), ov[u], O);
        M = mn;
    }
    out[((size_t)g * G + j) * D + d] = O / L;
}

struct AttnPlan {
    uint32_t gm, nchunks, bpc;
    size_t ws_bytes;
};

uint32_t attn_gm(uint32_t G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8; }

// ~256 workgroups: split each (sequence, KV head)'s tokens, up to tmax, into
// chunks of whole 128-token blocks
AttnPlan attn_plan(uint32_t hq, uint32_t hkv, uint32_t B, uint32_t tmax, uint32_t D) {
    AttnPlan pl;
    pl.gm = attn_gm(hq / hkv);
    uint32_t nblk = (tmax + kAttnBlk - 1) / kAttnBlk;
    if (nblk < 1) nblk = 1;
    const uint64_t units = (uint64_t)B * hkv;
    uint32_t want = units >= kAttnTargetWgs ? 1u : (uint32_t)(kAttnTargetWgs / units);
    // a workgroup walks its blocks one after another (each a memory round
    // trip): with many sequences, more and shorter chunks instead
    const uint32_t by_len = (nblk + kAttnMaxBpc - 1) / kAttnMaxBpc;
    if (want < by_len) want = by_len;
    if (want > nblk) want = nblk;
    pl.bpc = (nblk + want - 1) / want;
    pl.nchunks = (nblk + pl.bpc - 1) / pl.bpc;
    pl.ws_bytes = pl.nchunks > 1 ? KVQ_WORKSPACE_COUNTER_BYTES + units * pl.nchunks * pl.gm * (D + 4) * 4 : 0;
    return pl;
}

int check_heads(const char *fn, uint32_t hq, uint32_t hkv, uint32_t D) {
    if (hq == 0 || hkv == 0)
        return fail(KVQ_E_INVALID, "%s: num_q_heads=%u num_kv_heads=%u (want both > 0)", fn, hq, hkv);
    if (hq % hkv || hq / hkv > 8)
        return fail(KVQ_E_INVALID, "%s: num_q_heads=%u is not 1..8 times num_kv_heads=%u", fn, hq, hkv);
    if (D != 64 && D != 128 && D != 256)
        return fail(KVQ_E_INVALID, "%s: head_dim=%u (supported: 64, 128, 256)", fn, D);
    return KVQ_OK;
}

int check_attn(const char *fn, uint32_t hq, uint32_t hkv, uint32_t T, uint32_t D) {
    if (T == 0) return fail(KVQ_E_INVALID, "%s: num_tokens=0 (want > 0)", fn);
    const int st = check_heads(fn, hq, hkv, D);
    if (st) return st;
    if ((uint64_t)T * hkv * D >= 0x80000000ull) return fail(KVQ_E_INVALID, "%s: cache larger than 2 GiB", fn);
    if ((uint64_t)hq * D * 4 >= 0x80000000ull) return fail(KVQ_E_INVALID, "%s: queries larger than 2 GiB", fn);
    return KVQ_OK;
}

int check_varlen(const char *fn, uint32_t B, uint32_t hq, uint32_t hkv, uint32_t total, uint32_t tmax, uint32_t D,
                 const uint32_t *seq_start) {
    if (B == 0) return fail(KVQ_E_INVALID, "%s: batch=0 (want > 0)", fn);
    const int st = check_heads(fn, hq, hkv, D);
    if (st) return st;
    if (tmax > total) return fail(KVQ_E_INVALID, "%s: max_seq_tokens=%u exceeds total_tokens=%u", fn, tmax, total);
    if ((uint64_t)total * hkv * D >= 0x80000000ull) return fail(KVQ_E_INVALID, "%s: cache larger than 2 GiB", fn);
    if ((uint64_t)B * hq * D * 4 >= 0x80000000ull) return fail(KVQ_E_INVALID, "%s: queries larger than 2 GiB", fn);
    if ((uint64_t)B * hkv * hq >= 0x80000000ull) return fail(KVQ_E_INVALID, "%s: batch too large", fn);
    if (!seq_start || (reinterpret_cast<uintptr_t>(seq_start) & 3u))
        return fail(KVQ_E_INVALID, "%s: seq_start must be a 4-byte aligned device pointer", fn);
    return KVQ_OK;
}

template <int D, int GM, int NG>
void attn_launch(const float *q, uint32_t B, uint32_t G, uint32_t hkv, uint32_t T, const uint32_t *seq_start,
                 uint32_t tmax, const KvCache &C, float sc, const AttnPlan &pl, float *out, float *partials,
                 hipStream_t s) {
    const unsigned grid = B * hkv * pl.nchunks;
    attn_decode<D, GM, NG><<<grid, kAttnThreads, 0, s>>>(q, G, hkv, T, seq_start, tmax, C, sc, pl.nchunks, pl.bpc,
                                                         out, partials);
    if (pl.nchunks > 1)
        attn_merge<D, GM><<<B * hkv * G, D, 0, s>>>(partials, G, hkv, T, seq_start, tmax, pl.nchunks, pl.bpc, out);
}

#define KVQ_ATTN_ARGS q, B, G, hkv, T, seq_start, tmax, C, sc, pl, out, partials, s
#define KVQ_ATTN_PARAMS                                                                                          \
    const float *q, uint32_t B, uint32_t G, uint32_t hkv, uint32_t T, const uint32_t *seq_start, uint32_t tmax, \
        const KvCache &C, float sc, const AttnPlan &pl, float *out, float *partials, hipStream_t s

template <int D, int NG>
void attn_by_group(KVQ_ATTN_PARAMS) {
    switch (pl.gm) {
        case 1: attn_launch<D, 1, NG>(KVQ_ATTN_ARGS); break;
        case 2: attn_launch<D, 2, NG>(KVQ_ATTN_ARGS); break;
        case 4: attn_launch<D, 4, NG>(KVQ_ATTN_ARGS); break;
        default: attn_launch<D, 8, NG>(KVQ_ATTN_ARGS); break;
    }
}

// ng == 0: INT8 per-token cache; else INT4 with ng groups of 32..128 values per row
template <int D>
void attn_by_format(int ng, KVQ_ATTN_PARAMS) {
    if (ng == 0) attn_by_group<D, 0>(KVQ_ATTN_ARGS);
    if constexpr (D <= 128) {
        if (ng == 1) attn_by_group<D, 1>(KVQ_ATTN_ARGS);
    }
    if (ng == 2) attn_by_group<D, 2>(KVQ_ATTN_ARGS);
    if constexpr (D >= 128) {
        if (ng == 4) attn_by_group<D, 4>(KVQ_ATTN_ARGS);
    }
    if constexpr (D == 256) {
        if (ng == 8) attn_by_group<D, 8>(KVQ_ATTN_ARGS);
    }
}

// B sequences (seq_start NULL: one sequence of T tokens); T: cache tokens
int attn_run(const char *fn, const float *q, uint32_t B, uint32_t hq, uint32_t hkv, uint32_t T,
             const uint32_t *seq_start, uint32_t tmax, uint32_t D, int ng, const KvCache &C, float sc, float *out,
             void *workspace, size_t workspace_bytes, void *stream) {
    if (!(sc == sc) || __builtin_isinf(sc)) return fail(KVQ_E_INVALID, "%s: softmax_scale is not finite", fn);
    AttnPlan pl = attn_plan(hq, hkv, B, tmax, D);
    float *partials = nullptr;
    if (pl.nchunks > 1) {
        if (!workspace || workspace_bytes < pl.ws_bytes || !aligned16(workspace)) {
            pl.bpc = (tmax + kAttnBlk - 1) / kAttnBlk;   // no workspace: one workgroup per (sequence, KV head)
            if (pl.bpc < 1) pl.bpc = 1;
            pl.nchunks = 1;
        } else {
            partials = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + KVQ_WORKSPACE_COUNTER_BYTES);
        }
    }
    const uint32_t G = hq / hkv;
    hipStream_t s = as_stream(stream);
    if (D == 64) attn_by_format<64>(ng, KVQ_ATTN_ARGS);
    else if (D == 128) attn_by_format<128>(ng, KVQ_ATTN_ARGS);
    else attn_by_format<256>(ng, KVQ_ATTN_ARGS);
    return launch_status(fn);
}

#undef KVQ_ATTN_ARGS
#undef KVQ_ATTN_PARAMS

KvCache cache8(const int8_t *kc, const float *ks, const int8_t *vc, const float *vs) {
    KvCache C;
    C.kc = reinterpret_cast<const uint8_t *>(kc);
    C.vc = reinterpret_cast<const uint8_t *>(vc);
    C.ks = ks; C.vs = vs;
    C.kz = nullptr; C.vz = nullptr;
    return C;
}

KvCache cache4(const uint8_t *kp, const float *ks, const float *kz, const uint8_t *vp, const float *vs,
               const float *vz) {
    KvCache C;
    C.kc = kp; C.vc = vp;
    C.ks = ks; C.vs = vs;
    C.kz = kz; C.vz = vz;
    return C;
}

int check_group(const char *fn, uint32_t group_size, uint32_t head_dim) {
    if ((group_size != 32 && group_size != 64 && group_size != 128) || group_size > head_dim)
        return fail(KVQ_E_INVALID, "%s: group_size=%u (supported: 32, 64, 128, at most head_dim)", fn, group_size);
    return KVQ_OK;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" int kvq_attn_decode_workspace_bytes(uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t num_tokens,
                                               uint32_t head_dim, size_t *bytes) {
    if (!bytes) return fail(KVQ_E_INVALID, "kvq_attn_decode_workspace_bytes: null output pointer");
    *bytes = 0;
    const int st = check_attn("kvq_attn_decode_workspace_bytes", num_q_heads, num_kv_heads, num_tokens, head_dim);
    if (st) return st;
    *bytes = attn_plan(num_q_heads, num_kv_heads, 1, num_tokens, head_dim).ws_bytes;
    return KVQ_OK;
}

extern "C" int kvq_attn_decode_varlen_workspace_bytes(uint32_t batch, uint32_t num_q_heads, uint32_t num_kv_heads,
                                                      uint32_t max_seq_tokens, uint32_t head_dim, size_t *bytes) {
    const char *fn = "kvq_attn_decode_varlen_workspace_bytes";
    if (!bytes) return fail(KVQ_E_INVALID, "%s: null output pointer", fn);
    *bytes = 0;
    if (batch == 0) return fail(KVQ_E_INVALID, "%s: batch=0 (want > 0)", fn);
    const int st = check_heads(fn, num_q_heads, num_kv_heads, head_dim);
    if (st) return st;
    *bytes = attn_plan(num_q_heads, num_kv_heads, batch, max_seq_tokens, head_dim).ws_bytes;
    return KVQ_OK;
}

extern "C" int kvq_attn_decode_int8(const float *q, uint32_t num_q_heads, uint32_t num_kv_heads,
                                    uint32_t num_tokens, uint32_t head_dim, const int8_t *k_codes,
                                    const float *k_scales, const int8_t *v_codes, const float *v_scales,
                                    float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                    void *stream) {
    const char *fn = "kvq_attn_decode_int8";
    int st = check_attn(fn, num_q_heads, num_kv_heads, num_tokens, head_dim);
    if (st) return st;
    st = check_ptrs(fn, {q, k_codes, k_scales, v_codes, v_scales, out});
    if (st) return st;
    return attn_run(fn, q, 1, num_q_heads, num_kv_heads, num_tokens, nullptr, num_tokens, head_dim, 0,
                    cache8(k_codes, k_scales, v_codes, v_scales), softmax_scale, out, workspace, workspace_bytes,
                    stream);
}

extern "C" int kvq_attn_decode_int4(const float *q, uint32_t num_q_heads, uint32_t num_kv_heads,
                                    uint32_t num_tokens, uint32_t head_dim, uint32_t group_size,
                                    const uint8_t *k_packed, const float *k_scales, const float *k_zeros,
                                    const uint8_t *v_packed, const float *v_scales, const float *v_zeros,
                                    float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                    void *stream) {
    const char *fn = "kvq_attn_decode_int4";
    int st = check_attn(fn, num_q_heads, num_kv_heads, num_tokens, head_dim);
    if (st) return st;
    st = check_group(fn, group_size, head_dim);
    if (st) return st;
    st = check_ptrs(fn, {q, k_packed, k_scales, k_zeros, v_packed, v_scales, v_zeros, out});
    if (st) return st;
    return attn_run(fn, q, 1, num_q_heads, num_kv_heads, num_tokens, nullptr, num_tokens, head_dim,
                    (int)(head_dim / group_size), cache4(k_packed, k_scales, k_zeros, v_packed, v_scales, v_zeros),
                    softmax_scale, out, workspace, workspace_bytes, stream);
}

extern "C" int kvq_attn_decode_int8_varlen(const float *q, uint32_t batch, uint32_t num_q_heads,
                                           uint32_t num_kv_heads, uint32_t head_dim, const uint32_t *seq_start,
                                           uint32_t total_tokens, uint32_t max_seq_tokens, const int8_t *k_codes,
                                           const float *k_scales, const int8_t *v_codes, const float *v_scales,
                                           float softmax_scale, float *out, void *workspace,
                                           size_t workspace_bytes, void *stream) {
    const char *fn = "kvq_attn_decode_int8_varlen";
    int st = check_varlen(fn, batch, num_q_heads, num_kv_heads, total_tokens, max_seq_tokens, head_dim, seq_start);
    if (st) return st;
    st = check_ptrs(fn, {q, k_codes, k_scales, v_codes, v_scales, out});
    if (st) return st;
    return attn_run(fn, q, batch, num_q_heads, num_kv_heads, total_tokens, seq_start, max_seq_tokens, head_dim, 0,
                    cache8(k_codes, k_scales, v_codes, v_scales), softmax_scale, out, workspace, workspace_bytes,
                    stream);
}

extern "C" int kvq_attn_decode_int4_varlen(const float *q, uint32_t batch, uint32_t num_q_heads,
                                           uint32_t num_kv_heads, uint32_t head_dim, uint32_t group_size,
                                           const uint32_t *seq_start, uint32_t total_tokens,
                                           uint32_t max_seq_tokens, const uint8_t *k_packed, const float *k_scales,
                                           const float *k_zeros, const uint8_t *v_packed, const float *v_scales,
                                           const float *v_zeros, float softmax_scale, float *out, void *workspace,
                                           size_t workspace_bytes, void *stream) {
    const char *fn = "kvq_attn_decode_int4_varlen";
    int st = check_varlen(fn, batch, num_q_heads, num_kv_heads, total_tokens, max_seq_tokens, head_dim, seq_start);
    if (st) return st;
    st = check_group(fn, group_size, head_dim);
    if (st) return st;
    st = check_ptrs(fn, {q, k_packed, k_scales, k_zeros, v_packed, v_scales, v_zeros, out});
    if (st) return st;
    return attn_run(fn, q, batch, num_q_heads, num_kv_heads, total_tokens, seq_start, max_seq_tokens, head_dim,
                    (int)(head_dim / group_size), cache4(k_packed, k_scales, k_zeros, v_packed, v_scales, v_zeros),
                    softmax_scale, out, workspace, workspace_bytes, stream);
}
