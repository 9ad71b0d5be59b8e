// INT4 AWQ weight-only GEMV/GEMM with the fused Q/K/V layout, for gfx950.
//
// Follows boostr fused_int4_qkv.rs: QKV_AWQ_SHIFTS / unpack_awq_qkv (column j
// of an 8-column u32 word is the nibble at bit SHIFTS[j], SHIFTS = 0, 16, 4,
// 20, 8, 24, 12, 28) and fused_int4_qkv_q / _k / _v (out[m][j] = sum_k
// x[m][k] * (q - zero[k/gs][j]) * scale[k/gs][j], weights [K][n/8], fp32
// scales and zeros [K/gs][n]).  The page runs three dispatches of one thread
// per output with a serial K loop; here Q, K and V are one launch over the
// concatenated word columns, and the sum runs on the matrix cores:
//
//   out = sum_g s_g * (P_g - z_g * X_g),  P_g = sum_{k in g} x~_k * q_k,
//                                          X_g = sum_{k in g} x~_k
//
// with x~ = fp16(x) (round to nearest even) and the integer codes q exact in
// fp16, so P_g and X_g come from v_mfma_f32_16x16x32_f16 (X_g with an all-ones
// B operand) and the only rounding of the inputs is the activation's.  s and z
// are applied per group in fp32.
//
// Operand construction: one wave owns 16 word columns (128 output columns).
// Lane (wc = l % 16, kg = l / 16) loads the words of 8 consecutive K rows of
// word column wc; v_perm_b32 pairs the bytes of rows k and k+1 so that each
// 16-bit half holds the same column's nibbles from the two rows, and the
// "1024 + q" half-precision magic (OR with 0x6400, then subtract 1024, or
// scale by 1/16 for a nibble sitting 4 bits higher) yields the exact codes.
// The 8 column positions of a word become 8 MFMA B operands; MFMA number c
// computes output columns 8*wc + c.  A operands are the activation rows: lane
// (m, kg) holds x~[m][8*kg .. 8*kg+7] of the 32-wide K step, the same K order
// as the weights.
//
// Work split: a workgroup of 4 waves covers one 128-column tile, one chunk of
// 16 or 32 activation rows and 4 consecutive slices of the K groups; the waves
// meet in LDS.  When K is sliced across workgroups (small M needs it to fill
// 256 CUs), each workgroup writes its partial tile to the caller's workspace
// and the last one to arrive (a per-tile counter) adds the partials in a fixed
// order, writes the output and resets the counter.
#include "kvq_common.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;
constexpr int kTargetWaves = 2048;

struct Projs {
    const uint32_t *qw[3];
    const float *sc[3];
    const float *zr[3];
    float *out[3];
    uint32_t wstart[3];   // first global word column of each projection
    uint32_t n[3];        // output columns of each projection
    uint32_t count;
    uint32_t wtotal;      // total word columns
};

__device__ __forceinline__ int proj_of(const Projs &P, uint32_t gw) {
    return (P.count > 1 && gw >= P.wstart[1]) ? ((P.count > 2 && gw >= P.wstart[2]) ? 2 : 1) : 0;
}

// Agent-coherent (sc1) accesses for the partial tiles exchanged between
// workgroups that may run on different XCDs (whose L2s are not coherent).
__device__ __forceinline__ void store_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f16x2 h2_bits(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t h2_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// Exact codes of a nibble at bits 0-3 of each half: (1024 + q) - 1024.
__device__ __forceinline__ uint32_t nib_lo(uint32_t t) {
    const f16x2 h = h2_bits((t & 0x000F000Fu) | 0x64006400u);
    return h2_u32(h - f16x2{(_Float16)1024.0f, (_Float16)1024.0f});
}
// Exact codes of a nibble at bits 4-7 of each half: (1024 + 16q) / 16 - 64.
__device__ __forceinline__ uint32_t nib_hi(uint32_t t) {
    const f16x2 h = h2_bits((t & 0x00F000F0u) | 0x64006400u);
    return h2_u32(__builtin_elementwise_fma(h, f16x2{(_Float16)0.0625f, (_Float16)0.0625f},
                                            f16x2{(_Float16)-64.0f, (_Float16)-64.0f}));
}

// 8 words (K rows 0..7 of one word column) -> 8 B operands, operand c holding
// column c's codes for K rows 0..7 (row 2i in the low half of register i).
__device__ __forceinline__ void awq_operands(const uint32_t w[8], f16x8 B[8]) {
    uint32_t r[8][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // even columns live in bytes 0-1 of a word, odd columns in bytes 2-3
        const uint32_t ev = __builtin_amdgcn_perm(w[2 * i + 1], w[2 * i], 0x05040100u);
        const uint32_t od = __builtin_amdgcn_perm(w[2 * i + 1], w[2 * i], 0x07060302u);
        r[0][i] = nib_lo(ev);
        r[2][i] = nib_hi(ev);
        r[4][i] = nib_lo(ev >> 8);
        r[6][i] = nib_hi(ev >> 8);
        r[1][i] = nib_lo(od);
        r[3][i] = nib_hi(od);
        r[5][i] = nib_lo(od >> 8);
        r[7][i] = nib_hi(od >> 8);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        u32x4 v = {r[c][0], r[c][1], r[c][2], r[c][3]};
        B[c] = __builtin_bit_cast(f16x8, v);
    }
}

__device__ __forceinline__ f16x8 to_f16x8(f32x4 a, f32x4 b) {
    f16x8 h;
    h[0] = (_Float16)a.x; h[1] = (_Float16)a.y; h[2] = (_Float16)a.z; h[3] = (_Float16)a.w;
    h[4] = (_Float16)b.x; h[5] = (_Float16)b.y; h[6] = (_Float16)b.z; h[7] = (_Float16)b.w;
    return h;
}

__device__ __forceinline__ f32x4 mfma16(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// MT: 16-row activation tiles per chunk (1 or 2).  R: accumulator rows per
// lane that can hold real outputs (1 when m == 1, else 4).  KSG: 32-wide K
// steps per quantization group (group_size / 32).
template <int MT, int R, int KSG>
__global__ __launch_bounds__(kBlock) void awq_gemm(const float *__restrict__ x, uint32_t M, uint32_t K, Projs P,
                                                   uint32_t nchunks, uint32_t ks_b, uint32_t *__restrict__ counters,
                                                   float *__restrict__ partials) {
    constexpr int MR = 16 * MT;
    constexpr uint32_t GS = 32 * KSG;
    __shared__ f32x4 red[4][16][32];
    __shared__ int s_last;
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
    const int wc = lane & 15, kg = lane >> 4;

    uint32_t b = blockIdx.x;
    const uint32_t s = b % ks_b;
    b /= ks_b;
    const uint32_t c = b % nchunks, t = b / nchunks;
    const uint32_t G = K / GS;
    const uint32_t nsplit = ks_b * 4, split = s * 4 + wv;
    const uint32_t g0 = (uint32_t)((uint64_t)split * G / nsplit);
    const uint32_t g1 = (uint32_t)((uint64_t)(split + 1) * G / nsplit);

    const uint32_t gw = t * 16 + wc;
    const bool wok = gw < P.wtotal;
    const int p = proj_of(P, wok ? gw : 0);
    const uint32_t lw = (wok ? gw : 0) - P.wstart[p];
    const uint32_t np = P.n[p], wp = np / 8;
    const uint32_t *qcol = P.qw[p] + lw + (size_t)(kg * 8) * wp;
    const float *scol = P.sc[p] + 8 * lw;
    const float *zcol = P.zr[p] + 8 * lw;

    const float *xrow[MT];
    bool xok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint32_t m = c * MR + mt * 16 + wc;
        xok[mt] = m < M;
        xrow[mt] = x + (size_t)(xok[mt] ? m : 0) * K + kg * 8;
    }

    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) acc[mt][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
    f16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;
    const f16x8 zero8 = ones - ones;

    for (uint32_t g = g0; g < g1; ++g) {
        uint32_t w[KSG][8];
#pragma unroll
        for (int ks = 0; ks < KSG; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                w[ks][i] = wok ? __builtin_nontemporal_load(qcol + (size_t)(g * GS + ks * 32 + i) * wp) : 0u;
        f16x8 a[KSG][MT];
#pragma unroll
        for (int ks = 0; ks < KSG; ++ks)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (xok[mt]) {
                    const f32x4 *xp = reinterpret_cast<const f32x4 *>(xrow[mt] + g * GS + ks * 32);
                    a[ks][mt] = to_f16x8(xp[0], xp[1]);
                } else {
                    a[ks][mt] = zero8;
                }
            }
        f32x4 pg[MT][8], xg[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            xg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) pg[mt][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < KSG; ++ks) {
            f16x8 B[8];
            awq_operands(w[ks], B);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                xg[mt] = mfma16(a[ks][mt], ones, xg[mt]);
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) pg[mt][cc] = mfma16(a[ks][mt], B[cc], pg[mt][cc]);
            }
        }
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, z0 = s0, z1 = s0;
        if (wok) {
            const f32x4 *sp = reinterpret_cast<const f32x4 *>(scol + (size_t)g * np);
            const f32x4 *zp = reinterpret_cast<const f32x4 *>(zcol + (size_t)g * np);
            s0 = sp[0]; s1 = sp[1]; z0 = zp[0]; z1 = zp[1];
        }
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int cc = 0; cc < 8; ++cc)
#pragma unroll
                for (int i = 0; i < R; ++i)
                    acc[mt][cc][i] = __builtin_fmaf(sv[cc], __builtin_fmaf(-zv[cc], xg[mt][i], pg[mt][cc][i]),
                                                    acc[mt][cc][i]);
    }

    // Waves -> LDS, one 16-row tile at a time, as [row][column] with
    // row = 4*kg + i and column = 8*wc + cc; then 256 threads add the four
    // waves' values and write 16-byte pieces of the output (or partial) rows.
    const uint32_t tile_id = t * nchunks + c;
    float *part = partials + (size_t)tile_id * ks_b * (MR * 128);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * kg + i;
            red[wv][row][2 * wc] = f32x4{acc[mt][0][i], acc[mt][1][i], acc[mt][2][i], acc[mt][3][i]};
            red[wv][row][2 * wc + 1] = f32x4{acc[mt][4][i], acc[mt][5][i], acc[mt][6][i], acc[mt][7][i]};
        }
        __syncthreads();
        for (int e = threadIdx.x; e < 16 * 32; e += kBlock) {
            const int row = e >> 5, col4 = e & 31;
            const uint32_t m = c * MR + mt * 16 + row;
            const uint32_t gwo = t * 16 + (col4 >> 1);
            if (m >= M || gwo >= P.wtotal) continue;
            const f32x4 v = red[0][row][col4] + red[1][row][col4] + red[2][row][col4] + red[3][row][col4];
            if (ks_b == 1) {
                const int po = proj_of(P, gwo);
                const uint32_t col = 8 * (gwo - P.wstart[po]) + (col4 & 1) * 4;
                *reinterpret_cast<f32x4 *>(P.out[po] + (size_t)m * P.n[po] + col) = v;
            } else {
                float *dst = part + (size_t)s * (MR * 128) + (mt * 16 + row) * 128 + col4 * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) store_agent(dst + j, v[j]);
            }
        }
        __syncthreads();
    }
    if (ks_b == 1) return;

    // Cross-workgroup K reduction.  The partial tiles were written with
    // agent-coherent stores (sc1, below); once every thread's stores have
    // completed, one atomic per workgroup counts arrivals, and the last
    // workgroup of the tile reads all partials with agent-coherent loads,
    // adds them in split order (so the result does not depend on arrival
    // order) and resets the counter for the next call.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&counters[tile_id], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == ks_b - 1;
    }
    __syncthreads();
    if (!s_last) return;
    for (int e = threadIdx.x; e < MR * 32; e += kBlock) {
        const int row = e >> 5, col4 = e & 31;
        const uint32_t m = c * MR + row;
        const uint32_t gwo = t * 16 + (col4 >> 1);
        if (m >= M || gwo >= P.wtotal) continue;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (uint32_t q = 0; q < ks_b; ++q) {
            const float *src = part + (size_t)q * (MR * 128) + row * 128 + col4 * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += load_agent(src + j);
        }
        const int po = proj_of(P, gwo);
        const uint32_t col = 8 * (gwo - P.wstart[po]) + (col4 & 1) * 4;
        *reinterpret_cast<f32x4 *>(P.out[po] + (size_t)m * P.n[po] + col) = v;
    }
    if (threadIdx.x == 0) __hip_atomic_store(&counters[tile_id], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ host --

struct Plan {
    uint32_t mt, mr, nchunks, ntiles, ks_b;
    size_t counter_bytes, partial_bytes;
};

Plan make_plan(uint32_t m, uint32_t k, uint32_t gs, uint32_t wtotal) {
    Plan pl;
    pl.mt = m <= 16 ? 1 : 2;
    pl.mr = 16 * pl.mt;
    pl.nchunks = (m + pl.mr - 1) / pl.mr;
    pl.ntiles = (wtotal + 15) / 16;
    const uint32_t groups = k / gs;
    const uint64_t units = (uint64_t)pl.ntiles * pl.nchunks;
    uint64_t waves = kTargetWaves / (units ? units : 1);
    if (waves > groups) waves = groups;
    if (waves < 1) waves = 1;
    pl.ks_b = (uint32_t)(waves / 4 ? waves / 4 : 1);
    const size_t tiles = (size_t)pl.ntiles * pl.nchunks;
    pl.counter_bytes = pl.ks_b > 1 ? ((tiles * 4 + 255) / 256) * 256 : 0;
    pl.partial_bytes = pl.ks_b > 1 ? tiles * pl.ks_b * pl.mr * 128 * 4 : 0;
    return pl;
}

int check_proj(const char *fn, const int4_awq_proj_t *p, const char *which, uint32_t m, uint32_t k, uint32_t gs) {
    (void)m;
    (void)gs;
    if (!p->qweight || !p->scales || !p->zeros || !p->out)
        return fail(KVQ_E_INVALID, "%s: %s projection has a null pointer", fn, which);
    if (!aligned16(p->qweight) || !aligned16(p->scales) || !aligned16(p->zeros) || !aligned16(p->out))
        return fail(KVQ_E_INVALID, "%s: %s projection pointers must be 16-byte aligned", fn, which);
    if (p->n == 0 || p->n % 8)
        return fail(KVQ_E_INVALID, "%s: %s projection n=%u (want a positive multiple of 8)", fn, which, p->n);
    (void)k;
    return KVQ_OK;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" int int4_awq_workspace_bytes(uint32_t m, uint32_t k, uint32_t group_size, uint32_t n_total,
                                        size_t *bytes) {
    if (!bytes) return fail(KVQ_E_INVALID, "int4_awq_workspace_bytes: null output pointer");
    if (m == 0 || group_size == 0 || k % group_size || n_total % 8) {
        *bytes = 0;
        return KVQ_OK;
    }
    const Plan pl = make_plan(m, k, group_size, n_total / 8);
    *bytes = pl.counter_bytes + pl.partial_bytes;
    return KVQ_OK;
}

extern "C" int int4_awq_qkv_gemm(const float *x, uint32_t m, uint32_t k, uint32_t group_size,
                                 const int4_awq_proj_t *q_proj, const int4_awq_proj_t *k_proj,
                                 const int4_awq_proj_t *v_proj, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    const char *fn = "int4_awq_qkv_gemm";
    if (!x || !q_proj) return fail(KVQ_E_INVALID, "%s: null x or q projection", fn);
    if (!aligned16(x)) return fail(KVQ_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
    if (m == 0) return fail(KVQ_E_INVALID, "%s: m == 0", fn);
    if (group_size != 32 && group_size != 64 && group_size != 128 && group_size != 256)
        return fail(KVQ_E_INVALID, "%s: group_size=%u (supported: 32, 64, 128, 256)", fn, group_size);
    if (k == 0 || k % group_size)
        return fail(KVQ_E_INVALID, "%s: K=%u is not a positive multiple of group_size=%u", fn, k, group_size);
    if ((k_proj == nullptr) != (v_proj == nullptr))
        return fail(KVQ_E_INVALID, "%s: k and v projections must be both set or both NULL", fn);
    int st = check_proj(fn, q_proj, "q", m, k, group_size);
    if (st) return st;
    Projs P;
    P.count = 1;
    P.qw[0] = q_proj->qweight; P.sc[0] = q_proj->scales; P.zr[0] = q_proj->zeros; P.out[0] = q_proj->out;
    P.n[0] = q_proj->n;
    P.wstart[0] = 0;
    uint64_t wtotal = q_proj->n / 8;
    if (k_proj) {
        st = check_proj(fn, k_proj, "k", m, k, group_size);
        if (st) return st;
        st = check_proj(fn, v_proj, "v", m, k, group_size);
        if (st) return st;
        if (k_proj->n != v_proj->n)
            return fail(KVQ_E_INVALID, "%s: k and v projections differ in n (%u vs %u)", fn, k_proj->n, v_proj->n);
        const int4_awq_proj_t *kv[2] = {k_proj, v_proj};
        for (int i = 0; i < 2; ++i) {
            P.qw[i + 1] = kv[i]->qweight; P.sc[i + 1] = kv[i]->scales; P.zr[i + 1] = kv[i]->zeros;
            P.out[i + 1] = kv[i]->out; P.n[i + 1] = kv[i]->n;
            P.wstart[i + 1] = (uint32_t)wtotal;
            wtotal += kv[i]->n / 8;
        }
        P.count = 3;
    } else {
        for (int i = 1; i < 3; ++i) {
            P.qw[i] = P.qw[0]; P.sc[i] = P.sc[0]; P.zr[i] = P.zr[0]; P.out[i] = P.out[0];
            P.n[i] = 0; P.wstart[i] = (uint32_t)wtotal;
        }
    }
    if (wtotal > 0x0FFFFFFFull) return fail(KVQ_E_INVALID, "%s: total n too large", fn);
    P.wtotal = (uint32_t)wtotal;

    Plan pl = make_plan(m, k, group_size, P.wtotal);
    uint32_t *counters = nullptr;
    float *partials = nullptr;
    if (pl.ks_b > 1) {
        if (!workspace || workspace_bytes < pl.counter_bytes + pl.partial_bytes || !aligned16(workspace)) {
            pl.ks_b = 1;   // no (or too small) workspace: one workgroup per tile
        } else {
            counters = static_cast<uint32_t *>(workspace);
            partials = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pl.counter_bytes);
        }
    }
    const uint64_t blocks = (uint64_t)pl.ntiles * pl.nchunks * pl.ks_b;
    if (blocks > 0x7FFFFFFFull) return fail(KVQ_E_INVALID, "%s: problem too large", fn);
    hipStream_t s = as_stream(stream);
    const uint32_t ksg = group_size / 32;
#define KVQ_AWQ(MT, R, KSG) \
    awq_gemm<MT, R, KSG><<<(unsigned)blocks, kBlock, 0, s>>>(x, m, k, P, pl.nchunks, pl.ks_b, counters, partials)
#define KVQ_AWQ_K(MT, R)                     \
    switch (ksg) {                           \
        case 1: KVQ_AWQ(MT, R, 1); break;    \
        case 2: KVQ_AWQ(MT, R, 2); break;    \
        case 4: KVQ_AWQ(MT, R, 4); break;    \
        default: KVQ_AWQ(MT, R, 8); break;   \
    }
    if (pl.mt == 1) {
        if (m == 1) KVQ_AWQ_K(1, 1)
        else KVQ_AWQ_K(1, 4)
    } else {
        KVQ_AWQ_K(2, 4)
    }
#undef KVQ_AWQ_K
#undef KVQ_AWQ
    return launch_status(fn);
}
