// INT4 AWQ weight-only GEMV/GEMM with the fused Q/K/V layout, for gfx950.
//
// Follows boostr fused_int4_qkv.rs: QKV_AWQ_SHIFTS / unpack_awq_qkv (column j
// of an 8-column u32 word is the nibble at bit SHIFTS[j], SHIFTS = 0, 16, 4,
// 20, 8, 24, 12, 28) and fused_int4_qkv_q / _k / _v (out[m][j] = sum_k
// x[m][k] * (q - zero[k/gs][j]) * scale[k/gs][j], weights [K][n/8], fp32
// scales and zeros [K/gs][n]).  The page runs three dispatches of one thread
// per output with a serial K loop; here Q, K and V are one launch, and the
// sums run on the matrix cores:
//
//   out = sum_g s_g * (P_g - z_g * X_g),  P_g = sum_{k in g} x~_k * q_k,
//                                          X_g = sum_{k in g} x~_k
//
// with x~ = fp16(x) (round to nearest even) and the codes q exact, so P_g and
// X_g come from v_mfma_f32_16x16x32_f16 (X_g with an all-ones B operand) and
// the only rounding of the inputs is the activation's.  s and z are applied
// per group in fp32.
//
// Code unpacking costs one AND per two codes: the fp16 bit pattern q (0..15)
// is the subnormal q * 2^-24, exact, and the matrix cores multiply fp16
// subnormals exactly; a nibble sitting 4 bits higher reads as q * 2^-20.  The
// powers of two go into the per-group epilogue: s * (P - z X) =
// (s * 2^24) * (P' - (z * 2^-24) X) with P' the MFMA sum of x~ * q * 2^-24.
// v_perm_b32 first pairs the bytes of K rows k and k+1 of one word column so
// that each 16-bit half holds the same column's nibble from the two rows: the
// even columns of a word live in its bytes 0-1, the odd ones in bytes 2-3.
//
// Layout of the work (16 rows and more, awq_ring): one wave owns 16 word
// columns (128 output columns) of one projection, a chunk of 16 or 32
// activation rows, and a run of whole quantization groups.  Lane (wc = l % 16,
// kg = l / 16) supplies word column wc and K rows 8*kg .. 8*kg+7 of each
// 32-wide K step; MFMA number c computes output columns 8*wc + c.  The
// activation operand holds x~[m][8*kg .. 8*kg+7] in the same K order.  The
// waves of a workgroup take consecutive runs of groups of the same tile and
// add their sums in LDS; when more K slices are needed to fill the GPU,
// workgroups exchange fp32 partial tiles through the caller's workspace with
// device-scope (sc1) stores and loads, which bypass the per-XCD L2s that are
// not coherent with each other, and an agent-scope counter; the last
// workgroup of a tile adds them in slice order and resets the counter.
// Below 16 rows the products run on the vector ALUs (awq_gemv, further down).
#include "kvq_common.h"

#include <mutex>
#include <type_traits>

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr uint32_t kXcds = 8;           // XCDs of an MI355X (workgroups are dealt to them in turn)

struct Projs {
    const uint32_t *qw[3];
    const float *sc[3];
    const float *zr[3];
    float *out[3];
    uint32_t n[3];        // output columns of each projection
    uint32_t tstart[3];   // first 16-word-column tile of each projection
    uint32_t count;
    uint32_t ntiles;
};


// 8 words (K rows 0..7 of one word column) -> 8 B operands; operand c holds
// column c's codes (as fp16 subnormals, scaled 2^-24 or 2^-20) for rows 0..7,
// row 2i in the low half of register i.
__device__ __forceinline__ void awq_operands(const uint32_t w[8], f16x8 B[8]) {
    uint32_t r[8][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ev = __builtin_amdgcn_perm(w[2 * i + 1], w[2 * i], 0x05040100u);
        const uint32_t od = __builtin_amdgcn_perm(w[2 * i + 1], w[2 * i], 0x07060302u);
        const uint32_t ev8 = ev >> 8, od8 = od >> 8;
        r[0][i] = ev & 0x000F000Fu;    // column 0, scale 2^-24
        r[2][i] = ev & 0x00F000F0u;    // column 2, scale 2^-20
        r[4][i] = ev8 & 0x000F000Fu;   // column 4
        r[6][i] = ev8 & 0x00F000F0u;   // column 6
        r[1][i] = od & 0x000F000Fu;    // column 1
        r[3][i] = od & 0x00F000F0u;    // column 3
        r[5][i] = od8 & 0x000F000Fu;   // column 5
        r[7][i] = od8 & 0x00F000F0u;   // column 7
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const u32x4 v = {r[c][0], r[c][1], r[c][2], r[c][3]};
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

__device__ __forceinline__ f32x4 as_f32x4(u32x4 v) { return __builtin_bit_cast(f32x4, v); }

// Activation formats: XT 0 fp32 (two 16-byte loads per 8 values), 1 fp16
// (one load; the values go to the matrix cores unchanged), 2 bf16 (one load;
// widened exactly, then rounded to fp16 like fp32 input).
template <int XT>
__device__ __forceinline__ f16x8 act_f16x8(const u32x4 &lo, const u32x4 &hi) {
    if (XT == 0) return to_f16x8(as_f32x4(lo), as_f32x4(hi));
    if (XT == 1) return __builtin_bit_cast(f16x8, lo);
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[2 * i] = (_Float16)__uint_as_float(lo[i] << 16);
        h[2 * i + 1] = (_Float16)__uint_as_float(lo[i] & 0xFFFF0000u);
    }
    return h;
}

// The same 8 values as fp32 (fp32 as is, bf16 widened exactly), for the
// per-row power-of-two scaling (XT 0 and 2).
template <int XT>
__device__ __forceinline__ void act_f32x8(const u32x4 &lo, const u32x4 &hi, float v[8]) {
    if (XT == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = __uint_as_float(lo[j]);
            v[4 + j] = __uint_as_float(hi[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(lo[j] << 16);
            v[2 * j + 1] = __uint_as_float(lo[j] & 0xFFFF0000u);
        }
    }
}

// x * 2^e rounded to fp16 (nearest even); the product by a power of two is exact
template <int XT>
__device__ __forceinline__ f16x8 act_f16x8_scaled(const u32x4 &lo, const u32x4 &hi, int e) {
    float v[8];
    act_f32x8<XT>(lo, hi, v);
    f16x8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = (_Float16)__builtin_ldexpf(v[j], e);
    return h;
}

// The exponent E that puts a row's absmax (as non-negative float bits) into
// [2^14, 2^15): 0 for zero rows and rows holding inf or NaN, else clamped to
// +-126 so that 2^-E stays a normal float.
__device__ __forceinline__ int row_pow2(int amax_bits) {
    if (amax_bits == 0 || amax_bits >= 0x7F800000) return 0;
    int ex;
    (void)__builtin_frexpf(__int_as_float(amax_bits), &ex);   // absmax in [2^(ex-1), 2^ex)
    const int e = 15 - ex;
    return e < -126 ? -126 : (e > 126 ? 126 : e);
}

// ------------------------------------------ activation pre-scaling ---
//
// From 16 rows the matrix cores take fp16 activations.  fp16 keeps 11 bits
// only between 2^-14 and 65504: a row of tiny values (|x| ~ 1e-6) would keep
// a few bits and a row past 65504 would become inf.  So fp32 (and bf16) rows
// are scaled by a power of two 2^E_m that puts the row's absmax into
// [2^14, 2^15) and rounded to fp16 (nearest even) once, into the workspace;
// the product kernel reads that copy and multiplies each output row by
// 2^-E_m, which is exact.  The sums are linear in x, so the result is the
// same as with unscaled activations, except that every term now keeps 2^-11
// relative precision.  One workgroup per row: an absmax pass, then the scaled
// conversion (the row is read again from L2).  Rows that are zero or hold inf
// or NaN keep E = 0 (inf and NaN then reach the outputs as they would).
template <int XT>
__global__ __launch_bounds__(256) void x_pow2_f16(const void *__restrict__ x, uint32_t K, f16x8 *__restrict__ y,
                                                  float *__restrict__ inv_scale) {
    constexpr uint32_t XB = XT == 0 ? 4 : 2;
    __shared__ int wmax[4];
    const uint32_t m = blockIdx.x;
    const uint32_t n8 = K / 8;
    const rsrc_t rx = make_rsrc(static_cast<const uint8_t *>(x) + (size_t)m * K * XB, K * XB);
    // 8 values from the 16 or 32 bytes at 8-value chunk i (an offset past the
    // row reads zeros)
    auto raw8 = [&](uint32_t i, u32x4 r[2]) {
        const uint32_t off = i < n8 ? i * 8 * XB : kOffNone;
        r[0] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
        r[1] = XT == 0 ? __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, 0) : r[0];
    };
    auto unpack8 = [&](const u32x4 r[2], float v[8]) {
        if (XT == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[q] = __uint_as_float(r[0][q]);
                v[4 + q] = __uint_as_float(r[1][q]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[2 * q] = __uint_as_float(r[0][q] << 16);
                v[2 * q + 1] = __uint_as_float(r[0][q] & 0xFFFF0000u);
            }
        }
    };
    auto load8 = [&](uint32_t i, float v[8]) {
        u32x4 r[2];
        raw8(i, r);
        unpack8(r, v);
    };
    // absmax over the row (non-negative floats, inf and NaN included, order
    // as their bits); rows up to 8192 values stay in registers for the
    // conversion (every load issued before the first use, no branch around
    // them), longer ones are read again (from L2)
    constexpr int NR = 4;   // 8-value chunks per thread kept in registers
    const bool held = n8 <= NR * 256;
    float v[NR][8];
    int amax = 0;
    if (held) {
        u32x4 r[NR][2];
#pragma unroll
        for (int j = 0; j < NR; ++j) raw8(threadIdx.x + 256 * j, r[j]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            unpack8(r[j], v[j]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int b = __float_as_int(v[j][q]) & 0x7FFFFFFF;
                amax = b > amax ? b : amax;
            }
        }
    } else {
        for (uint32_t i = threadIdx.x; i < n8; i += 256) {
            float u[8];
            load8(i, u);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int b = __float_as_int(u[q]) & 0x7FFFFFFF;
                amax = b > amax ? b : amax;
            }
        }
    }
    amax = team_ext<64, true>(amax);
    if (lane_id() == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) amax = wmax[w] > amax ? wmax[w] : amax;
    const int e = row_pow2(amax);
    if (threadIdx.x == 0) inv_scale[m] = __builtin_ldexpf(1.0f, -e);
    auto store8 = [&](uint32_t i, const float *u) {
        f16x8 h;
#pragma unroll
        for (int q = 0; q < 8; ++q) h[q] = (_Float16)__builtin_ldexpf(u[q], e);
        y[(size_t)m * n8 + i] = h;
    };
    if (held) {
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const uint32_t i = threadIdx.x + 256 * j;
            if (i < n8) store8(i, v[j]);
        }
    } else {
        for (uint32_t i = threadIdx.x; i < n8; i += 256) {
            float u[8];
            load8(i, u);
            store8(i, u);
        }
    }
}

// ------------------------------------------------ matrix-core ring ---
//
// 16 rows and more: P_g and X_g on the matrix cores, s and z per group in
// fp32, codes unpacked by awq_operands, with every wave streaming its own K range through a private ring of R LDS
// stages, filled by direct-to-LDS loads (buffer_load ... lds).  A stage is KB
// rows of K: the tile's 16 weight words of each row (KB x 64 bytes), the
// chunk's MR activation rows over those KB columns, and, on the last stage of
// a quantization group, the group's 128 scales and 128 zeros.  The wave
// issues R stages, then per stage waits for exactly that stage (loads return
// in order, so vmcnt <= L * stages issued after it), reads it into registers,
// refills the slot with stage +R and multiplies while the loads fly.  No
// barrier is needed until the waves of the workgroup add their sums, so
// R stages of every wave are always in flight without holding registers.
//
// LDS layouts, chosen so that the reads of a fragment are free of bank
// conflicts:
//  * weights: the 32 rows of a K step are stored in the order 4i + kg for
//    row 8kg + i, so word i of the lanes (wc, kg) lies in 4 consecutive 64-byte
//    rows: one 256-byte line per read, every lane a different bank;
//  * activations: row m of the stage holds its 16-byte chunks with chunk c at
//    slot c ^ swz(m), swz(m) = (m / RPB) mod CPR (CPR chunks per row, RPB rows
//    per 256 bytes), so the 16 rows read at the same K offset fall into 16
//    different 16-byte bank groups.
template <int MT, int XT, int KB, int R, int WV>
struct RingCfg {
    static constexpr int MR = 16 * MT;
    static constexpr int XB = XT == 0 ? 4 : 2;
    static constexpr int SUB = KB / 32;            // 32-wide K steps per stage
    static constexpr int W_BYTES = KB * 64;        // KB rows x 16 words
    static constexpr int X_ROW = KB * XB;          // one activation row of a stage
    static constexpr int X_BYTES = MR * X_ROW;
    static constexpr int CPR = X_ROW / 16;
    static constexpr int RPB = 16 / CPR;
    static constexpr int W_INSTR = W_BYTES / 1024;
    static constexpr int X_INSTR = X_BYTES / 1024;
    static constexpr int SZ_INSTR = 4;             // scales, zeros: 2 x 256-byte loads each
    static constexpr int L = W_INSTR + X_INSTR + SZ_INSTR;   // loads per stage
    static constexpr int STAGE = W_BYTES + X_BYTES + 1024;
    static constexpr int WAVE_BYTES = R * STAGE;
    static_assert(KB == 32 || KB == 64, "stage rows");
    static constexpr int SUMS = WV * 16 * 32 * 16;   // the waves' sums, stored over the ring at the end
    static constexpr int LDS = (WV * WAVE_BYTES > SUMS + 16 ? WV * WAVE_BYTES : SUMS + 16);
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert(L * (R - 1) < 64, "vmcnt range");
    static_assert(X_BYTES % 1024 == 0 && CPR >= 4 && CPR <= 16, "stage shape");
};

// wait until at most `later` stages of L loads are in flight
template <int L, int MAXL>
__device__ __forceinline__ void ring_wait(int later) {
    if constexpr (MAXL >= 3) {
        if (later >= 3) { wait_vm<3 * L>(); return; }
    }
    if constexpr (MAXL >= 2) {
        if (later == 2) { wait_vm<2 * L>(); return; }
    }
    if constexpr (MAXL >= 1) {
        if (later == 1) { wait_vm<L>(); return; }
    }
    wait_vm<0>();
}

template <int MT, int XT, int KB, int R, int WV>
__global__ __launch_bounds__(WV * kWave) void awq_ring(const void *__restrict__ x, uint32_t M, uint32_t K,
                                                      uint32_t gs, Projs P, uint32_t nchunks, uint32_t ks_b,
                                                      uint32_t *__restrict__ counters, float *__restrict__ partials,
                                                      const float *__restrict__ rscale, int inscale) {
    using C = RingCfg<MT, XT, KB, R, WV>;
    constexpr int MR = C::MR;
    constexpr int NTH = WV * kWave;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[C::LDS];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wc = lane & 15, kg = lane >> 4;

    // Tile, row chunk and K slice of this workgroup.  Workgroups go to the
    // XCDs in turn (index mod kXcds), each XCD with its own L2.  A tile's rows
    // of weights are 64-byte runs, so tiles 2p and 2p+1 of a projection share
    // every 128-byte line: the pair is placed on one XCD (dispatched
    // together), which fetches each line from HBM once instead of twice.
    // With several row chunks, all workgroups of a pair sit on the XCD of
    // index p mod kXcds (the chunks re-read the same weights); with one
    // chunk, the pair's workgroups of K slice bs go to XCD (p*ks_b + bs) mod
    // kXcds, so each XCD's L2 holds few K slices of the activations.  Slots
    // past the last tile exit at once.
    const uint32_t per_tile = nchunks * ks_b;
    const uint32_t npairs = (P.ntiles + 1) / 2;
    const uint32_t xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    uint32_t pair, h, r;
    if (nchunks > 1) {
        pair = xcd + kXcds * (j / (2 * per_tile));
        const uint32_t rr = j % (2 * per_tile);
        h = rr % 2;
        r = rr / 2;
    } else {
        h = j % 2;
        const uint32_t g = kXcds * (j / 2) + xcd;
        pair = g / ks_b;
        r = g % ks_b;
    }
    const uint32_t t = 2 * pair + h;
    if (pair >= npairs || t >= P.ntiles) return;
    const uint32_t c = r / ks_b, bs = r % ks_b;
    const int p = (P.count > 1 && t >= P.tstart[1]) ? ((P.count > 2 && t >= P.tstart[2]) ? 2 : 1) : 0;
    const uint32_t np = pick(p, P.n[0], P.n[1], P.n[2]), wp = np / 8;
    const uint32_t tp = t - pick(p, P.tstart[0], P.tstart[1], P.tstart[2]);

    // this wave's whole groups [g0, g1) and its stages
    const uint32_t ngroups = K / gs;
    const uint32_t nwaves = ks_b * WV, u = bs * WV + wv;
    const uint32_t g0 = (uint32_t)((uint64_t)u * ngroups / nwaves);
    const uint32_t g1 = (uint32_t)((uint64_t)(u + 1) * ngroups / nwaves);
    const uint32_t spg = gs / KB;                      // stages per group
    const int nst = (int)((g1 - g0) * spg);
    const uint32_t krow0 = g0 * gs;

    // buffer resources and the per-lane halves of the load offsets
    const u32x4 rw = buffer_rsrc(pick(p, P.qw[0], P.qw[1], P.qw[2]), K * wp * 4);
    const u32x4 rx = buffer_rsrc(x, M * K * C::XB);
    const uint32_t szb = ngroups * np * 4;
    const u32x4 rs = buffer_rsrc(pick(p, P.sc[0], P.sc[1], P.sc[2]), szb);
    const u32x4 rz = buffer_rsrc(pick(p, P.zr[0], P.zr[1], P.zr[2]), szb);
    uint32_t w_off[C::W_INSTR];
#pragma unroll
    for (int j = 0; j < C::W_INSTR; ++j) {
        const int rho = 16 * (j & 1) + (lane >> 2);
        const uint32_t row = 32 * (j >> 1) + 8 * (rho & 3) + (rho >> 2);
        w_off[j] = row * wp * 4 + (tp * 16 + 4 * (lane & 3)) * 4;   // past the row: unused columns
    }
    uint32_t x_off[C::X_INSTR];
#pragma unroll
    for (int j = 0; j < C::X_INSTR; ++j) {
        const int e = j * 64 + lane;
        const int ml = e / C::CPR, cs = e % C::CPR;
        const int ch = cs ^ ((ml / C::RPB) & (C::CPR - 1));
        const uint32_t m = c * MR + ml;
        x_off[j] = m < M ? m * K * C::XB + ch * 16 : kOffNone;   // rows past M read zeros
    }
    const uint32_t sz_off = (tp * 128 + lane) * 4;

    const uint32_t ring0 = lds_offset(ring) + wv * C::WAVE_BYTES;
    auto issue = [&](int b) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(ring0 + (uint32_t)(b % R) * C::STAGE);
        const uint32_t k0 = krow0 + (uint32_t)b * KB;
        const uint32_t sw = __builtin_amdgcn_readfirstlane(k0 * wp * 4);
        const uint32_t sx = __builtin_amdgcn_readfirstlane(k0 * C::XB);
#pragma unroll
        for (int j = 0; j < C::W_INSTR; ++j) lds_buf16(rw, w_off[j], sw, base + j * 1024);
#pragma unroll
        for (int j = 0; j < C::X_INSTR; ++j) lds_buf16(rx, x_off[j], sx, base + C::W_BYTES + j * 1024);
        // scales and zeros of the group, on its last stage only (other
        // stages issue the same loads out of range: no traffic, same count)
        const bool gend = ((uint32_t)b + 1) % spg == 0;
        const uint32_t g = g0 + (uint32_t)b / spg;
        const uint32_t ss = __builtin_amdgcn_readfirstlane(g * np * 4);
        const uint32_t o = gend ? sz_off : kOffNone;
        const uint32_t sz0 = base + C::W_BYTES + C::X_BYTES;
        lds_buf4(rs, o, ss, sz0);
        lds_buf4(rs, gend ? sz_off + 256 : kOffNone, ss, sz0 + 256);
        lds_buf4(rz, o, ss, sz0 + 512);
        lds_buf4(rz, gend ? sz_off + 256 : kOffNone, ss, sz0 + 768);
    };

    f32x4 acc[MT][8], pg[MT][8], xg[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        xg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) acc[mt][cc] = pg[mt][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;

    for (int b = 0; b < R && b < nst; ++b) issue(b);
    // Per-row power-of-two scaling inside the wave (fp32 and bf16 input, when
    // the wave's whole K range fits in its ring, nst <= R): every stage has
    // been issued, so wait for all of them, take each of the wave's rows'
    // absmax over its K range, and scale the activations by 2^E into fp16
    // below; the wave's sums are multiplied by 2^-E per output row at the
    // end (exact).  Lane (wc, kg) holds row mt*16+wc; its 4 K quarters are
    // lanes 16 apart.
    int erow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) erow[mt] = 0;
    if (XT != 1 && inscale) {
        wait_vm<0>();
        asm volatile("" ::: "memory");
        int amax[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) amax[mt] = 0;
        for (int b = 0; b < nst; ++b) {
            const uint8_t *st = ring + wv * C::WAVE_BYTES + (b % R) * C::STAGE;
#pragma unroll
            for (int s = 0; s < C::SUB; ++s) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int ml = mt * 16 + wc;
                    const int swz = (ml / C::RPB) & (C::CPR - 1);
                    const uint8_t *xr = st + C::W_BYTES + ml * C::X_ROW;
                    u32x4 lo, hi;
                    if (XT == 0) {
                        const int c0 = 8 * s + 2 * kg;
                        lo = *reinterpret_cast<const u32x4 *>(xr + ((c0 ^ swz) << 4));
                        hi = *reinterpret_cast<const u32x4 *>(xr + (((c0 + 1) ^ swz) << 4));
                    } else {
                        lo = *reinterpret_cast<const u32x4 *>(xr + (((4 * s + kg) ^ swz) << 4));
                        hi = lo;
                    }
                    float v[8];
                    act_f32x8<XT>(lo, hi, v);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int bits = __float_as_int(v[q]) & 0x7FFFFFFF;
                        amax[mt] = bits > amax[mt] ? bits : amax[mt];
                    }
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            int a = amax[mt];
            auto r32 = __builtin_amdgcn_permlane32_swap((uint32_t)a, (uint32_t)a, false, false);
            a = (int)r32[0] > (int)r32[1] ? (int)r32[0] : (int)r32[1];
            auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)a, (uint32_t)a, false, false);
            a = (int)r16[0] > (int)r16[1] ? (int)r16[0] : (int)r16[1];
            erow[mt] = row_pow2(a);
        }
    }
    for (int b = 0; b < nst; ++b) {
        const int later = (nst - b < R ? nst - b : R) - 1;
        ring_wait<C::L, R - 1>(later);
        asm volatile("" ::: "memory");
        const uint8_t *st = ring + wv * C::WAVE_BYTES + (b % R) * C::STAGE;
        uint32_t w[C::SUB][8];
        u32x4 xv[C::SUB][MT][2];
#pragma unroll
        for (int s = 0; s < C::SUB; ++s) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                w[s][i] = *reinterpret_cast<const uint32_t *>(st + s * 2048 + (4 * i + kg) * 64 + wc * 4);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int ml = mt * 16 + wc;
                const int swz = (ml / C::RPB) & (C::CPR - 1);
                const uint8_t *xr = st + C::W_BYTES + ml * C::X_ROW;
                if (XT == 0) {
                    const int c0 = 8 * s + 2 * kg;
                    xv[s][mt][0] = *reinterpret_cast<const u32x4 *>(xr + ((c0 ^ swz) << 4));
                    xv[s][mt][1] = *reinterpret_cast<const u32x4 *>(xr + (((c0 + 1) ^ swz) << 4));
                } else {
                    xv[s][mt][0] = *reinterpret_cast<const u32x4 *>(xr + (((4 * s + kg) ^ swz) << 4));
                    xv[s][mt][1] = xv[s][mt][0];
                }
            }
        }
        const bool gend = ((uint32_t)b + 1) % spg == 0;
        f32x4 s0, s1, z0, z1;
        if (gend) {
            const uint8_t *sz = st + C::W_BYTES + C::X_BYTES;
            s0 = *reinterpret_cast<const f32x4 *>(sz + 32 * wc);
            s1 = *reinterpret_cast<const f32x4 *>(sz + 32 * wc + 16);
            z0 = *reinterpret_cast<const f32x4 *>(sz + 512 + 32 * wc);
            z1 = *reinterpret_cast<const f32x4 *>(sz + 512 + 32 * wc + 16);
        }
        // the slot's reads are done: refill it while this stage is multiplied
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (b + R < nst) issue(b + R);
        // A group's first K step starts its sums from a zero accumulator, so
        // its epilogue need not clear them (~70 vector instructions per group
        // at 32 rows).  bf16 input keeps the clearing: its extra widening
        // leaves no registers for the second copy of this step.
        constexpr bool kZeroStart = XT != 2;
        auto multiply = [&](auto fresh) {
#pragma unroll
            for (int s = 0; s < C::SUB; ++s) {
                f16x8 B[8];
                awq_operands(w[s], B);
                const bool z = decltype(fresh)::value && s == 0;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f16x8 a = (XT != 1 && inscale)
                                        ? act_f16x8_scaled<XT>(xv[s][mt][0], xv[s][mt][1], erow[mt])
                                        : act_f16x8<XT>(xv[s][mt][0], xv[s][mt][1]);
                    xg[mt] = mfma16(a, ones, z ? f32x4{0.f, 0.f, 0.f, 0.f} : xg[mt]);
#pragma unroll
                    for (int cc = 0; cc < 8; ++cc)
                        pg[mt][cc] = mfma16(a, B[cc], z ? f32x4{0.f, 0.f, 0.f, 0.f} : pg[mt][cc]);
                }
            }
        };
        if (kZeroStart && (uint32_t)b % spg == 0) multiply(std::true_type{});
        else multiply(std::false_type{});
        if (gend) {
            // columns 0,1,4,5 were unpacked as q*2^-24, columns 2,3,6,7 as q*2^-20
            const float f[8] = {0x1p24f, 0x1p24f, 0x1p20f, 0x1p20f, 0x1p24f, 0x1p24f, 0x1p20f, 0x1p20f};
            const float sv[8] = {s0.x * f[0], s0.y * f[1], s0.z * f[2], s0.w * f[3],
                                 s1.x * f[4], s1.y * f[5], s1.z * f[6], s1.w * f[7]};
            const float zv[8] = {z0.x / f[0], z0.y / f[1], z0.z / f[2], z0.w / f[3],
                                 z1.x / f[4], z1.y / f[5], z1.z / f[6], z1.w / f[7]};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[mt][cc][i] = __builtin_fmaf(sv[cc], __builtin_fmaf(-zv[cc], xg[mt][i], pg[mt][cc][i]),
                                                        acc[mt][cc][i]);
                    if (!kZeroStart) pg[mt][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                if (!kZeroStart) xg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    // Waves -> LDS (the ring's memory, once every wave is done with it), one
    // 16-row tile at a time, as [row][column] with row = 4*kg + i and column
    // = 8*wc + cc; then the threads add the waves' values in wave order and
    // write 16-byte pieces of the output (or partial) rows.
    __syncthreads();
    f32x4(*red)[16][32] = reinterpret_cast<f32x4(*)[16][32]>(ring);
    int *s_last = reinterpret_cast<int *>(ring + C::SUMS);
    const uint32_t tile_id = t * nchunks + c;
    float *part = partials + (size_t)tile_id * ks_b * (MR * 128);
    const rsrc_t rp = make_rsrc(part, ks_b * (MR * 128) * 4);
    float *outp = pick(p, P.out[0], P.out[1], P.out[2]);
    // activations scaled by 2^E per row inside the wave: undo it on the lane's
    // output rows 4kg..4kg+3, whose exponents lanes 4kg..4kg+3 hold
    if (XT != 1 && inscale) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 sc;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sc[i] = __builtin_ldexpf(1.0f, -__builtin_amdgcn_ds_bpermute((4 * kg + i) * 4, erow[mt]));
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) acc[mt][cc] *= sc;
        }
    }
    // activations pre-scaled by 2^E per row: undo it (exact) on the lane's output rows
    if (rscale) {
        const rsrc_t rr = make_rsrc(rscale, M * 4);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 sc = as_f32x4(__builtin_amdgcn_raw_buffer_load_b128(rr, (c * MR + mt * 16 + 4 * kg) * 4, 0, 0));
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) acc[mt][cc] *= sc;   // rows past M: zero sums times zero
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * kg + i;
            red[wv][row][2 * wc] = f32x4{acc[mt][0][i], acc[mt][1][i], acc[mt][2][i], acc[mt][3][i]};
            red[wv][row][2 * wc + 1] = f32x4{acc[mt][4][i], acc[mt][5][i], acc[mt][6][i], acc[mt][7][i]};
        }
        __syncthreads();
        for (int e = threadIdx.x; e < 16 * 32; e += NTH) {
            const int row = e >> 5, col4 = e & 31;
            const uint32_t m = c * MR + mt * 16 + row;
            const uint32_t lwo = tp * 16 + (col4 >> 1);
            if (m >= M || lwo >= wp) continue;
            f32x4 v = red[0][row][col4];
#pragma unroll
            for (int w2 = 1; w2 < WV; ++w2) v += red[w2][row][col4];
            if (ks_b == 1) {
                *reinterpret_cast<f32x4 *>(outp + (size_t)m * np + 8 * lwo + (col4 & 1) * 4) = v;
            } else {
                const uint32_t off = ((bs * MR + mt * 16 + row) * 128 + col4 * 4) * 4;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp, off, 0, kAuxSc1);
            }
        }
        __syncthreads();
    }
    if (ks_b == 1) return;

    // cross-workgroup K reduction: every thread's device-scope stores have
    // completed before the barrier, so they are visible at the coherence
    // point before the counter moves; the last workgroup's device-scope loads
    // are issued after it has seen the count
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&counters[tile_id], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        *s_last = prev == ks_b - 1;
    }
    __syncthreads();
    if (!*s_last) return;
    for (int e = threadIdx.x; e < MR * 32; e += NTH) {
        const int row = e >> 5, col4 = e & 31;
        const uint32_t m = c * MR + row;
        const uint32_t lwo = tp * 16 + (col4 >> 1);
        if (m >= M || lwo >= wp) continue;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (uint32_t q0 = 0; q0 < ks_b; q0 += 8) {
            u32x4 tq[8];
#pragma unroll
            for (int uu = 0; uu < 8; ++uu) {
                const uint32_t q = q0 + uu;
                const uint32_t off = q < ks_b ? ((q * MR + row) * 128 + col4 * 4) * 4 : kOffNone;
                tq[uu] = __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, kAuxSc1);
            }
#pragma unroll
            for (int uu = 0; uu < 8; ++uu)
                if (q0 + uu < ks_b) v += as_f32x4(tq[uu]);
        }
        *reinterpret_cast<f32x4 *>(outp + (size_t)m * np + 8 * lwo + (col4 & 1) * 4) = v;
    }
    if (threadIdx.x == 0) __hip_atomic_store(&counters[tile_id], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------- fp32 GEMV ---
//
// Below 16 rows the products run on the vector ALUs in fp32, as the page's
// kernel does (x is never rounded): a weight-streaming GEMV.  A workgroup
// owns a tile of 256 output columns of one projection; each of its GW waves
// takes whole blocks of rows of it.  Lane (cl, kl) of a wave covers
// CPL consecutive columns (CPL/8 words of every weight row: one 16-, 8- or
// 4-byte load per row, so the CL = 256/CPL column lanes of a row read 128
// contiguous bytes) and RPL = gs/KL consecutive rows of the group, KL =
// 64/CL lanes splitting the group's rows.  Codes are unpacked in registers:
// (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) hold the 8 nibbles of a word
// as bytes, which v_cvt_f32_ubyte0..3 turn into exact floats; byte b of the
// low part is the nibble at bit 8b (column 0, 4, 1, 5 of the word in AWQ
// order), of the high part the nibble at bit 8b+4 (columns 2, 6, 3, 7).
//
// Per group g the lane forms P[m][c] = sum_k x[m][k] q[k][c] and X[m] =
// sum_k x[m][k] over its rows (fp32 FMAs, x staged once per group in LDS);
// the KL partial sums of a column are combined by a reduce-scatter over the
// lanes (v_permlane32_swap, v_permlane16_swap, then DPP row_ror:8), which
// leaves every lane 4 columns, and the lane adds s (P - z X) for them.  That
// is the page's sum of x (q - z) s regrouped per group (the scale and zero are
// constant over a group); every product and sum stays fp32.
//
// The waves of a workgroup are added in LDS in wave order; when a tile's
// groups are split over several workgroups ("slices"), their fp32 partial
// tiles are exchanged through the workspace with device-scope stores and
// loads and an agent-scope counter, and the last workgroup adds them in
// slice order (deterministic) and resets the counter.
constexpr uint32_t kGemvTile = 256;   // output columns per workgroup

// s_waitcnt vmcnt(N) with N a template constant (gfx9 encoding)
template <int N>
__device__ __forceinline__ void gemv_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// v_permlane32_swap / v_permlane16_swap based halving of a set of 2H values:
// lanes with the given bit clear keep the sums of the first H values over
// the lane pair, lanes with it set the sums of the second H.
template <int H, int BIT>
__device__ __forceinline__ void halve(float *v) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
        if (BIT == 5) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + H]), false,
                                                            false);
            v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        } else if (BIT == 4) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + H]), false,
                                                            false);
            v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        } else {
            // lanes 8 apart inside a row of 16: row_ror:8 brings the partner's value
            const bool hi = (lane_id() & 8) != 0;
            const float keep = hi ? v[i + H] : v[i];
            const float send = hi ? v[i] : v[i + H];
            v[i] = keep + dpp_move<0x128>(send);
        }
    }
}

// Sum over the KL lanes that share a column set (lane bits 3..5 above the
// column-lane bits): all-reduce, every lane gets the same bits.
template <int KL>
__device__ __forceinline__ float klane_sum(float v) {
    if (KL >= 8) v += dpp_move<0x128>(v);
    if (KL >= 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if (KL >= 2) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}

// CPL: columns per lane (32, 16 or 8).  MR: activation rows the accumulators
// are built for (M <= MR), taken MRP at a time over the codes held in
// registers.  RB: rows per block, min(group size, 128): a wave takes whole
// blocks, and a group of 256 rows is two blocks with the same scale and
// zero (s (P - z X) is linear in P and X, so the blocks add).  gs (run
// time): group size.  xt (run time): activation format (0 fp32, 1 fp16,
// 2 bf16; 16-bit values are widened exactly).
template <int CPL, int MR, int MRP, int RB, int GW>
__global__ __launch_bounds__(GW * kWave) void awq_gemv(const void *__restrict__ x, uint32_t M, uint32_t K,
                                                              uint32_t gs, int xt, Projs P, uint32_t slices,
                                                              uint32_t gpw,
                                                              uint32_t *__restrict__ counters,
                                                              float *__restrict__ partials) {
    constexpr int CL = (int)kGemvTile / CPL;     // column lanes
    constexpr int KL = kWave / CL;               // lanes splitting a group's rows
    constexpr int RPL = RB / KL;                 // rows per lane per block
    constexpr int WPL = CPL / 8;                 // words per lane per row
    constexpr int NW = RPL * WPL;                // words per lane per group
    static_assert(KL >= 2 && KL <= 8 && RPL >= 4 && RPL % 4 == 0, "lane layout");
    static_assert(NW <= 64 && MR % MRP == 0, "codes of a group per lane; row passes");
    __shared__ __attribute__((aligned(16))) float xs[GW][MR][RB];
    __shared__ __attribute__((aligned(16))) f32x4 red[GW][MR][kGemvTile / 4];
    __shared__ int s_last;
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cl = lane % CL, kl = lane / CL;

    const uint32_t t = blockIdx.x / slices, slice = blockIdx.x % slices;
    const int p = (P.count > 1 && t >= P.tstart[1]) ? ((P.count > 2 && t >= P.tstart[2]) ? 2 : 1) : 0;
    const uint32_t np = pick(p, P.n[0], P.n[1], P.n[2]), wp = np / 8;
    const uint32_t col0 = (t - pick(p, P.tstart[0], P.tstart[1], P.tstart[2])) * kGemvTile;
    const uint32_t lcol = col0 + cl * CPL;             // first column of this lane
    const bool cok = lcol < np;                        // n % CPL == 0: a lane is wholly in or out
    const uint32_t nblocks = K / RB, ngroups = K / gs;

    const uint32_t wbytes = K * wp * 4;
    const rsrc_t rw = make_rsrc(pick(p, P.qw[0], P.qw[1], P.qw[2]), wbytes);
    const uint32_t szbytes = ngroups * np * 4;
    const rsrc_t rs = make_rsrc(pick(p, P.sc[0], P.sc[1], P.sc[2]), szbytes);
    const rsrc_t rz = make_rsrc(pick(p, P.zr[0], P.zr[1], P.zr[2]), szbytes);
    const uint32_t xb = xt == 0 ? 4 : 2;
    const rsrc_t rx = make_rsrc(x, M * K * xb);

    // after the reduce-scatter a lane keeps columns cb .. cb+3 of its CPL
    const int cb = (CPL == 32 ? 16 * ((lane >> 5) & 1) + 8 * ((lane >> 4) & 1) + 4 * ((lane >> 3) & 1)
                              : (CPL == 16 ? 8 * ((lane >> 5) & 1) + 4 * ((lane >> 4) & 1) : 4 * ((lane >> 5) & 1)));

    float acc[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[m][c] = 0.0f;

    const uint32_t bbeg = (slice * GW + wv) * gpw;
    for (uint32_t bi = 0; bi < gpw; ++bi) {
        const uint32_t b = bbeg + bi;
        if (b >= nblocks) break;                            // wave-uniform
        const uint32_t g = b * RB / gs;                     // the block's quantization group
        // activation slab x[0..M)[b*RB .. +RB) -> this wave's LDS rows:
        // issued first, so its wait below does not hold the code loads
        constexpr int XV = RB / 4;                          // float4 per row
        constexpr int XL = (MR * XV + kWave - 1) / kWave;   // loads per lane
        u32x4 xv[XL];
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const uint32_t e = j * kWave + lane;            // float4 index in [MR][XV]
            const uint32_t m = e / XV, q4 = e % XV;
            const bool ok = m < M;
            if (xt == 0) {
                xv[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (m * K + b * RB + q4 * 4) * 4 : kOffNone, 0, 0);
            } else {
                const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(rx, ok ? (m * K + b * RB + q4 * 4) * 2 : kOffNone,
                                                                     0, 0);
                xv[j] = u32x4{h[0], h[1], 0u, 0u};
            }
        }
        // codes of the lane's rows, then this group's scales and zeros for
        // the 4 columns the lane keeps
        uint32_t w[NW];
        const uint32_t row0 = b * RB + kl * RPL;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const uint32_t off = cok ? ((row0 + r) * wp + lcol / 8) * 4 : kOffNone;
            if (WPL == 4) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
                w[4 * r] = v[0]; w[4 * r + 1] = v[1]; w[4 * r + 2] = v[2]; w[4 * r + 3] = v[3];
            } else if (WPL == 2) {
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rw, off, 0, 0);
                w[2 * r] = v[0]; w[2 * r + 1] = v[1];
            } else {
                w[r] = __builtin_amdgcn_raw_buffer_load_b32(rw, off, 0, 0);
            }
        }
        const uint32_t soff = cok ? (g * np + lcol + cb) * 4 : kOffNone;
        const f32x4 sv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, soff, 0, 0));
        const f32x4 zv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, soff, 0, 0));
        __builtin_amdgcn_sched_barrier(0);
        gemv_wait_vm<(RPL + 2 < 63 ? RPL + 2 : 63)>();      // the activation loads have landed (in-order count)
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const uint32_t e = j * kWave + lane;
            if (e < (uint32_t)(MR * XV)) {
                f32x4 f;
                if (xt == 0) {
                    f = __builtin_bit_cast(f32x4, xv[j]);
                } else if (xt == 1) {
                    const _Float16 *hh = reinterpret_cast<const _Float16 *>(&xv[j]);
                    f = f32x4{(float)hh[0], (float)hh[1], (float)hh[2], (float)hh[3]};
                } else {
                    f = f32x4{__uint_as_float(xv[j][0] << 16), __uint_as_float(xv[j][0] & 0xFFFF0000u),
                              __uint_as_float(xv[j][1] << 16), __uint_as_float(xv[j][1] & 0xFFFF0000u)};
                }
                reinterpret_cast<f32x4 *>(&xs[wv][0][0])[e] = f;
            }
        }
        // the reads below are this wave's, after its own writes (LDS
        // operations of a wave complete in order): stop code motion only
        asm volatile("" ::: "memory");

        // rows in passes of MRP over the codes in registers (unrolled: the
        // accumulators are indexed by compile-time row numbers)
#pragma unroll
        for (int mp = 0; mp < MR; mp += MRP) {
            if ((uint32_t)mp >= M) break;                   // wave-uniform
            float pm[MRP][CPL];
            float xsum[MRP];
#pragma unroll
            for (int i = 0; i < MRP; ++i) {
                xsum[i] = 0.0f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) pm[i][c] = 0.0f;
            }
#pragma unroll
            for (int r4 = 0; r4 < RPL; r4 += 4) {
                f32x4 x4[MRP];
#pragma unroll
                for (int i = 0; i < MRP; ++i)
                    x4[i] = *reinterpret_cast<const f32x4 *>(&xs[wv][mp + i][kl * RPL + r4]);   // zeros past M
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = r4 + rr;
                    float q[CPL];
#pragma unroll
                    for (int u = 0; u < WPL; ++u) {
                        const uint32_t wd = w[r * WPL + u];
                        const uint32_t lo = wd & 0x0F0F0F0Fu, hi = (wd >> 4) & 0x0F0F0F0Fu;
                        // word column j sits at AWQ shift {0,16,4,20,8,24,12,28}[j]
                        q[8 * u + 0] = (float)(lo & 0xFFu);
                        q[8 * u + 4] = (float)((lo >> 8) & 0xFFu);
                        q[8 * u + 1] = (float)((lo >> 16) & 0xFFu);
                        q[8 * u + 5] = (float)(lo >> 24);
                        q[8 * u + 2] = (float)(hi & 0xFFu);
                        q[8 * u + 6] = (float)((hi >> 8) & 0xFFu);
                        q[8 * u + 3] = (float)((hi >> 16) & 0xFFu);
                        q[8 * u + 7] = (float)(hi >> 24);
                    }
#pragma unroll
                    for (int i = 0; i < MRP; ++i) {
                        const float xm = x4[i][rr];
                        xsum[i] += xm;
#pragma unroll
                        for (int c = 0; c < CPL; ++c) pm[i][c] = __builtin_fmaf(xm, q[c], pm[i][c]);
                    }
                }
                // keep the unpacking of later rows (and passes) from being
                // hoisted here: it would hold all the unpacked codes at once
                if (MR > 4) __builtin_amdgcn_sched_barrier(0);
            }
            // combine the KL lanes of each column: reduce-scatter down to 4
            // columns per lane, all-reduce of the activation sums
#pragma unroll
            for (int i = 0; i < MRP; ++i) {
                if (CPL == 32) { halve<16, 5>(pm[i]); halve<8, 4>(pm[i]); halve<4, 3>(pm[i]); }
                if (CPL == 16) { halve<8, 5>(pm[i]); halve<4, 4>(pm[i]); }
                if (CPL == 8) { halve<4, 5>(pm[i]); }
                const float xg = klane_sum<KL>(xsum[i]);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc[mp + i][c] = __builtin_fmaf(sv[c], __builtin_fmaf(-zv[c], xg, pm[i][c]), acc[mp + i][c]);
            }
        }
        // the next block's activation slab overwrites this wave's LDS rows
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    // waves -> LDS [wave][row][column/4], then 4 columns per thread summed in wave order
#pragma unroll
    for (int m = 0; m < MR; ++m)
        red[wv][m][(cl * CPL + cb) / 4] = f32x4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
    __syncthreads();
    const uint32_t tile_id = t;
    float *part = partials + ((size_t)tile_id * slices) * (MR * kGemvTile);
    const rsrc_t rp = make_rsrc(part, slices * (MR * kGemvTile) * 4);
    float *outp = pick(p, P.out[0], P.out[1], P.out[2]);
    for (uint32_t e = threadIdx.x; e < M * (kGemvTile / 4); e += GW * kWave) {
        const uint32_t m = e / (kGemvTile / 4), c4 = e % (kGemvTile / 4);
        if (col0 + c4 * 4 >= np) continue;
        f32x4 v = red[0][m][c4];
#pragma unroll
        for (int w2 = 1; w2 < GW; ++w2) v += red[w2][m][c4];
        if (slices == 1) {
            *reinterpret_cast<f32x4 *>(outp + (size_t)m * np + col0 + c4 * 4) = v;
        } else {
            const uint32_t off = ((slice * MR + m) * kGemvTile + c4 * 4) * 4;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp, off, 0, kAuxSc1);
        }
    }
    if (slices == 1) return;

    // cross-workgroup sum, as in awq_ring: stores complete and visible at
    // device scope before the counter moves; the last workgroup loads after
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&counters[tile_id], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == slices - 1;
    }
    __syncthreads();
    if (!s_last) return;
    for (uint32_t e = threadIdx.x; e < M * (kGemvTile / 4); e += GW * kWave) {
        const uint32_t m = e / (kGemvTile / 4), c4 = e % (kGemvTile / 4);
        if (col0 + c4 * 4 >= np) continue;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (uint32_t q0 = 0; q0 < slices; q0 += 8) {
            u32x4 tv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t q = q0 + u;
                const uint32_t off = q < slices ? ((q * MR + m) * kGemvTile + c4 * 4) * 4 : kOffNone;
                tv[u] = __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, kAuxSc1);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (q0 + u < slices) v += as_f32x4(tv[u]);
        }
        *reinterpret_cast<f32x4 *>(outp + (size_t)m * np + col0 + c4 * 4) = v;
    }
    if (threadIdx.x == 0) __hip_atomic_store(&counters[tile_id], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ host --

// ---- matrix-core ring plan (m >= 16)
constexpr int kRingWaves = 8;
constexpr int kRingStages = 2;
constexpr uint32_t kRingTargetWgs = 256;   // one 8-wave workgroup per CU

struct RingPlan {
    uint32_t mt, mr, nchunks, ks_b, kb;
    bool inscale;                       // rows scaled inside each wave (its K range fits its ring)
    size_t counter_bytes, partial_bytes;
    size_t x16_offset, x16_bytes;       // pre-scaled fp16 activations (fp32 and bf16 input), behind the partials
    size_t scale_offset, scale_bytes;   // their per-row 2^-E
    size_t ws_bytes;                    // workspace this plan uses in full
};

uint32_t ring_kb(uint32_t mt, uint32_t gs, int xt) { return (gs >= 64 && !(mt == 2 && xt == KVQ_DT_F32)) ? 64 : 32; }

// 16 rows per wave up to 16 rows, else 32-row chunks; 64-row stages except
// where the group is 32 rows or two fp32 row tiles would not fit the ring;
// K slices (a power of two, whole groups per wave, then one more if K is
// split and it fits) until ~one workgroup per CU.  fp32 and bf16 rows are scaled by powers of two into fp16: inside
// each wave when its whole K range fits its ring, else by the pre-pass into
// the workspace (then the product reads fp16).
RingPlan ring_plan(uint32_t m, uint32_t k, uint32_t gs, uint32_t ntiles, int xt) {
    RingPlan pl;
    pl.mt = m <= 16 ? 1 : 2;
    pl.mr = 16 * pl.mt;
    pl.nchunks = (m + pl.mr - 1) / pl.mr;
    const uint64_t units = (uint64_t)ntiles * pl.nchunks;
    const uint32_t ngroups = k / gs;
    pl.ks_b = 1;
    while (units * pl.ks_b * 2 <= kRingTargetWgs && (uint64_t)pl.ks_b * 2 * kRingWaves <= ngroups) pl.ks_b *= 2;
    // when K is split already, one more slice if it still fits one workgroup
    // per CU: a CU streams only its share of HBM, so more busy CUs move the
    // weights sooner (some waves may then hold no group and add zeros)
    if (pl.ks_b > 1 && units * (pl.ks_b + 1) <= kRingTargetWgs && pl.ks_b + 1 <= ngroups) pl.ks_b += 1;
    const size_t tiles = (size_t)ntiles * pl.nchunks;
    if (tiles * 4 > KVQ_WORKSPACE_COUNTER_BYTES) pl.ks_b = 1;   // more tiles than counters: no exchange
    pl.kb = ring_kb(pl.mt, gs, xt);
    const uint32_t gpw = (ngroups + pl.ks_b * kRingWaves - 1) / (pl.ks_b * kRingWaves);   // most groups of a wave
    pl.inscale = xt != KVQ_DT_F16 && gpw * (gs / pl.kb) <= (uint32_t)kRingStages;
    const bool pre = xt != KVQ_DT_F16 && !pl.inscale;
    if (pre) pl.kb = ring_kb(pl.mt, gs, KVQ_DT_F16);   // the product then reads the fp16 copy
    pl.counter_bytes = pl.ks_b > 1 ? KVQ_WORKSPACE_COUNTER_BYTES : 0;
    pl.partial_bytes = pl.ks_b > 1 ? tiles * pl.ks_b * pl.mr * 128 * 4 : 0;
    // the counter area is always kept (zero) in front when the copy is there
    pl.x16_offset = KVQ_WORKSPACE_COUNTER_BYTES + pl.partial_bytes;
    pl.x16_bytes = pre ? ((size_t)m * k * 2 + 255) / 256 * 256 : 0;
    pl.scale_offset = pl.x16_offset + pl.x16_bytes;
    pl.scale_bytes = pre ? ((size_t)m * 4 + 255) / 256 * 256 : 0;
    pl.ws_bytes = pre ? pl.scale_offset + pl.scale_bytes : pl.counter_bytes + pl.partial_bytes;
    return pl;
}

// two fp32 row tiles per wave only fit the ring with 32-row stages
template <int MT, int XT>
void ring_launch(const RingPlan &pl, uint64_t blocks, const void *x, uint32_t m, uint32_t k, uint32_t gs,
                 const Projs &P, uint32_t *counters, float *partials, const float *rscale, hipStream_t s) {
    if constexpr (!(MT == 2 && XT == 0)) {
        if (pl.kb == 64) {
            awq_ring<MT, XT, 64, kRingStages, kRingWaves><<<(unsigned)blocks, kRingWaves * kWave, 0, s>>>(
                x, m, k, gs, P, pl.nchunks, pl.ks_b, counters, partials, rscale, pl.inscale ? 1 : 0);
            return;
        }
    }
    awq_ring<MT, XT, 32, kRingStages, kRingWaves><<<(unsigned)blocks, kRingWaves * kWave, 0, s>>>(
        x, m, k, gs, P, pl.nchunks, pl.ks_b, counters, partials, rscale, pl.inscale ? 1 : 0);
}

int check_proj(const char *fn, const int4_awq_proj_t *p, const char *which, uint32_t k, uint32_t gs) {
    if (!p->qweight || !p->scales || !p->zeros || !p->out)
        return fail(KVQ_E_INVALID, "%s: %s projection has a null pointer", fn, which);
    if (!aligned16(p->qweight) || !aligned16(p->scales) || !aligned16(p->zeros) || !aligned16(p->out))
        return fail(KVQ_E_INVALID, "%s: %s projection pointers must be 16-byte aligned", fn, which);
    if (p->n == 0 || p->n % 8)
        return fail(KVQ_E_INVALID, "%s: %s projection n=%u (want a positive multiple of 8)", fn, which, p->n);
    if ((uint64_t)k * p->n / 2 >= 0x80000000ull || (uint64_t)(k / gs) * p->n * 4 >= 0x80000000ull)
        return fail(KVQ_E_INVALID, "%s: %s projection larger than 2 GiB", fn, which);
    return KVQ_OK;
}

uint32_t tiles_of(uint32_t n) { return (n / 8 + 15) / 16; }

// ---- fp32 GEMV plan (m < kGemvMaxM)
constexpr uint32_t kGemvMaxM = 16;        // the matrix-core path takes 16 rows and more
constexpr uint32_t kGemvTargetWgs = 192;  // ~1 workgroup per CU: every load of a call in flight at once
// rows per block (a wave's unit of work) and waves per workgroup: up to 2
// activation rows, 64-row blocks in 8-wave workgroups (a workgroup still
// covers 512 rows, so the exchange is unchanged, and each wave's unpacking
// and FMAs are half those of a 128-row block); more rows, 128-row blocks
// (64 with 8 rows, to keep the codes in registers) in 4-wave workgroups
constexpr uint32_t kGemvRbSmall = 64, kGemvGwSmall = 8;
constexpr uint32_t kGemvGwLarge = 4;

struct GemvPlan {
    uint32_t mr, rb, gw, slices, gpw;
    size_t ws_bytes;   // counters + partial tiles, 0 when one workgroup covers a tile's K
};

// rows the accumulators are built for; 9..15 rows run as two launches of 8
uint32_t gemv_mr(uint32_t m) { return m <= 1 ? 1 : (m <= 2 ? 2 : (m <= 4 ? 4 : 8)); }

GemvPlan gemv_plan(uint32_t m, uint32_t k, uint32_t gs, uint32_t tiles, bool have_ws) {
    GemvPlan g;
    g.mr = gemv_mr(m);
    const uint32_t rbmax = g.mr <= 2 ? kGemvRbSmall : (g.mr >= 8 ? 64 : 128);
    g.rb = gs < rbmax ? gs : rbmax;
    g.gw = g.mr <= 2 ? kGemvGwSmall : kGemvGwLarge;
    const uint32_t nblocks = k / g.rb;
    // one block per wave while the grid stays at or under the target,
    // otherwise more blocks per wave; slices of gw*gpw blocks
    uint32_t gpw = 1;
    while ((uint64_t)tiles * ((nblocks + g.gw * gpw - 1) / (g.gw * gpw)) > kGemvTargetWgs && g.gw * gpw < nblocks)
        gpw *= 2;
    g.gpw = gpw;
    g.slices = (nblocks + g.gw * gpw - 1) / (g.gw * gpw);
    if (tiles * 4 > KVQ_WORKSPACE_COUNTER_BYTES) g.slices = 1;   // more tiles than counters
    if (!have_ws || g.slices == 1) {
        g.slices = 1;
        g.gpw = (nblocks + g.gw - 1) / g.gw;
    }
    g.ws_bytes = g.slices > 1 ? KVQ_WORKSPACE_COUNTER_BYTES + (size_t)tiles * g.slices * g.mr * kGemvTile * 4 : 0;
    return g;
}

uint32_t gemv_tiles_of(uint32_t n) { return (n + kGemvTile - 1) / kGemvTile; }

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" int int4_awq_workspace_bytes(uint32_t m, uint32_t k, uint32_t group_size, uint32_t n_total,
                                        size_t *bytes) {
    if (!bytes) return fail(KVQ_E_INVALID, "int4_awq_workspace_bytes: null output pointer");
    *bytes = 0;
    if (m == 0 || group_size < 32 || group_size % 32 || k % group_size || n_total % 8) return KVQ_OK;
    // splitting n_total into up to three projections adds at most two tiles
    for (uint32_t extra = 0; extra <= 2; ++extra) {
        if (m < kGemvMaxM) {
            const GemvPlan g = gemv_plan(m, k, group_size, gemv_tiles_of(n_total) + extra, true);
            if (g.ws_bytes > *bytes) *bytes = g.ws_bytes;
        } else {
            const RingPlan pl = ring_plan(m, k, group_size, tiles_of(n_total) + extra, KVQ_DT_F32);
            if (pl.ws_bytes > *bytes) *bytes = pl.ws_bytes;
        }
    }
    return KVQ_OK;
}

namespace kvq {
namespace {

// need: when set, validate, store the workspace bytes this call's full plan
// uses, and launch nothing.
int awq_run(const char *fn, const void *x, int xt, uint32_t m, uint32_t k, uint32_t group_size,
            const int4_awq_proj_t *q_proj, const int4_awq_proj_t *k_proj, const int4_awq_proj_t *v_proj,
            void *workspace, size_t workspace_bytes, void *stream, size_t *need = nullptr) {
    if (xt != KVQ_DT_F32 && xt != KVQ_DT_F16 && xt != KVQ_DT_BF16)
        return fail(KVQ_E_INVALID, "%s: x dtype %d is not fp32 (0), fp16 (1) or bf16 (2)", fn, xt);
    if (!x || !q_proj) return fail(KVQ_E_INVALID, "%s: null x or q projection", fn);
    if (!aligned16(x)) return fail(KVQ_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
    if (m == 0) return fail(KVQ_E_INVALID, "%s: m == 0", fn);
    if (group_size != 32 && group_size != 64 && group_size != 128 && group_size != 256)
        return fail(KVQ_E_INVALID, "%s: group_size=%u (supported: 32, 64, 128, 256)", fn, group_size);
    if (k == 0 || k % group_size)
        return fail(KVQ_E_INVALID, "%s: K=%u is not a positive multiple of group_size=%u", fn, k, group_size);
    if ((uint64_t)m * k * 4 >= 0x80000000ull) return fail(KVQ_E_INVALID, "%s: x larger than 2 GiB", fn);
    if ((k_proj == nullptr) != (v_proj == nullptr))
        return fail(KVQ_E_INVALID, "%s: k and v projections must be both set or both NULL", fn);
    int st = check_proj(fn, q_proj, "q", k, group_size);
    if (st) return st;
    const int4_awq_proj_t *list[3] = {q_proj, k_proj, v_proj};
    if (k_proj) {
        st = check_proj(fn, k_proj, "k", k, group_size);
        if (st) return st;
        st = check_proj(fn, v_proj, "v", k, group_size);
        if (st) return st;
        if (k_proj->n != v_proj->n)
            return fail(KVQ_E_INVALID, "%s: k and v projections differ in n (%u vs %u)", fn, k_proj->n, v_proj->n);
    }
    Projs P;
    P.count = k_proj ? 3 : 1;
    uint32_t tiles = 0;
    for (uint32_t i = 0; i < 3; ++i) {
        const int4_awq_proj_t *pr = i < P.count ? list[i] : q_proj;
        P.qw[i] = pr->qweight; P.sc[i] = pr->scales; P.zr[i] = pr->zeros; P.out[i] = pr->out;
        P.n[i] = i < P.count ? pr->n : 0;
        P.tstart[i] = tiles;
        if (i < P.count) tiles += tiles_of(pr->n);
    }
    P.ntiles = tiles;
    hipStream_t s = as_stream(stream);

    if (m < kGemvMaxM) {
        // fp32 weight-streaming GEMV: 256-column tiles per projection
        Projs G = P;
        uint32_t gt = 0;
        bool c32 = true, c16 = true;
        for (uint32_t i = 0; i < 3; ++i) {
            G.tstart[i] = gt;
            if (i < P.count) {
                gt += gemv_tiles_of(P.n[i]);
                c32 = c32 && P.n[i] % 32 == 0;
                c16 = c16 && P.n[i] % 16 == 0;
            }
        }
        G.ntiles = gt;
        if (need) {
            *need = gemv_plan(m, k, group_size, gt, true).ws_bytes;
            return KVQ_OK;
        }
        GemvPlan gp = gemv_plan(m, k, group_size, gt, false);
        uint32_t *counters = nullptr;
        float *partials = nullptr;
        const GemvPlan gw = gemv_plan(m, k, group_size, gt, true);
        if (gw.slices > 1 && workspace && aligned16(workspace) && workspace_bytes >= gw.ws_bytes) {
            gp = gw;
            counters = static_cast<uint32_t *>(workspace);
            partials = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + KVQ_WORKSPACE_COUNTER_BYTES);
        }
        const unsigned blocks = gt * gp.slices;
        // columns per lane: 32 up to 2 rows, 16 up to 4, 8 above (and
        // whenever a projection's n is not a multiple of the wider choice);
        // 9..15 rows: rows 0-7, then the rest, with the output pointers moved
#define KVQ_GEMV5(CPL, MR, MRP, RB, GW, XP, MM, PP)                                                            \
    awq_gemv<CPL, MR, MRP, RB, GW><<<blocks, GW * kWave, 0, s>>>(XP, MM, k, group_size, xt, PP, gp.slices, gp.gpw, \
                                                                counters, partials)
#define KVQ_GEMV4(CPL, MR, MRP, RB, XP, MM, PP)                                           \
    do {                                                                                  \
        if (gp.gw == kGemvGwSmall) KVQ_GEMV5(CPL, MR, MRP, RB, kGemvGwSmall, XP, MM, PP); \
        else KVQ_GEMV5(CPL, MR, MRP, RB, kGemvGwLarge, XP, MM, PP);                       \
    } while (0)
#define KVQ_GEMV(CPL, MR, MRP, XP, MM, PP)                                 \
    do {                                                                   \
        if (gp.rb == 32) KVQ_GEMV4(CPL, MR, MRP, 32, XP, MM, PP);          \
        else if (gp.rb == 64) KVQ_GEMV4(CPL, MR, MRP, 64, XP, MM, PP);     \
        else KVQ_GEMV4(CPL, MR, MRP, 128, XP, MM, PP);                     \
    } while (0)
        if (gp.mr == 1) {
            if (c32) KVQ_GEMV(32, 1, 1, x, m, G);
            else KVQ_GEMV(8, 1, 1, x, m, G);
        } else if (gp.mr == 2) {
            if (c32) KVQ_GEMV(32, 2, 2, x, m, G);
            else KVQ_GEMV(8, 2, 2, x, m, G);
        } else if (gp.mr == 4) {
            if (c16) KVQ_GEMV(16, 4, 4, x, m, G);
            else KVQ_GEMV(8, 4, 4, x, m, G);
        } else {
            KVQ_GEMV(8, 8, 4, x, (m < 8 ? m : 8u), G);
            if (m > 8) {
                int st = launch_status(fn);
                if (st) return st;
                Projs G2 = G;
                for (uint32_t i = 0; i < 3; ++i) G2.out[i] = G.out[i] + (size_t)8 * G.n[i];
                const void *x2 = static_cast<const uint8_t *>(x) + (size_t)8 * k * (xt == KVQ_DT_F32 ? 4 : 2);
                KVQ_GEMV(8, 8, 4, x2, m - 8, G2);
            }
        }
#undef KVQ_GEMV
#undef KVQ_GEMV4
#undef KVQ_GEMV5
        return launch_status(fn);
    }

    RingPlan pl = ring_plan(m, k, group_size, P.ntiles, xt);
    if (need) {
        *need = pl.ws_bytes;
        return KVQ_OK;
    }
    uint32_t *counters = nullptr;
    float *partials = nullptr;
    const float *rscale = nullptr;
    const bool have_ws = workspace && aligned16(workspace) && workspace_bytes >= pl.ws_bytes;
    if (pl.ks_b > 1) {
        if (!have_ws) {
            pl.ks_b = 1;   // no (or too small) workspace: one workgroup per tile
        } else {
            counters = static_cast<uint32_t *>(workspace);
            partials = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pl.counter_bytes);
        }
    }
    if (pl.x16_bytes && have_ws) {
        // fp32 / bf16 activations: per-row power-of-two scaling into fp16
        f16x8 *x16 = reinterpret_cast<f16x8 *>(static_cast<uint8_t *>(workspace) + pl.x16_offset);
        float *sc = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pl.scale_offset);
        if (xt == KVQ_DT_F32) x_pow2_f16<0><<<m, 256, 0, s>>>(x, k, x16, sc);
        else x_pow2_f16<2><<<m, 256, 0, s>>>(x, k, x16, sc);
        int st = launch_status(fn);
        if (st) return st;
        x = x16;
        xt = KVQ_DT_F16;
        rscale = sc;
    } else if (pl.x16_bytes) {
        // without a workspace the product kernel rounds the activations
        // itself, unscaled
        pl.kb = ring_kb(pl.mt, group_size, xt);
    }
    // the kernel's placement: tile pairs on one XCD (see there)
    const uint64_t npairs = (P.ntiles + 1) / 2;
    const uint64_t blocks = pl.nchunks > 1
                                ? (uint64_t)kXcds * ((npairs + kXcds - 1) / kXcds) * 2 * pl.nchunks * pl.ks_b
                                : 2 * (uint64_t)kXcds * ((npairs * pl.ks_b + kXcds - 1) / kXcds);
    if (blocks > 0x7FFFFFFFull) return fail(KVQ_E_INVALID, "%s: problem too large", fn);
    if (pl.mt == 1) {
        if (xt == KVQ_DT_F32) ring_launch<1, 0>(pl, blocks, x, m, k, group_size, P, counters, partials, rscale, s);
        else if (xt == KVQ_DT_F16) ring_launch<1, 1>(pl, blocks, x, m, k, group_size, P, counters, partials, rscale, s);
        else ring_launch<1, 2>(pl, blocks, x, m, k, group_size, P, counters, partials, rscale, s);
    } else {
        if (xt == KVQ_DT_F32) ring_launch<2, 0>(pl, blocks, x, m, k, group_size, P, counters, partials, rscale, s);
        else if (xt == KVQ_DT_F16) ring_launch<2, 1>(pl, blocks, x, m, k, group_size, P, counters, partials, rscale, s);
        else ring_launch<2, 2>(pl, blocks, x, m, k, group_size, P, counters, partials, rscale, s);
    }
    return launch_status(fn);
}

}  // namespace
}  // namespace kvq

extern "C" int int4_awq_qkv_gemm(const float *x, uint32_t m, uint32_t k, uint32_t group_size,
                                 const int4_awq_proj_t *q_proj, const int4_awq_proj_t *k_proj,
                                 const int4_awq_proj_t *v_proj, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    return awq_run("int4_awq_qkv_gemm", x, KVQ_DT_F32, m, k, group_size, q_proj, k_proj, v_proj, workspace,
                   workspace_bytes, stream);
}

extern "C" int int4_awq_qkv_gemm_dt(const void *x, int x_dtype, uint32_t m, uint32_t k, uint32_t group_size,
                                    const int4_awq_proj_t *q_proj, const int4_awq_proj_t *k_proj,
                                    const int4_awq_proj_t *v_proj, void *workspace, size_t workspace_bytes,
                                    void *stream) {
    return awq_run("int4_awq_qkv_gemm_dt", x, x_dtype, m, k, group_size, q_proj, k_proj, v_proj, workspace,
                   workspace_bytes, stream);
}

// ---------------------------------------------------- without allocation --
//
// int4_awq_qkv_gemm for callers that cannot allocate (code under HIP graph
// capture, serving loops, hosts that forbid hipMalloc): the workspace is a
// file-scope device array, one copy per GPU held until the process ends.
// Host code reaches it only through the address hipGetSymbolAddress returns
// for the current device (the array's name on the host is a stand-in, not a
// device address).  Its counter area starts zero (module load) and every
// call leaves it zero; partial tiles and the fp16 activation copy are
// written before they are read by each call.  Calls that overlap on one GPU
// share the array and race.

namespace kvq {
namespace {

constexpr size_t kNoAllocScratchBytes = KVQ_INT4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

int scratch_of_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KVQ_E_LAUNCH, "int4_awq_qkv_gemm_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KVQ_E_UNSUPPORTED, "int4_awq_qkv_gemm_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(e == hipErrorNoBinaryForGpu ? KVQ_E_UNSUPPORTED : KVQ_E_LAUNCH,
                        "int4_awq_qkv_gemm_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KVQ_OK;
}

}  // namespace
}  // namespace kvq

extern "C" int int4_awq_qkv_gemm_noalloc(const float *x, uint32_t m, uint32_t k, uint32_t group_size,
                                         const int4_awq_proj_t *q_proj, const int4_awq_proj_t *k_proj,
                                         const int4_awq_proj_t *v_proj, void *stream) {
    const char *fn = "int4_awq_qkv_gemm_noalloc";
    size_t need = 0;
    int st = awq_run(fn, x, KVQ_DT_F32, m, k, group_size, q_proj, k_proj, v_proj, nullptr, 0, stream, &need);
    if (st) return st;
    if (need > kNoAllocScratchBytes)
        return fail(KVQ_E_INVALID, "%s: this shape needs %zu bytes of scratch, more than the %zu the library holds "
                    "per GPU; use int4_awq_qkv_gemm with a workspace", fn, need, kNoAllocScratchBytes);
    void *ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st) return st;
    return awq_run(fn, x, KVQ_DT_F32, m, k, group_size, q_proj, k_proj, v_proj, ws, kNoAllocScratchBytes, stream);
}
