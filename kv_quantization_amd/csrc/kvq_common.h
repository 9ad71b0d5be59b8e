// Internal helpers shared by the libkvq.so translation units: error
// reporting, argument checks and a few wave-level device primitives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

#include "kvq.h"

namespace kvq {

// Records a printf-style message for kvq_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Status after a launch: KVQ_OK, or KVQ_E_UNSUPPORTED / KVQ_E_LAUNCH with the
// runtime's message.
int launch_status(const char *what);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int kWave = 64;

// Native vector types (usable with the nontemporal load/store builtins).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- device --

// Butterfly reductions over aligned lane teams of size W (a power of two <=
// 64); every lane of the team ends with the result.
template <int W>
__device__ __forceinline__ float team_max(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

template <int W>
__device__ __forceinline__ float team_min(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}

template <int W>
__device__ __forceinline__ float team_sum(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Max of NON-NEGATIVE floats (absolute values) over lane teams with DPP lane
// moves inside the VALU, no LDS round trip.  Non-negative floats order like
// their bit patterns as unsigned integers, so the max runs on the bits (no
// NaN canonicalisation; +0 is the identity, which lanes outside a DPP row
// mask read).  Steps: swap neighbours, swap pairs, mirror half-rows of 8,
// mirror rows of 16; after each, a lane holds the max over its aligned 2, 4,
// 8, 16 lanes.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
    return v > o ? v : o;
}

// Aligned teams of W <= 16 lanes; every lane of the team gets the result.
template <int W>
__device__ __forceinline__ float team_absmax_dpp(float a) {
    static_assert(W == 2 || W == 4 || W == 8 || W == 16, "DPP teams of 2..16 lanes");
    uint32_t v = __float_as_uint(a);
    v = dpp_umax<0xB1>(v);                   // quad_perm [1,0,3,2]
    if (W >= 4) v = dpp_umax<0x4E>(v);       // quad_perm [2,3,0,1]
    if (W >= 8) v = dpp_umax<0x141>(v);      // row_half_mirror
    if (W >= 16) v = dpp_umax<0x140>(v);     // row_mirror
    return __uint_as_float(v);
}

// The whole wave, as a uniform value: rows of 16 as above, then lane 15 of
// each row into the next row (rows 1 and 3), lane 31 into rows 2 and 3, and
// lane 63 (which then holds the max of all four rows) read out.
__device__ __forceinline__ float wave_absmax_dpp(float a) {
    uint32_t v = __float_as_uint(team_absmax_dpp<16>(a));
    v = dpp_umax<0x142, 0xA>(v);             // row_bcast:15
    v = dpp_umax<0x143, 0xC>(v);             // row_bcast:31
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)v, 63));
}

// Raw buffer resources: loads through them take an SGPR base, a per-lane
// 32-bit offset and a uniform offset, and a lane whose offset is at or past
// the stated size reads zeros without touching memory, so predicated loads
// need no branch (branches around loads make the compiler wait for every
// outstanding load where the paths meet).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw (untyped) buffer, gfx9 family
constexpr uint32_t kOffNone = 0x80000000u;     // a lane offset past every resource used here (sizes < 2 GiB)

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, (int)kRsrcWord3);
}

// Uniform selection among up to three per-part pointers or sizes (explicit
// selects keep the values in SGPRs; indexing a kernel-argument array would
// load them into VGPRs and force per-lane buffer-resource loops).
template <typename T>
__device__ __forceinline__ T pick(int p, T a0, T a1, T a2) {
    return p == 0 ? a0 : (p == 1 ? a1 : a2);
}

// RN(v / s) for a quantization scale s (normal, >= 1e-8) given y = RN(1/s),
// in three operations instead of a full IEEE division: Markstein's sequence
// (q = RN(v y); the residual v - q s is exact by FMA; RN(q + residual * y))
// yields the correctly rounded quotient whenever the residual does not
// underflow.  It can only underflow for |v| below about 2^-100, i.e. for
// quotients below 2^-70 here (s >= 1e-8), far under every code boundary
// (E4M3's smallest half-step 2^-10, rint's 0.5), so the codes equal those
// of an IEEE division.  The sequence turns -0 / s into +0, so zeros pass
// through unchanged (E4M3 has a negative-zero code).  (Checked on 2e9 random
// pairs: same sign always, and every value mismatch had a quotient below
// 2^-82.)
__device__ __forceinline__ float div_by_scale(float v, float s, float y) {
    const float q = v * y;
    const float r = __builtin_fmaf(__builtin_fmaf(-q, s, v), y, q);
    return v == 0.0f ? v : r;
}

}  // namespace kvq
