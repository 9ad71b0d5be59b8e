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
