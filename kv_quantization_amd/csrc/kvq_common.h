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

}  // namespace kvq
