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

// Every pointer set and 16-byte aligned, else KVQ_E_INVALID naming the call.
inline int check_ptrs(const char *fn, std::initializer_list<const void *> ps) {
    for (const void *p : ps) {
        if (!p) return fail(KVQ_E_INVALID, "%s: null pointer argument", fn);
        if (!aligned16(p)) return fail(KVQ_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
    }
    return KVQ_OK;
}

constexpr int kWave = 64;

// Native vector types (usable with the nontemporal load/store builtins).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- device --

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Reductions over aligned lane teams of W = 1..64 lanes, every lane of the
// team ending with the result, without LDS round trips: DPP lane moves inside
// the VALU for teams up to a row of 16 (swap neighbours, swap pairs, mirror
// half-rows of 8, mirror rows of 16: after each step a lane holds the result
// over its aligned 2, 4, 8, 16 lanes), then v_permlane16_swap (rows 0<->1,
// 2<->3) and v_permlane32_swap (halves).  Called with both operands equal, a
// swap returns each lane its own and its partner's value, whichever way the
// rows move.  The reductions run on integers: finite floats map to signed
// integers of the same order (-0 just below +0), and non-negative floats
// (absolute values) are already ordered by their bits.
template <int CTRL, bool MAX>
__device__ __forceinline__ int dpp_ext(int v) {
    const int id = MAX ? (int)0x80000000 : 0x7FFFFFFF;   // identity: what a masked lane reads
    const int o = __builtin_amdgcn_update_dpp(id, v, CTRL, 0xF, 0xF, false);
    return MAX ? (v > o ? v : o) : (v < o ? v : o);
}

template <int W, bool MAX>
__device__ __forceinline__ int team_ext(int v) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "teams of 1..64 lanes");
    if (W >= 2) v = dpp_ext<0xB1, MAX>(v);       // quad_perm [1,0,3,2]
    if (W >= 4) v = dpp_ext<0x4E, MAX>(v);       // quad_perm [2,3,0,1]
    if (W >= 8) v = dpp_ext<0x141, MAX>(v);      // row_half_mirror
    if (W >= 16) v = dpp_ext<0x140, MAX>(v);     // row_mirror
    if (W >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
        const int a = (int)r[0], b = (int)r[1];
        v = MAX ? (a > b ? a : b) : (a < b ? a : b);
    }
    if (W >= 64) {
        const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
        const int a = (int)r[0], b = (int)r[1];
        v = MAX ? (a > b ? a : b) : (a < b ? a : b);
    }
    return v;
}

__device__ __forceinline__ int float_order(float f) {
    const int b = __float_as_int(f);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float order_float(int o) { return __int_as_float(o ^ ((o >> 31) & 0x7FFFFFFF)); }

template <int W>
__device__ __forceinline__ float team_max(float v) { return order_float(team_ext<W, true>(float_order(v))); }

template <int W>
__device__ __forceinline__ float team_min(float v) { return order_float(team_ext<W, false>(float_order(v))); }

// Max of non-negative floats (absolute values).
// Sum over an aligned team of W lanes with the same lane moves.  Each step
// adds a lane's value and its partner's, and fp addition is commutative, so
// every lane of the team ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int W>
__device__ __forceinline__ float team_sum(float v) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "teams of 1..64 lanes");
    if (W >= 2) v += dpp_move<0xB1>(v);
    if (W >= 4) v += dpp_move<0x4E>(v);
    if (W >= 8) v += dpp_move<0x141>(v);
    if (W >= 16) v += dpp_move<0x140>(v);
    if (W >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if (W >= 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}

template <int W>
__device__ __forceinline__ float team_absmax(float v) { return __int_as_float(team_ext<W, true>(__float_as_int(v))); }

// Raw buffer resources: loads through them take an SGPR base, a per-lane
// 32-bit offset and a uniform offset, and a lane whose offset is at or past
// the stated size reads zeros without touching memory, so predicated loads
// need no branch (branches around loads make the compiler wait for every
// outstanding load where the paths meet).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw (untyped) buffer, gfx9 family
constexpr uint32_t kOffNone = 0x80000000u;     // a lane offset past every resource used here (sizes < 2 GiB)

// Cache-policy operand of the buffer intrinsics: sc1 makes a load or store
// coherent at agent scope (the encoding an agent-scope relaxed atomic load or
// store uses on this family), which partial tiles exchanged between
// workgroups on different XCDs (whose L2s are not coherent) need.
constexpr int kAuxSc1 = 16;

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

// LDS byte offset of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Raw buffer resource (4 SGPRs): base, stride 0, size in bytes (reads past
// it return zero), untyped dword format of the gfx9 family.
__device__ __forceinline__ u32x4 buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// Direct loads into LDS, written as inline assembly so that the compiler does
// not add its conservative "all LDS DMA complete" wait before every LDS read;
// a ring waits explicitly (wait_vm) for exactly the stage it is about to
// read.  lds_wave_base must be wave-uniform (it goes to M0).  M0 is named as
// clobbered; nothing else in these kernels keeps a value in M0 (gfx9 LDS
// instructions do not use it), so the "reserved register" warning does not
// apply.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_buf16(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_wave_base) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 ::"v"(voff), "s"(rsrc), "s"(soff), "s"(lds_wave_base) : "memory", "m0");
}
__device__ __forceinline__ void lds_buf4(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_wave_base) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 ::"v"(voff), "s"(rsrc), "s"(soff), "s"(lds_wave_base) : "memory", "m0");
}
__device__ __forceinline__ void lds_glb16(const void *g, uint32_t lds_wave_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_wave_base), "v"(g) : "memory", "m0");
}
#pragma clang diagnostic pop

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// RN(v / s) for a quantization scale s (normal, >= 1e-8) given y = RN(1/s),
// in three operations instead of a full IEEE division: Markstein's sequence
// (q = RN(v y); the residual v - q s is exact by FMA; RN(q + residual * y))
// yields the correctly rounded quotient whenever the residual does not
// underflow.  It can only underflow for |v| below about 2^-100, i.e. for
// quotients below 2^-70 here (s >= 1e-8), far under every code boundary
// (E4M3's smallest half-step 2^-10, rint's 0.5), so the codes equal those
// of an IEEE division.  The sequence turns -0 / s into +0, so zeros pass
// through unchanged (E4M3 has a negative-zero code).  tests/
// div_by_scale_check.c runs this sequence against IEEE division on the CPU
// over ~40 million seeded pairs of the codecs' kinds plus every code
// boundary: the quotients agree bit for bit except a few below 2^-80, which
// keep their sign.
__device__ __forceinline__ float div_by_scale(float v, float s, float y) {
    const float q = v * y;
    const float r = __builtin_fmaf(__builtin_fmaf(-q, s, v), y, q);
    return v == 0.0f ? v : r;
}

}  // namespace kvq
