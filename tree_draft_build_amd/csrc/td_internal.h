// Internal helpers of libtreedraft (gfx950, wave64).  Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>

#include "treedraft.h"

namespace td {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// host side: error reporting and validation
// ---------------------------------------------------------------------------

void set_error(const char *fmt, ...);
void clear_error();

// Records the message and returns the status, so validation reads as
// `if (bad) return fail(TD_EINVAL, "...")`.
inline td_status fail(td_status st, const char *msg) {
    set_error("%s", msg);
    return st;
}

// Checks the launch that was just enqueued.
td_status check_launch(const char *what);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned8(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Events attached to the calling thread's next kernel launches (set by
// td_verify_step_events for the duration of one call): the first launch
// records `start` when it begins executing, every launch records `stop` when
// it ends, so the last launch's end stands.  Both null: plain launches.
// Events attached to the calling thread's next launches: start to launch
// `first` and stop to launches first .. last (the last one recorded counts);
// `next` numbers the launches made meanwhile.
struct LaunchEvents {
    hipEvent_t start, stop;
    int first, last, next;
};
extern thread_local LaunchEvents t_launch_events;

// hipLaunchKernelGGL, with the thread's launch events attached when set.
#define TD_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                      \
    do {                                                                                       \
        ::td::LaunchEvents &td_ev_ = ::td::t_launch_events;                                    \
        const int td_i_ = td_ev_.start || td_ev_.stop ? td_ev_.next++ : -1;                    \
        hipEvent_t td_a_ = td_i_ == td_ev_.first ? td_ev_.start : nullptr;                     \
        hipEvent_t td_b_ = td_i_ >= td_ev_.first && td_i_ <= td_ev_.last ? td_ev_.stop : nullptr; \
        if (td_a_ || td_b_) {                                                                  \
            hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, td_a_, td_b_, 0, __VA_ARGS__); \
        } else {                                                                               \
            hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);               \
        }                                                                                      \
    } while (0)

// ---------------------------------------------------------------------------
// device side
// ---------------------------------------------------------------------------

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------------------
// Register-only lane exchanges (no LDS round trip).  Level L of a 6-level
// butterfly pairs every lane with one lane of a disjoint group:
//   L=0: lane ^ 1            (DPP quad_perm [1,0,3,2])
//   L=1: lane ^ 2            (DPP quad_perm [2,3,0,1])
//   L=2: 7 - lane within 8   (DPP row_half_mirror)
//   L=3: 15 - lane within 16 (DPP row_mirror)
//   L=4: lane ^ 16           (v_permlane16_swap, gfx950)
//   L=5: lane ^ 32           (v_permlane32_swap, gfx950)
// After levels 0..k every lane of an aligned group of 2^(k+1) lanes has
// combined the whole group, so any associative, commutative merge applied at
// levels 0..5 leaves the full wave's result in every lane.  Levels 0..3 stay
// inside 16-lane rows.
// ---------------------------------------------------------------------------
template <int L>
__device__ __forceinline__ uint32_t xchg(uint32_t x) {
    if constexpr (L == 0) return __builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, false);
    else if constexpr (L == 1) return __builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, false);
    else if constexpr (L == 2) return __builtin_amdgcn_update_dpp(0u, x, 0x141, 0xF, 0xF, false);
    else if constexpr (L == 3) return __builtin_amdgcn_update_dpp(0u, x, 0x140, 0xF, 0xF, false);
    else if constexpr (L == 4) {
        auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return ((__lane_id() >> 4) & 1) ? r[0] : r[1];
    } else {
        auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (__lane_id() >> 5) ? r[0] : r[1];
    }
}
// lane ^ 8 (DPP row_ror:8 within the 16-lane row): with levels 4 and 5 it
// combines the 8 lanes l % 8 + 8 k of an aligned group of 64 only, keeping
// lanes of different l % 8 apart.
__device__ __forceinline__ float xor8_f(float x) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x128, 0xF, 0xF, false));
}
template <int L> __device__ __forceinline__ int xchg_i(int x) {
    return static_cast<int>(xchg<L>(static_cast<uint32_t>(x)));
}
template <int L> __device__ __forceinline__ float xchg_f(float x) {
    return __uint_as_float(xchg<L>(__float_as_uint(x)));
}
template <int L> __device__ __forceinline__ double xchg_d(double x) {
    const uint64_t u = __double_as_longlong(x);
    const uint64_t lo = xchg<L>(static_cast<uint32_t>(u));
    const uint64_t hi = xchg<L>(static_cast<uint32_t>(u >> 32));
    return __longlong_as_double(static_cast<long long>(lo | (hi << 32)));
}

// Wave-wide max / sum over the 64 lanes of a wavefront (every lane gets it).
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, xchg_f<0>(v));
    v = fmaxf(v, xchg_f<1>(v));
    v = fmaxf(v, xchg_f<2>(v));
    v = fmaxf(v, xchg_f<3>(v));
    v = fmaxf(v, xchg_f<4>(v));
    v = fmaxf(v, xchg_f<5>(v));
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
    v += xchg_d<0>(v);
    v += xchg_d<1>(v);
    v += xchg_d<2>(v);
    v += xchg_d<3>(v);
    v += xchg_d<4>(v);
    v += xchg_d<5>(v);
    return v;
}
// max / sum over the 16 lanes of a row (levels 0..3)
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, xchg_f<0>(v));
    v = fmaxf(v, xchg_f<1>(v));
    v = fmaxf(v, xchg_f<2>(v));
    v = fmaxf(v, xchg_f<3>(v));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += xchg_f<0>(v);
    v += xchg_f<1>(v);
    v += xchg_f<2>(v);
    v += xchg_f<3>(v);
    return v;
}

}  // namespace td
