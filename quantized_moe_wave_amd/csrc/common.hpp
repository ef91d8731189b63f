// Device-side types and helpers shared by the MoE FFN kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kQ4Bytes = 144;    // bytes of one Q4_K super-block
constexpr int kQ4Weights = 256;  // weights of one Q4_K super-block
constexpr int kRowGroup = 16;    // rows per repacked row group (= MFMA N)
constexpr int kGroupSbBytes = kRowGroup * kQ4Bytes;  // 2304: one row group x one super-block
constexpr int kGroupQsBytes = 2048;                  // quant part of that block
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;
constexpr int kTileM = 16;       // tokens per expert tile in the MFMA expert kernel

// Staged activation layout (one row = one token or one expert slot, K = nsb*256):
//   hilo  : for super-block b, k-step s (32 columns), lane group g (8 columns):
//           16 halves = 8 "hi" then 8 "lo" values of the scaled row, at half
//           offset ((b*8 + s)*4 + g)*16. Element e holds column
//           256b + 32s + 8g + kPerm[e] (the order the Q4_K nibble unpack yields).
//   xs    : per (row, b) 16 halves: hi of the 8 k-step sums, then their lo.
//   sinv  : per (row, b) the power of two that undoes the row scaling.
// kPerm = {0, 2, 1, 3, 4, 6, 5, 7}.
__device__ __forceinline__ int perm8(int e) { return (e & 4) | ((e & 1) << 1) | ((e >> 1) & 1); }

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(f16, (uint16_t)bits16);
}

__device__ __forceinline__ f16x2 u32_as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t f16x2_as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Cross-workgroup hand-off within one launch. Data handed to another
// workgroup is written with agent-scope atomic stores and read with
// agent-scope atomic loads (coherent accesses on this multi-XCD part); the
// writers wait until their stores have completed, and the completion counter
// is updated with release/acquire semantics at agent scope.
__device__ __forceinline__ void wait_own_stores() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ uint32_t counter_arrive_acq_rel(uint32_t *c) {
    return __hip_atomic_fetch_add(c, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS writes of this wave visible to its other lanes: wait for LDS operations
// only (s_waitcnt lgkmcnt(0); vmcnt and expcnt left at their maxima so global
// loads and stores stay in flight), then keep the compiler from moving LDS
// accesses across the point.
__device__ __forceinline__ void lds_wave_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
}

// DPP moves within rows of 16 lanes (gfx9 dpp_ctrl encodings): quad_perm
// [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2), row_half_mirror
// (lane i of each 8 <-> 7 - i), row_mirror (lane i of each 16 <-> 15 - i),
// row_ror 8 (lane ^ 8 within 16). A register-to-register move, where a
// shuffle through ds_bpermute costs an LDS round trip.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140, kDppXor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Largest value of this lane's row of 16, on every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    return fmaxf(v, dpp_f<kDppMirror>(v));
}

// Wave-wide reductions (64 lanes; every lane must be active). wave_max: the
// four row maxima combined from lanes 0, 16, 32, 48.
__device__ __forceinline__ float wave_max(float v) {
    v = row16_max(v);
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// wave_sum: the butterfly of adds by lane ^ 1, 2, 4, 8, 16, 32, in that order
// (every lane the same tree, so the same value), as DPP moves within rows (the
// 4- and 8-steps as mirrors: after the steps before, a lane's mirror partner
// holds the same value as its xor partner) and the four row sums combined as
// (r0 + r1) + (r2 + r3).
__device__ __forceinline__ double wave_sum(double v) {
    v += dpp_d<kDppXor1>(v);
    v += dpp_d<kDppXor2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    v += dpp_d<kDppMirror>(v);
    return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}

}  // namespace moe
