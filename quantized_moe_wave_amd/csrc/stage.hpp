// Activation staging for the MFMA expert kernels.
//
// The expert matmuls run on fp16 MFMA with exact-integer weight operands
// (q * scale <= 945 is exact in fp16). fp16 alone would carry only 11 bits of
// each activation, so every activation row is split, per Q4_K super-block of
// 256 columns, into a power-of-two scale s and two fp16 parts:
//     x * s = hi + lo,   hi = fp16(x * s),   lo = fp16(x * s - hi)
// which keeps ~22 bits. s puts the block's largest |x * s| just under 2^10, so
// the 32-column sums used for the Q4_K min term stay below 2^15 in fp16 too.
// The kernels multiply each super-block's partial product by sinv = 1/s, which
// is exact. Layout: see common.hpp.
//
// Grid: one wave per (row, super-block), 4 waves per workgroup. Lanes 0..31
// each handle one 8-column fragment.
#pragma once
#include "common.hpp"

namespace moe {

// One wave stages super-block b of one row: src points at the row's fp32
// values (K = nsb*256 columns); lanes 0..31 each own one 8-column fragment.
__device__ __forceinline__ void stage_row_sb(const float *__restrict__ src, int nsb, int b, f16 *__restrict__ hilo_row,
                                             f16 *__restrict__ xs_row, float *__restrict__ sinv_row) {
    const int lane = threadIdx.x & 63;
    const int f = lane & 31;  // fragment: k-step s = f / 4, lane group g = f % 4
    const int s = f >> 2, g = f & 3;
    const float *p = src + b * kQ4Weights + s * 32 + g * 8;
    float v[8];
    {
        float4 a = *(const float4 *)p;
        float4 c = *(const float4 *)(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = wave_max(lane < 32 ? m : 0.f);
    int ex = 0;
    if (m > 0.f) (void)frexpf(m, &ex);  // m < 2^ex
    int se = 10 - ex;
    se = se > 100 ? 100 : (se < -100 ? -100 : se);
    if (!(m > 0.f) || !(m < INFINITY)) se = 0;
    const float sc = ldexpf(1.f, se);

    f16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float y = v[perm8(e)] * sc;  // exact: power-of-two scaling
        const f16 h = (f16)y;
        hi[e] = h;
        lo[e] = (f16)(y - (float)h);
    }
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) part += v[i] * sc;
    // sum of the 32 columns of k-step s: lanes 4s .. 4s+3
    part += __shfl_xor(part, 1, kWave);
    part += __shfl_xor(part, 2, kWave);
    if (lane < 32) {
        f16 *dst = hilo_row + (size_t)((b * 8 + s) * 4 + g) * 16;
        *(f16x8 *)dst = hi;
        *(f16x8 *)(dst + 8) = lo;
        if (g == 0) {
            const f16 h = (f16)part;
            f16 *xd = xs_row + (size_t)b * 16;
            xd[s] = h;
            xd[8 + s] = (f16)(part - (float)h);
        }
        if (lane == 0) sinv_row[b] = ldexpf(1.f, -se);
    }
}

__global__ __launch_bounds__(256) void stage_kernel(const float *__restrict__ src, int rows, int K, int ld_src,
                                                    f16 *__restrict__ hilo, f16 *__restrict__ xs,
                                                    float *__restrict__ sinv) {
    const int nsb = K / kQ4Weights;
    const long unit = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= (long)rows * nsb) return;
    const int row = (int)(unit / nsb), b = (int)(unit % nsb);
    stage_row_sb(src + (size_t)row * ld_src, nsb, b, hilo + (size_t)row * (2 * K), xs + (size_t)row * nsb * 16,
                 sinv + (size_t)row * nsb);
}

}  // namespace moe
