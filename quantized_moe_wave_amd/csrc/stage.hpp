// Activation staging for the MFMA expert kernels.
//
// The expert matmuls run on fp16 MFMA with exact-integer weight operands
// (q * scale <= 945 is exact in fp16). fp16 alone would carry only 11 bits of
// each activation, so every activation row is split, per Q4_K super-block of
// 256 columns, into a power-of-two scale s and two fp16 parts:
//     x * s = hi + lo,   hi = fp16(x * s),   lo = fp16(x * s - hi)
// which keeps ~22 bits. s puts the block's largest |x * s| just under 2^10, so
// the 32-column sums used for the Q4_K min term stay below 2^15 in fp16 too.
// The kernels multiply the partial products by sinv = 1/s, which is exact.
// The decode path scales each super-block on its own; the general path
// (stage_kernel) uses one scale per row. With Q8_K-style activations both
// stage the codes of each super-block instead (hi = q, lo = 0, 1/s replaced
// by the block's d). Layout: see common.hpp.
#pragma once
#include "common.hpp"

namespace moe {

// Power-of-two exponent se for a block whose largest magnitude is m:
// |x * 2^se| < 2^10 (se clamped to +-100; 0 for an all-zero or non-finite m).
__device__ __forceinline__ int stage_exponent(float m) {
    int ex = 0;
    if (m > 0.f) (void)frexpf(m, &ex);  // m < 2^ex
    int se = 10 - ex;
    se = se > 100 ? 100 : (se < -100 ? -100 : se);
    if (!(m > 0.f) || !(m < INFINITY)) se = 0;
    return se;
}

// One wave stages super-block b of one row with scale 2^se (se < -1000: use
// the block's own scale): src points at the row's fp32 values (K = nsb*256
// columns); lanes 0..31 each own one 8-column fragment.
// With nw (the block's RMSNorm weight, or null) the staged values are the
// normalised row: fp32(src[c] * nw[c] * inv_rms), the product in double.
// q8: Q8_K-style codes instead (q8_code: per super-block, amax = max |v|,
// q = rint(v * (127 / amax)) in [-127, 127], all in fp32); hi holds q (exact
// in fp16), lo 0, the sums are sums of q (exact), and 1/s is d = amax / 127.
__device__ __forceinline__ float q8_code(float v, float iscale) {
    return fminf(fmaxf(rintf(v * iscale), -127.f), 127.f);
}
__device__ __forceinline__ void stage_row_sb(const float *__restrict__ src, int nsb, int b, f16 *__restrict__ hilo_row,
                                             f16 *__restrict__ xs_row, float *__restrict__ sinv_row,
                                             int se = -10000, const float *__restrict__ nw = nullptr,
                                             double inv_rms = 1.0, bool q8 = false) {
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
    if (nw) {
        const float *q = nw + b * kQ4Weights + s * 32 + g * 8;
        const float4 a = *(const float4 *)q;
        const float4 c = *(const float4 *)(q + 4);
        const float w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)((double)v[i] * w[i] * inv_rms);
    }
    float q8_d = 0.f;
    if (q8) {
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
        m = wave_max(lane < 32 ? m : 0.f);
        const float is = m > 0.f ? 127.f / m : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = q8_code(v[i], is);  // codes, staged with scale 1 below
        q8_d = m / 127.f;
        se = 0;
    } else if (se < -1000) {
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
        se = stage_exponent(wave_max(lane < 32 ? m : 0.f));
    }
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
    part += dpp_f<kDppXor1>(part);
    part += dpp_f<kDppXor2>(part);
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
        if (lane == 0) sinv_row[b] = q8 ? q8_d : ldexpf(1.f, -se);
    }
}

// Staging of a whole row with one scale, by one wave (the grouped GEMM
// applies the row's 1/s once, after its last super-block; the
// per-super-block 1/s entries all hold the row's value). The row's largest
// magnitude sets s. Same fragments, rounding and sums as stage_row_sb, but
// all 64 lanes work: lanes 0-31 take the even super-block of each pair, lanes
// 32-63 the odd one. Rows of up to 2 * kStageRegPairs super-blocks are read
// once (every load issued before the first use); longer rows are read twice.
constexpr int kStageRegPairs = 8;

// Pairs of super-blocks of a row in registers: slot i holds pair p = p0 +
// ps * i (super-block 2p on lanes 0-31 and 2p + 1 on lanes 32-63, 8 columns
// per lane). A whole row (p0 = 0, ps = 1) takes up to kStageRegPairs pairs;
// a workgroup of 4 waves splits a row as p0 = wave, ps = 4.
template <int SLOTS>
struct StagedPairs {
    float4 va[SLOTS], vb[SLOTS];
    int p0, ps;
};
using StagedRow = StagedPairs<kStageRegPairs>;
constexpr int kStagePartSlots = kStageRegPairs / 4;  // one wave's slots when 4 waves share a row
using StagedPart = StagedPairs<kStagePartSlots>;

// Issue the loads of pairs p0, p0 + ps, ... of a row into sp (no wait: the
// caller may do other work while they are in flight). Requires the row's
// (nsb + 1) / 2 pairs to fit: p0 + ps * SLOTS >= (nsb + 1) / 2.
template <int SLOTS>
__device__ __forceinline__ void stage_pairs_load(const float *__restrict__ r, int nsb, int p0, int ps,
                                                 StagedPairs<SLOTS> &sp) {
    const int lane = threadIdx.x & 63;
    const int f = lane & 31, hb = lane >> 5;
    const int off = (f >> 2) * 32 + (f & 3) * 8;
    const int npairs = (nsb + 1) >> 1;
    sp.p0 = p0;
    sp.ps = ps;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
        const int p = p0 + ps * i;
        if (p < npairs) {
            const int b = min(2 * p + hb, nsb - 1);  // an odd tail repeats the last block (not stored)
            sp.va[i] = *(const float4 *)(r + b * kQ4Weights + off);
            sp.vb[i] = *(const float4 *)(r + b * kQ4Weights + off + 4);
        }
    }
}

// A whole row (stage_pairs_load with p0 = 0, ps = 1). Requires
// (nsb + 1) / 2 <= kStageRegPairs.
__device__ __forceinline__ void stage_row_load(const float *__restrict__ r, int nsb, StagedRow &sr) {
    stage_pairs_load(r, nsb, 0, 1, sr);
}

// The 8 columns (a, c) of super-block b owned by this lane, scaled by sc:
// fp16 hi/lo in fragment order, the k-step's 32-column sum (over the 4 lanes
// of the k-step), and 1/s. All lanes must call it together.
__device__ __forceinline__ void stage_emit(int b, float4 a, float4 c, float sc, float sinv, int nsb,
                                           f16 *__restrict__ hilo_row, f16 *__restrict__ xs_row,
                                           float *__restrict__ sinv_row) {
    const int f = threadIdx.x & 31, s = f >> 2, g = f & 3;
    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
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
    // sum of the 32 columns of k-step s: lanes 4s .. 4s+3 of this half
    part += dpp_f<kDppXor1>(part);
    part += dpp_f<kDppXor2>(part);
    if (b < nsb) {
        f16 *dst = hilo_row + (size_t)((b * 8 + s) * 4 + g) * 16;
        *(f16x8 *)dst = hi;
        *(f16x8 *)(dst + 8) = lo;
        if (g == 0) {
            const f16 h = (f16)part;
            f16 *xd = xs_row + (size_t)b * 16;
            xd[s] = h;
            xd[8 + s] = (f16)(part - (float)h);
        }
        if (f == 0) sinv_row[b] = sinv;
    }
}

// The block's RMSNorm on pairs loaded by stage_pairs_load, with its weight gp
// (loaded the same way) and 1/rms r: each value becomes fp32(x * g * r), the
// products in double.
template <int SLOTS>
__device__ __forceinline__ void staged_pairs_normalise(StagedPairs<SLOTS> &sp, const StagedPairs<SLOTS> &gp, int nsb,
                                                       double r) {
    const int npairs = (nsb + 1) >> 1;
    auto nz = [&](float4 &v, const float4 &g) {
        v.x = (float)((double)v.x * g.x * r);
        v.y = (float)((double)v.y * g.y * r);
        v.z = (float)((double)v.z * g.z * r);
        v.w = (float)((double)v.w * g.w * r);
    };
    // pair by pair (a scheduling fence between pairs), so that the double
    // intermediates of one pair only are live at a time
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
        if (sp.p0 + sp.ps * i < npairs) {
            nz(sp.va[i], gp.va[i]);
            nz(sp.vb[i], gp.vb[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}
__device__ __forceinline__ void staged_row_normalise(StagedRow &sr, const StagedRow &gr, int nsb, double r) {
    staged_pairs_normalise(sr, gr, nsb, r);
}

// This lane's sum of squares (each square exact in double) over the values
// it holds, the repeated block of an odd tail left out.
template <int SLOTS>
__device__ __forceinline__ double staged_pairs_sumsq(const StagedPairs<SLOTS> &sp, int nsb) {
    const int hb = (threadIdx.x & 63) >> 5;
    const int npairs = (nsb + 1) >> 1;
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
        const int p = sp.p0 + sp.ps * i;
        if (p < npairs && 2 * p + hb < nsb) {
            const float v[8] = {sp.va[i].x, sp.va[i].y, sp.va[i].z, sp.va[i].w,
                                sp.vb[i].x, sp.vb[i].y, sp.vb[i].z, sp.vb[i].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += (double)v[e] * v[e];
        }
    }
    return ss;
}

// Largest value over the 32 lanes of this lane's half of the wave.
__device__ __forceinline__ float half_wave_max(float m) {
    m = row16_max(m);
    const float lo = fmaxf(readlane_f(m, 0), readlane_f(m, 16)), hi = fmaxf(readlane_f(m, 32), readlane_f(m, 48));
    return (threadIdx.x & 32) ? hi : lo;
}

// Q8_K-style codes of one super-block held as 8 columns per lane by a half
// wave (q8_code over the block's amax, all in fp32, as stage_row_sb), stored
// with scale 1 and d = amax / 127 in place of 1/s.
__device__ __forceinline__ void stage_emit_q8(int b, float4 a, float4 c, int nsb, f16 *__restrict__ hilo_row,
                                              f16 *__restrict__ xs_row, float *__restrict__ sinv_row) {
    float m = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                    fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w))));
    m = half_wave_max(m);
    const float is = m > 0.f ? 127.f / m : 0.f;
    a = float4{q8_code(a.x, is), q8_code(a.y, is), q8_code(a.z, is), q8_code(a.w, is)};
    c = float4{q8_code(c.x, is), q8_code(c.y, is), q8_code(c.z, is), q8_code(c.w, is)};
    stage_emit(b, a, c, 1.f, m / 127.f, nsb, hilo_row, xs_row, sinv_row);
}

// This lane's largest magnitude over the values it holds (the repeated block
// of an odd tail may count: it repeats a value of the row).
template <int SLOTS>
__device__ __forceinline__ float staged_pairs_absmax(const StagedPairs<SLOTS> &sp, int nsb) {
    const int npairs = (nsb + 1) >> 1;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
        if (sp.p0 + sp.ps * i < npairs) {
            const float4 a = sp.va[i], c = sp.vb[i];
            m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                               fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w)))));
        }
    }
    return m;
}

// Store the held pairs with the row's scale 2^se (q8: Q8_K codes per
// super-block instead, stage_emit_q8, and se unused).
template <int SLOTS>
__device__ __forceinline__ void staged_pairs_emit(const StagedPairs<SLOTS> &sp, int nsb, int se,
                                                  f16 *__restrict__ hilo_row, f16 *__restrict__ xs_row,
                                                  float *__restrict__ sinv_row, bool q8) {
    const int hb = (threadIdx.x & 63) >> 5;
    const int npairs = (nsb + 1) >> 1;
    const float sc = ldexpf(1.f, se), sinv = ldexpf(1.f, -se);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
        const int p = sp.p0 + sp.ps * i;
        if (p < npairs) {
            if (q8)
                stage_emit_q8(2 * p + hb, sp.va[i], sp.vb[i], nsb, hilo_row, xs_row, sinv_row);
            else
                stage_emit(2 * p + hb, sp.va[i], sp.vb[i], sc, sinv, nsb, hilo_row, xs_row, sinv_row);
        }
    }
}

// Scale and store a row loaded by stage_row_load (q8: Q8_K codes per
// super-block instead, stage_emit_q8).
__device__ __forceinline__ void stage_row_store(const StagedRow &sr, int nsb, f16 *__restrict__ hilo_row,
                                                f16 *__restrict__ xs_row, float *__restrict__ sinv_row,
                                                bool q8 = false) {
    const int se = q8 ? 0 : stage_exponent(wave_max(staged_pairs_absmax(sr, nsb)));
    staged_pairs_emit(sr, nsb, se, hilo_row, xs_row, sinv_row, q8);
}

// Load, scale and store one row (one wave; q8: Q8_K codes per super-block).
__device__ __forceinline__ void stage_row_wave(const float *__restrict__ r, int nsb, f16 *__restrict__ hilo_row,
                                               f16 *__restrict__ xs_row, float *__restrict__ sinv_row,
                                               bool q8 = false) {
    const int npairs = (nsb + 1) >> 1;
    if (npairs <= kStageRegPairs) {
        StagedRow sr;
        stage_row_load(r, nsb, sr);
        stage_row_store(sr, nsb, hilo_row, xs_row, sinv_row, q8);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int f = lane & 31, hb = lane >> 5;
    const int off = (f >> 2) * 32 + (f & 3) * 8;
    if (q8) {
        for (int p = 0; p < npairs; ++p) {
            const int b = 2 * p + hb, bl = min(b, nsb - 1);
            stage_emit_q8(b, *(const float4 *)(r + bl * kQ4Weights + off),
                          *(const float4 *)(r + bl * kQ4Weights + off + 4), nsb, hilo_row, xs_row, sinv_row);
        }
        return;
    }
    float m = 0.f;
    for (int c = lane * 4; c < nsb * kQ4Weights; c += 256) {
        const float4 a = *(const float4 *)(r + c);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
    }
    const int se = stage_exponent(wave_max(m));
    const float sc = ldexpf(1.f, se), sinv = ldexpf(1.f, -se);
    for (int p = 0; p < npairs; ++p) {
        const int b = 2 * p + hb, bl = min(b, nsb - 1);
        stage_emit(b, *(const float4 *)(r + bl * kQ4Weights + off), *(const float4 *)(r + bl * kQ4Weights + off + 4),
                   sc, sinv, nsb, hilo_row, xs_row, sinv_row);
    }
}

// One wave per row (stage_row_wave; q8: Q8_K codes).
__global__ __launch_bounds__(256) void stage_kernel(const float *__restrict__ src, int rows, int K, int ld_src,
                                                    f16 *__restrict__ hilo, f16 *__restrict__ xs,
                                                    float *__restrict__ sinv, int q8) {
    const int nsb = K / kQ4Weights;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    stage_row_wave(src + (size_t)row * ld_src, nsb, hilo + (size_t)row * (2 * K), xs + (size_t)row * nsb * 16,
                   sinv + (size_t)row * nsb, q8 != 0);
}

}  // namespace moe
