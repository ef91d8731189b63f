// Grouped GEMM for full 128-row expert tiles (prefill-sized buckets).
//
// Same arithmetic as expert.hpp (see there for the passages it follows and
// for the precision scheme): per Q4_K super-block b of the reduction
// dimension, P = sum_k A_hi*B + A_lo*B on v_mfma_f32_16x16x32_f16 with
// B = sub-block scale x quant (exact fp16), Q = min-term MFMA, and
// acc += sinv_row * (d_col * P - dmin_col * Q) in fp32.
//
// Work split: a workgroup owns a 128 x 128 output tile (128 rows of one
// expert's bucket, 8 repacked 16-row weight groups); its 4 waves form a 2 x 2
// grid of 64 x 64 sub-tiles (4 x 4 MFMA tiles each). Only full 128-row
// chunks of a bucket come here; the remainders go to expert_m16_kernel.
//
// Data movement, all by direct global->LDS loads (no staging registers):
//   A (staged activations): a ring of 3 LDS buffers, each a quarter
//   super-block (2 k-steps = 256 bytes of each of the 128 rows, 32 KB); each
//   lane gathers one 16-byte slot of one row, slot j of row r stored at slot
//   j ^ (r % 16) so that the 16 lanes reading one k-step/lane-group of 16 rows
//   hit 16 distinct 16-byte bank groups.
//   B (repacked quants + headers of the tile's 8 weight groups, 18 KB per
//   super-block): double-buffered per super-block, shared by the two waves of
//   a column; each wave reads its raw words per chunk and builds fragments.
//   k-step sums and 1/s of every row: double-buffered per super-block.
// The loads are issued in a fixed order, so "chunk c has landed" is a fixed
// s_waitcnt vmcnt(n) per wave (vmcnt(0) in the last super-block), followed by
// a barrier.
#pragma once
#include "common.hpp"
#include "expert.hpp"

namespace moe {

constexpr int kBigM = 128;                      // rows per tile
constexpr int kBigGroups = 8;                   // 16-row weight groups per tile (128 columns)
constexpr int kChunkBytes = 256;                // bytes of one row per A chunk (2 k-steps)
constexpr int kRing = 3;                        // A chunks: one in use, two in flight
constexpr int kABufBytes = kBigM * kChunkBytes; // 32 KB
constexpr int kBLoadsPerWave = 5;               // 4 waves x 5 x 1 KB >= 8 x 2304 B
constexpr int kBBufBytes = 4 * kBLoadsPerWave * 1024;  // 20 KB (18 KB used)
constexpr int kXsBytes = kBigM * 32;            // k-step sums of 128 rows
constexpr int kSvBytes = 256 * 4;               // 1/s slots (see issue_bx)
constexpr size_t kGemmLds = (size_t)kRing * kABufBytes + 2 * kBBufBytes + 2 * kXsBytes + 2 * kSvBytes;

__device__ __forceinline__ void load_lds16(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)lds_base, 4, 0, 0);
}

// s_waitcnt vmcnt(N) only (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void expert_gemm_kernel(const uint8_t *__restrict__ W, int ngroups, int nsb,
                                                            const int4 *__restrict__ tiles,
                                                            const int32_t *__restrict__ n_tiles,
                                                            const int32_t *__restrict__ entries, int k,
                                                            const f16 *__restrict__ a_hilo,
                                                            const f16 *__restrict__ a_xs,
                                                            const float *__restrict__ a_sinv,
                                                            float *__restrict__ outp, int out_ld) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *abuf = smem;
    uint8_t *bbuf = abuf + kRing * kABufBytes;
    uint8_t *xsbuf = bbuf + 2 * kBBufBytes;
    float *svbuf = (float *)(xsbuf + 2 * kXsBytes);

    const int tile = blockIdx.x;
    const int ntl = *n_tiles;
    const u32x4 tr = *(const u32x4 *)&tiles[tile];
    if (tile >= ntl) return;
    const int e = (int)tr.x, r0 = (int)tr.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n = lane & 15, g = lane >> 4;
    const int K = nsb * kQ4Weights;
    const int rg0 = blockIdx.y * kBigGroups;

    // ---- A gather offsets: rows 32*wave + 4*i + lane/16 (i = 0..7), slot
    // (lane%16) ^ (row%16) of each chunk (in halves; staged rows stay far
    // below 2^32 halves)
    uint32_t arow_o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 32 * wave + 4 * i + (lane >> 4);
        const int src = GATEUP ? entries[r0 + r] / k : r0 + r;
        const int slot = (lane & 15) ^ (r & 15);
        arow_o[i] = (uint32_t)src * (uint32_t)(2 * K) + (uint32_t)slot * 8u;
    }
    // k-step sums and 1/s: rows 32*wave + lane/2 and 32*wave + lane%32
    const int xr = 32 * wave + (lane >> 1);
    const int xsrc = GATEUP ? entries[r0 + xr] / k : r0 + xr;
    const f16 *xs_p = a_xs + (size_t)xsrc * nsb * 16 + (lane & 1) * 8;
    const int sr = 32 * wave + (lane & 31);
    const int ssrc = GATEUP ? entries[r0 + sr] / k : r0 + sr;
    const float *sv_p = a_sinv + (size_t)ssrc * nsb;
    // ---- B gather: flat 16-byte slot f = (wave*5 + i)*64 + lane of the
    // tile's 8 x 2304 bytes (slots beyond 8*144 reload slot 0: padding)
    const uint8_t *bsrc[kBLoadsPerWave];
#pragma unroll
    for (int i = 0; i < kBLoadsPerWave; ++i) {
        int f = (wave * kBLoadsPerWave + i) * 64 + lane;
        if (f >= kBigGroups * 144) f = 0;
        const int rg = f / 144, slot = f % 144;
        bsrc[i] = W + (size_t)((size_t)e * ngroups + rg0 + rg) * nsb * kGroupSbBytes + slot * 16;
    }

    auto issue_a = [&](int c) {  // chunk c = 4*b + q into ring buffer c % 3   (8 loads)
        const int b = c >> 2, q = c & 3;
        uint8_t *dst = abuf + (c % kRing) * kABufBytes + (32 * wave) * kChunkBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) load_lds16(a_hilo + arow_o[i] + b * 512 + q * 128, dst + i * 1024);
    };
    auto issue_bx = [&](int b) {  // B, k-step sums and 1/s of super-block b   (5 + 2 loads)
        uint8_t *bd = bbuf + (b & 1) * kBBufBytes + wave * kBLoadsPerWave * 1024;
#pragma unroll
        for (int i = 0; i < kBLoadsPerWave; ++i) load_lds16(bsrc[i] + (size_t)b * kGroupSbBytes, bd + i * 1024);
        load_lds16(xs_p + b * 16, xsbuf + (b & 1) * kXsBytes + (32 * wave) * 32);
        // 64 lanes write 64 floats per wave: lanes 32..63 repeat lanes 0..31,
        // so row r sits at slot r + 32*(r/32)
        load_lds4(sv_p + b, svbuf + (b & 1) * 256 + 64 * wave);
    };

    f32x4 acc[4][4], P[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
            P[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // prologue, in this order (scheduling barriers pin the order; the waits
    // count loads in issue order): BX(0), A(0), A(1)
    const int nchunks = 4 * nsb;
    issue_bx(0);
    __builtin_amdgcn_sched_barrier(0);
    issue_a(0);
    __builtin_amdgcn_sched_barrier(0);
    issue_a(1);
    __builtin_amdgcn_sched_barrier(0);

    for (int b = 0; b < nsb; ++b) {
        const uint8_t *bb = bbuf + (b & 1) * kBBufBytes;
        uint32_t scw[4][2], mnw[4][2];
        float dd[4], dmin[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 4 * b + q;
            // chunk c (and, for q == 0, BX(b), issued before it) has landed
            // once at most N later loads of this wave are outstanding: A(c+1)
            // (8) and, for q == 1 or 2, BX(b+1) (7). The last super-block
            // waits for everything.
            if (b == nsb - 1)
                wait_vm<0>();
            else if (q == 1 || q == 2)
                wait_vm<15>();
            else
                wait_vm<8>();
            __builtin_amdgcn_s_waitcnt(0xC07F);  // own LDS reads done before the buffer is refilled
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (c + 2 < nchunks) issue_a(c + 2);
            __builtin_amdgcn_sched_barrier(0);
            if (q == 0 && b + 1 < nsb) issue_bx(b + 1);
            __builtin_amdgcn_sched_barrier(0);

            if (q == 0) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const u32x4 hdr = *(const u32x4 *)(bb + (wn * 4 + cb) * kGroupSbBytes + kGroupQsBytes + n * 16);
                    unpack_scales(hdr, scw[cb], mnw[cb]);
                    dd[cb] = half_bits_to_float(hdr.x & 0xFFFFu);
                    dmin[cb] = half_bits_to_float(hdr.x >> 16);
                }
            }
            // raw quant words of this chunk: half p = q/2, chunk-in-half q%2
            u32x2 qw[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                qw[cb] = *(const u32x2 *)(bb + (wn * 4 + cb) * kGroupSbBytes + (q >> 1) * 1024 + lane * 16 +
                                          (q & 1) * 8);

            const uint8_t *ab = abuf + (c % kRing) * kABufBytes;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int ks = 2 * q + s2;
                f16x8 Bf[4];
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const f16 scv = (f16)(float)byte_of(scw[cb], ks);
                    const f16x2 sc2 = {scv, scv};
                    const f16x2 neg2 = sc2 * (f16)(-1024.f);
                    Bf[cb] = q_times_scale(qw[cb].x, qw[cb].y, s2, sc2, neg2);
                }
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int r = wm * 64 + rb * 16 + n;  // A row of this lane (r % 16 == n)
                    const int jh = (s2 * 8 + 2 * g) ^ n;
                    const int jl = (s2 * 8 + 2 * g + 1) ^ n;
                    const f16x8 Ahi = *(const f16x8 *)(ab + r * kChunkBytes + jh * 16);
                    const f16x8 Alo = *(const f16x8 *)(ab + r * kChunkBytes + jl * 16);
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) {
                        P[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bf[cb], P[rb][cb], 0, 0, 0);
                        P[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bf[cb], P[rb][cb], 0, 0, 0);
                    }
                }
            }
        }

        // super-block b complete: min term and epilogue
        const uint8_t *xsb = xsbuf + (b & 1) * kXsBytes;
        const float *svb = svbuf + (b & 1) * 256;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int r = wm * 64 + rb * 16 + n;
            const f16x4 Am = *(const f16x4 *)(xsb + r * 32 + g * 8);
            const int ro = wm * 64 + rb * 16 + 4 * g;  // first output row of this lane
            const f32x4 sv = *(const f32x4 *)(svb + ro + 32 * (ro >> 5));
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                f16x4 Bm;
#pragma unroll
                for (int i = 0; i < 4; ++i) Bm[i] = (f16)(float)byte_of(mnw[cb], 4 * (g & 1) + i);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 Q = __builtin_amdgcn_mfma_f32_16x16x16f16(Am, Bm, zero, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[rb][cb][i] += sv[i] * (dd[cb] * P[rb][cb][i] - dmin[cb] * Q[i]);
                P[rb][cb] = zero;
            }
        }
    }

    // results: rows r0 + wm*64 + rb*16 + 4g + i, columns of weight group
    // rg0 + wn*4 + cb
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int rg = rg0 + wn * 4 + cb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t row = (size_t)r0 + wm * 64 + rb * 16 + 4 * g + i;
                if (GATEUP) {
                    const float u = __shfl_xor(acc[rb][cb][i], 8, kWave);
                    if (n < 8) outp[row * out_ld + rg * 8 + n] = silu_f(acc[rb][cb][i]) * u;
                } else {
                    outp[row * out_ld + rg * kRowGroup + n] = acc[rb][cb][i];
                }
            }
        }
    }
}

}  // namespace moe
