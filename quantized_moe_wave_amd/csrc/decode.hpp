// Small-batch (decode) path: T <= kSmallT tokens per call, three launches.
//
//   router_small_kernel       router logits (fp64) and x staging
//   gateup_pair_kernel        one (token, slot) pair x one 16-row weight group
//                             per workgroup, its waves splitting the
//                             reduction dimension; the workgroup finds the
//                             pair's expert itself (top-k of its token)
//   down_combine_small_kernel down projection of one token's k experts fused
//                             with the router-weighted sum (slot order), the
//                             experts and weights handed over by the gate/up
//                             launch; one extra workgroup writes the routing
//                             outputs (indices, weights, bucket layout)
//
// Every gate/up workgroup recomputing its token's top-k from the logits (a few
// hundred 64-bit key compares per thread) is cheaper at decode than handing the
// choice between workgroups of one launch, which costs several dependent memory
// round trips; across the launch boundary to down/combine the hand-off is free
// (its loads ride with the h loads), so that launch ranks nothing.
//
// Same arithmetic as the general path (router.hpp, stage.hpp, expert.hpp); the
// layer's definition and the readings are cited there. Only the work split
// differs: at decode every stage is latency-bound, so the point is fewer
// launches and more independent loads in flight per wave.
#pragma once
#include "common.hpp"
#include "expert.hpp"
#include "norm.hpp"
#include "router.hpp"
#include "stage.hpp"

namespace moe {

constexpr int kSmallT = 4;

// Exclusive prefix sum over the 256 threads of a workgroup; *total = sum.
// red must hold 4 ints; contains two barriers.
__device__ __forceinline__ int block_exclusive_scan(int v, int *red, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += red[w];
    *total = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return before + x - v;
}

// One wave per expert (waves 0 .. E-1 of the grid) and one per (token,
// super-block) staging unit of x (the T*nsb waves after them), so that no
// wave does both one after the other.
// norm_w (the block's RMSNorm weight, or null): x holds the residual stream
// and every value is used normalised, fp32(x * norm_w * inv_rms), each wave
// computing the 1/rms of the rows it reads (row_inv_rms).
template <int TT>
__device__ __forceinline__ void logits_small_body(const float *__restrict__ x, const float *__restrict__ wr,
                                                  const float *__restrict__ bias, int T, int H, int E,
                                                  double *__restrict__ logits, f16 *__restrict__ x_hilo,
                                                  f16 *__restrict__ x_xs, float *__restrict__ x_sinv,
                                                  const float *__restrict__ norm_w, double eps, int q8) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nsb = H / kQ4Weights;
    const int wpb = blockDim.x >> 6;  // waves per workgroup
    const int nw = gridDim.x * wpb;

    for (int u = blockIdx.x * wpb + wave - E; u < T * nsb; u += nw) {
        if (u < 0) break;  // an expert wave
        const int t = u / nsb, b = u % nsb;
        const double ir = norm_w ? row_inv_rms(x + (size_t)t * H, H, eps) : 1.0;
        stage_row_sb(x + (size_t)t * H, nsb, b, x_hilo + (size_t)t * 2 * H, x_xs + (size_t)t * nsb * 16,
                     x_sinv + (size_t)t * nsb, -10000, norm_w, ir, q8 != 0);
    }

    // Loads are unconditional (chunk indices clamped) so that all of a wave's
    // loads are in flight together; out-of-range terms are skipped. TT = T
    // (one instance per token count): no wave loads a row twice.
    for (int e = blockIdx.x * wpb + wave; e < E; e += nw) {
        double acc[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = 0.0;
        // 1/rms of each token's row: from the chunk registers below when the
        // whole row fits one pass of them (nsb <= 8), else read ahead here
        const bool rms_ahead = norm_w && nsb > 8;
        double ir[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) ir[t] = (rms_ahead && t < T) ? row_inv_rms(x + (size_t)t * H, H, eps) : 1.0;
        const float *wrow = wr + (size_t)e * H;
        for (int c0 = 0; c0 < nsb; c0 += 8) {
            float4 wv[8], xv[TT][8];
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[i] = *(const float4 *)(wrow + min(c0 + i, nsb - 1) * kQ4Weights + lane * 4);
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    xv[t][i] = *(const float4 *)(x + (size_t)min(t, T - 1) * H + min(c0 + i, nsb - 1) * kQ4Weights +
                                                 lane * 4);
            if (norm_w) {
                float4 gv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) gv[i] = *(const float4 *)(norm_w + min(c0 + i, nsb - 1) * kQ4Weights + lane * 4);
                if (!rms_ahead) {
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        if (t < T) {
                            double ss = 0.0;
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                if (i < nsb) {
                                    ss += (double)xv[t][i].x * xv[t][i].x;
                                    ss += (double)xv[t][i].y * xv[t][i].y;
                                    ss += (double)xv[t][i].z * xv[t][i].z;
                                    ss += (double)xv[t][i].w * xv[t][i].w;
                                }
                            }
                            ir[t] = 1.0 / sqrt(wave_sum(ss) / (double)H + eps);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        if (t >= T) continue;
                        const float4 g4 = gv[i];
                        xv[t][i].x = (float)((double)xv[t][i].x * g4.x * ir[t]);
                        xv[t][i].y = (float)((double)xv[t][i].y * g4.y * ir[t]);
                        xv[t][i].z = (float)((double)xv[t][i].z * g4.z * ir[t]);
                        xv[t][i].w = (float)((double)xv[t][i].w * g4.w * ir[t]);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (t < T && c0 + i < nsb) {
                        double a = acc[t];
                        a = fma((double)wv[i].x, (double)xv[t][i].x, a);
                        a = fma((double)wv[i].y, (double)xv[t][i].y, a);
                        a = fma((double)wv[i].z, (double)xv[t][i].z, a);
                        a = fma((double)wv[i].w, (double)xv[t][i].w, a);
                        acc[t] = a;
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t < T) {
                double s = wave_sum(acc[t]);
                if (lane == 0) {
                    if (bias) s += (double)bias[e];
                    logits[(size_t)t * E + e] = s;
                }
            }
        }
    }
}

// Rank-based top-k of one token for a whole workgroup (E <= 256): the k
// winners' experts and logits land in LDS at their slot. Same rule as the
// other selections (rank_key: larger logit first, equal logits to the lower
// index; NaN counts as -inf). The keys are padded with -inf keys to 256
// entries (a pad never beats a real candidate: it is not larger, and on a tie
// its index is higher). Candidate c's rank counts the keys above its own.
// Every lane of a wave walks the same range of j, so each LDS read is a
// broadcast: for E <= 128 candidate c = tid % 128 and the workgroup's first
// 128 * P threads (P = 2 or 4 parts, as many as it has) count 128 / P keys
// each, the parts' counts summed by part 0; for larger E candidate c = tid
// counts all 256. The thread that writes a winner is the one that loaded it
// (tid == c). lg: 256 LDS words of 8 bytes, which hold the keys.
__device__ __forceinline__ void topk_block(const double *lrow, int E, int k, double *lg, int *sel_e,
                                           double *sel_v) {
    __shared__ int rk_part[3][128];
    uint64_t *keys = (uint64_t *)lg;
    const int tid = threadIdx.x;
    const bool act = tid < 256;  // threads past 256 only join the barriers (and count, for E <= 128)
    double v = -INFINITY;
    if (act) {
        const int c = min(tid, E - 1);
        const double x = lrow[c];
        v = (tid < E && x == x) ? x : -INFINITY;
        keys[tid] = rank_key(v, tid);
    }
    __syncthreads();
    const bool split = E <= 128;
    const int nparts = (int)blockDim.x >= 512 ? 4 : 2;  // workgroups of 256 threads or more
    const int part = split ? tid >> 7 : 0;
    const bool on = split ? part < nparts : act;
    const int span = split ? 128 / nparts : 256;
    const int c = split ? (tid & 127) : (tid & 255);
    const int j0 = part * span;
    const int nj = on ? span : 0;
    const uint64_t key = keys[c];
    int rank = 0;
    for (int jj = 0; jj < nj; jj += 8) {
        uint64_t b[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const ulonglong2 p2 = *(const ulonglong2 *)&keys[j0 + jj + 2 * q];
            b[2 * q] = p2.x;
            b[2 * q + 1] = p2.y;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) rank += (int)(b[q] > key);
    }
    if (on && split && part > 0) rk_part[part - 1][c] = rank;
    __syncthreads();
    if (on && c < E && part == 0) {
        for (int q = 1; q < (split ? nparts : 1); ++q) rank += rk_part[q - 1][c];
        if (rank < k) {
            sel_e[rank] = c;
            sel_v[rank] = v;
        }
    }
    __syncthreads();
}

// Routing outputs of all T tokens: idx/w per token, then the stable bucket
// layout of the T*k <= 256 pairs, the latter by wave 0 alone (lane l owns
// experts 4l .. 4l+3, E <= 256).
__device__ __forceinline__ void routing_outputs_small(const double *logits, int T, int E, int k, double *lg, int *sel_e,
                                                   double *sel_v, int32_t *idx_out, float *w_out, int32_t *counts,
                                                   int32_t *offsets, int32_t *entries, int32_t *pos) {
    __shared__ int sidx[kSmallT * kMaxTopK];
    __shared__ int off_l[kRankMaxExperts];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int t = 0; t < T; ++t) {
        topk_block(logits + (size_t)t * E, E, k, lg, sel_e, sel_v);
        if (wave == 0) {
            const double ex = (lane < k) ? exp(sel_v[lane] - sel_v[0]) : 0.0;
            const double z = wave_sum(ex);
            if (lane < k) {
                idx_out[(size_t)t * k + lane] = sel_e[lane];
                w_out[(size_t)t * k + lane] = (float)(ex / z);
                sidx[t * k + lane] = sel_e[lane];
            }
        }
        if (t + 1 < T) __syncthreads();  // sel_e / sel_v / lg are reused by the next token
    }
    if (wave != 0) return;  // the bucket layout is wave 0's alone
    lds_wave_sync();
    const int S = T * k;
    // counts of experts 4*lane .. 4*lane + 3
    int cnt[4] = {0, 0, 0, 0};
    for (int s = 0; s < S; ++s) {
        const int e = sidx[s];  // broadcast
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt[i] += (int)(e == 4 * lane + i);
    }
    const int lsum = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    int incl = lsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    int run = incl - lsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * lane + i;
        if (e < E) {
            counts[e] = cnt[i];
            offsets[e] = run;
            off_l[e] = run;
        }
        run += cnt[i];
    }
    if (lane == 63) offsets[E] = incl;  // = S
    lds_wave_sync();
    // pair s: its place in expert e's bucket is the number of earlier pairs of e
    for (int s0 = 0; s0 < S; s0 += 64) {
        const int s = s0 + lane;
        const int e = s < S ? sidx[s] : -1;
        int r = 0;
        for (int q = 0; q < s0 + 64 && q < S; ++q) r += (int)((q < s) & (sidx[q] == e));
        if (s < S) {
            const int p = off_l[e] + r;
            entries[p] = s;
            pos[s] = p;
        }
    }
}

// Router of the small path: logits (fp64) and the staged x rows; grid of
// E + T*nsb one-wave workgroups. The top-k
// is recomputed from the logits by every workgroup of the next two launches
// (each needs only its own token's choice), which is cheaper than handing the
// choice from workgroup to workgroup.
template <int TT>
__global__ __launch_bounds__(64) void router_small_kernel(const float *__restrict__ x, const float *__restrict__ wr,
                                                           const float *__restrict__ bias, int T, int H, int E,
                                                           double *__restrict__ logits, f16 *__restrict__ x_hilo,
                                                           f16 *__restrict__ x_xs, float *__restrict__ x_sinv,
                                                           const float *__restrict__ norm_w, double eps, int q8) {
    logits_small_body<TT>(x, wr, bias, T, H, E, logits, x_hilo, x_xs, x_sinv, norm_w, eps, q8);
}

constexpr int kSmallMaxH = 4096;  // hidden sizes the small path stages in LDS

// One super-block of one 16x16 tile, added to acc:
//   P = sum over the 8 k-steps of A (hi, then lo) x B, B = sub-block scale x
//       quant (exact fp16) built from this lane's repacked quant words q0, q1;
//   Q = min-term MFMA of am (k-step sums, hi | lo) with the mins;
//   acc[i] += sv[i] * (d * P[i] - dmin * Q[i]) with d, dmin of this lane's
//   weight row (header hdr). afrag(s, hi, lo) supplies A's k-step s.
// At decode this is a wave's whole share of the work, so its latency is what
// counts: the hi and lo products go to two accumulators, so that no MFMA
// waits for the one just before it, and A of k-step s+1 is read (from LDS)
// while k-step s runs; the two are summed before the scales (two, not four:
// the gate/up kernel must stay within 80 registers to keep 6 waves per SIMD).
template <typename AF>
__device__ __forceinline__ void mma_sb_fn(const u32x4 &q0, const u32x4 &q1, const u32x4 &hdr, AF afrag, f16x4 am,
                                          const float sv[4], int g, f32x4 &acc) {
    uint32_t sc[2], mn[2];
    unpack_scales(hdr, sc, mn);
    const float dd = half_bits_to_float(hdr.x & 0xFFFFu);
    const float dmin = half_bits_to_float(hdr.x >> 16);
    f32x4 Ph = {0.f, 0.f, 0.f, 0.f}, Pl = {0.f, 0.f, 0.f, 0.f};
    f16x8 ahi[2], alo[2];
    afrag(0, ahi[0], alo[0]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (s + 1 < 8) afrag(s + 1, ahi[(s + 1) & 1], alo[(s + 1) & 1]);
        const u32x4 &q = (s < 4) ? q0 : q1;
        const int cc = (s >> 1) & 1;
        const uint32_t dA = cc ? q.z : q.x;
        const uint32_t dB = cc ? q.w : q.y;
        const f16 scv = (f16)(float)byte_of(sc, s);
        const f16x2 sc2 = {scv, scv};
        const f16x2 neg2 = sc2 * (f16)(-1024.f);
        const f16x8 B = q_times_scale(dA, dB, s & 1, sc2, neg2);
        Ph = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[s & 1], B, Ph, 0, 0, 0);
        Pl = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[s & 1], B, Pl, 0, 0, 0);
    }
    f16x4 Bm;
#pragma unroll
    for (int i = 0; i < 4; ++i) Bm[i] = (f16)(float)byte_of(mn, 4 * (g & 1) + i);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 Q = __builtin_amdgcn_mfma_f32_16x16x16f16(am, Bm, zero, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[i] += sv[i] * (dd * (Ph[i] + Pl[i]) - dmin * Q[i]);
    }
}

// Grid (T*k pairs, I/8 row groups), kGpWaves waves. Pair p = t*k + j: the
// workgroup stages token t's A row in LDS and computes the 8 gate + 8 up rows
// of row group rg of expert idx[p] for that single row (MFMA row 0), the waves
// splitting the super-blocks (one each at H = 2048, so that each wave's chain
// of dependent MFMAs is one super-block long). Output h[p][I] = SiLU(gate) * up;
// the first row group's workgroup also writes dsel[p] (the pair's expert) and
// dw[p] (its renormalised router weight) for down_combine_small_kernel.
constexpr int kGpWaves = 8;

__global__ __launch_bounds__(kGpWaves * 64) void gateup_pair_kernel(const uint8_t *__restrict__ GU, int ngroups, int nsb,
                                                          const double *__restrict__ logits, int E, int k,
                                                          const f16 *__restrict__ x_hilo, const f16 *__restrict__ x_xs,
                                                          const float *__restrict__ x_sinv, float *__restrict__ h,
                                                          int I, int32_t *__restrict__ dsel, float *__restrict__ dw) {
    __shared__ __attribute__((aligned(16))) f16 arow[2 * kSmallMaxH];
    __shared__ __attribute__((aligned(16))) f16 axs[kSmallMaxH / kQ4Weights * 16];
    __shared__ float asv[kSmallMaxH / kQ4Weights];
    __shared__ f32x4 red[kGpWaves][64];
    __shared__ __attribute__((aligned(16))) double lg[kRankMaxExperts];
    __shared__ int sel_e[kMaxTopK];
    __shared__ double sel_v[kMaxTopK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = blockIdx.x, t = p / k, rg = blockIdx.y;
    const int n = lane & 15, g = lane >> 4;
    const int H = nsb * kQ4Weights;

    // token t's staged row: loaded into registers first, so that these loads
    // and the top-k's logit loads are in flight together; stored to LDS after
    constexpr int NT = kGpWaves * 64;
    constexpr int kRowLoads = kSmallMaxH / 4 / NT;  // 16-byte pieces per thread
    u32x4 xr[kRowLoads];
    const u32x4 *xsrc = (const u32x4 *)(x_hilo + (size_t)t * 2 * H);
#pragma unroll
    for (int i = 0; i < kRowLoads; ++i) xr[i] = xsrc[min(tid + NT * i, H / 4 - 1)];
    const u32x2 xsr = ((const u32x2 *)(x_xs + (size_t)t * nsb * 16))[min(tid, nsb * 4 - 1)];
    const float svr = x_sinv[(size_t)t * nsb + min(tid, nsb - 1)];
    // expert of pair p = t*k + j: slot j of token t's top-k
    topk_block(logits + (size_t)t * E, E, k, lg, sel_e, sel_v);
    const int e = sel_e[p - t * k];
    const uint8_t *wg = GU + (size_t)((size_t)e * ngroups + rg) * nsb * kGroupSbBytes;

    // wave w takes super-blocks w, w + kGpWaves, ...; two per pass (the
    // second only where it exists: the condition is uniform over the wave)
    auto load_pass = [&](int b0, u32x4 (&q0)[2], u32x4 (&q1)[2], u32x4 (&hd)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i == 0 || b0 + kGpWaves * i < nsb) {
                const uint8_t *blk = wg + (size_t)min(b0 + kGpWaves * i, nsb - 1) * kGroupSbBytes;
                q0[i] = *(const u32x4 *)(blk + lane * 16);
                q1[i] = *(const u32x4 *)(blk + 1024 + lane * 16);
                hd[i] = *(const u32x4 *)(blk + kGroupQsBytes + n * 16);
            }
        }
    };
    // the weight loads go out as soon as the expert is known, ahead of the
    // row's LDS stores and the barrier
    u32x4 q0[2], q1[2], hd[2];
    load_pass(wave, q0, q1, hd);
#pragma unroll
    for (int i = 0; i < kRowLoads; ++i)
        if (tid + NT * i < H / 4) ((u32x4 *)arow)[tid + NT * i] = xr[i];
    if (tid < nsb * 4) ((u32x2 *)axs)[tid] = xsr;
    if (tid < nsb) asv[tid] = svr;
    __syncthreads();
    // hand the pair's expert and renormalised weight to the down/combine
    // launch (one workgroup per pair), so that it need not rank the logits
    // again before its weight loads
    if (rg == 0 && wave == 0) {
        const double ex = (lane < k) ? exp(sel_v[lane] - sel_v[0]) : 0.0;
        const double z = wave_sum(ex);
        if (lane == p - t * k) {
            dsel[p] = e;
            dw[p] = (float)(ex / z);
        }
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const bool a_ok = (n == 0);  // the tile's only row
    for (int b0 = wave; b0 < nsb; b0 += 2 * kGpWaves) {
        if (b0 != wave) load_pass(b0, q0, q1, hd);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int b = b0 + kGpWaves * i;
            if (b < nsb) {
                auto afrag = [&](int s, f16x8 &hi, f16x8 &lo) {
                    const f16 *ap = &arow[((b * 8 + s) * 4 + g) * 16];
                    const f16x8 hv = *(const f16x8 *)ap;
                    const f16x8 lv = *(const f16x8 *)(ap + 8);
                    hi = a_ok ? hv : f16x8{};
                    lo = a_ok ? lv : f16x8{};
                };
                const f16x4 amv = *(const f16x4 *)&axs[b * 16 + 4 * g];
                const float sv[4] = {g == 0 ? asv[b] : 0.f, 0.f, 0.f, 0.f};
                mma_sb_fn(q0[i], q1[i], hd[i], afrag, a_ok ? amv : f16x4{}, sv, g, acc);
            }
        }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    float r = red[0][lane][0];
#pragma unroll
    for (int w = 1; w < kGpWaves; ++w) r += red[w][lane][0];
    const float u = dpp_f<kDppXor8>(r);
    if (lane < 8) h[(size_t)p * I + rg * 8 + lane] = silu_f(r) * u;
}

constexpr int kDcWaves = 8;        // waves per down/combine workgroup
constexpr int kDcMaxPairs = 2;     // unit pairs a wave holds in flight

// Grid (2 * H/16 half row groups + 1, T tokens), kDcWaves waves. Workgroup x
// computes rows 8 (x % 2) .. 8 (x % 2) + 7 of row group x / 2 for token t. The
// token's experts and router weights come from gateup_pair_kernel (dsel, dw).
// The k*nsb (slot j, super-block b) units of the token go in pairs (2P, 2P+1)
// to the waves; a wave stages both units' 256 h values (row t*k + j of
// gateup_pair_kernel's output) in LDS (power-of-two scale, fp16 hi/lo,
// sub-block sums) and runs one MFMA tile for the pair: A rows 0 and 1 are the
// two units' staged h, B columns 0-7 the 8 weight rows of the first unit's
// expert and super-block, columns 8-15 those of the second's, so C[0][0..7]
// and C[1][8..15] are the two units' partials (each element the same sum as a
// tile of its own: an output element depends on its row and column only).
// Two half row groups per row group use every CU at the 30b shape (257
// workgroups of one pair per wave instead of 129 of two units per wave).
// Then out[t][rows] = sum_j w[t][j] * sum_b partial[j][b] in slot order.
__global__ __launch_bounds__(kDcWaves * 64) void down_combine_small_kernel(
    const uint8_t *__restrict__ Wd, int ngroups, int nsb, const double *__restrict__ logits, int E, int T, int k,
    const float *__restrict__ h, int I, const int32_t *__restrict__ dsel, const float *__restrict__ dw,
    const float *__restrict__ resid, float *__restrict__ out, int H, int32_t *__restrict__ idx_out,
    float *__restrict__ w_out, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ entries, int32_t *__restrict__ pos, int q8) {
    const int x = blockIdx.x, t = blockIdx.y;
    const int rg = x >> 1, hf = x & 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int units = k * nsb, npairs = (units + 1) >> 1;
    __shared__ float part[kMaxTopK * 6][8];
    // per wave: the current pair's two staged h blocks [k-step][g][hi 8 |
    // lo 8], their sub-block sums and 1/s (reused pair after pair)
    __shared__ __attribute__((aligned(16))) f16 afrag[kDcWaves][2][8 * 4 * 16];
    __shared__ __attribute__((aligned(16))) f16 axs[kDcWaves][2][16];
    __shared__ float asinv[kDcWaves][2];
    __shared__ __attribute__((aligned(16))) double lg[kRankMaxExperts];
    __shared__ int sel_e[kMaxTopK];
    __shared__ double sel_v[kMaxTopK];

    // The last workgroup of each token column (x == 2 * ngroups) has no down
    // rows: the first one writes the routing outputs of all T tokens, the
    // others leave.
    if (x == 2 * ngroups) {
        if (t == 0)
            routing_outputs_small(logits, T, E, k, lg, sel_e, sel_v, idx_out, w_out, counts, offsets, entries, pos);
        return;
    }
    // unit v of pair slot i, unit half uh (0, 1) of this pass: clamped to a
    // valid unit (a missing second unit of an odd count repeats the first and
    // its result is dropped)
    auto unit_of = [&](int base, int i, int uh) {
        const int P = min(base + i * kDcWaves + wave, npairs - 1);
        return min(2 * P + uh, units - 1);
    };
    // h rows are pair-indexed (t*k + j), so the first pass's h loads do not
    // wait for the routing: issued here, they are in flight with its loads.
    // Lane holds columns 4*lane .. +3 of each unit's super-block.
    float4 hv0[kDcMaxPairs][2];
#pragma unroll
    for (int i = 0; i < kDcMaxPairs; ++i)
#pragma unroll
        for (int uh = 0; uh < 2; ++uh) {
            const int u = unit_of(0, i, uh);
            const int j = u / nsb, b = u % nsb;
            hv0[i][uh] = *(const float4 *)(h + ((size_t)t * k + j) * I + b * kQ4Weights + lane * 4);
        }
    // the token's k experts and renormalised weights, lane j holding slot j,
    // as gateup_pair_kernel ranked them (loaded together with the h rows)
    const int my_e = dsel[(size_t)t * k + min(lane, k - 1)];
    const float my_w = lane < k ? dw[(size_t)t * k + lane] : 0.f;
    // this lane's weight row within the group, and which unit of a pair its
    // column belongs to
    const int wrow = hf * 8 + (n & 7), mine = n >> 3;
    for (int base = 0; base < npairs; base += kDcWaves * kDcMaxPairs) {
        u32x4 q0[kDcMaxPairs], q1[kDcMaxPairs], hdr[kDcMaxPairs];
        float4 hv[kDcMaxPairs][2];
#pragma unroll
        for (int i = 0; i < kDcMaxPairs; ++i) {
            // loads unconditional (clamped): B column n of this lane is weight
            // row wrow of unit `mine` of the pair
            const int u = unit_of(base, i, mine);
            const int j = u / nsb, b = u % nsb;
            const int e = __shfl(my_e, j, kWave);
            const uint8_t *blk = Wd + ((size_t)((size_t)e * ngroups + rg) * nsb + b) * kGroupSbBytes;
            q0[i] = *(const u32x4 *)(blk + (g * 16 + wrow) * 16);
            q1[i] = *(const u32x4 *)(blk + 1024 + (g * 16 + wrow) * 16);
            hdr[i] = *(const u32x4 *)(blk + kGroupQsBytes + wrow * 16);
#pragma unroll
            for (int uh = 0; uh < 2; ++uh) {
                if (base == 0) {
                    hv[i][uh] = hv0[i][uh];
                } else {
                    const int uu = unit_of(base, i, uh);
                    hv[i][uh] = *(const float4 *)(h + ((size_t)t * k + uu / nsb) * I + (uu % nsb) * kQ4Weights +
                                                  lane * 4);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kDcMaxPairs; ++i) {
            const int P = base + i * kDcWaves + wave;
            if (P >= npairs) break;
            // stage both units of the pair
#pragma unroll
            for (int uh = 0; uh < 2; ++uh) {
                float v[4] = {hv[i][uh].x, hv[i][uh].y, hv[i][uh].z, hv[i][uh].w};
                float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
                m = wave_max(m);
                int ex = 0;
                if (m > 0.f) (void)frexpf(m, &ex);
                int se = 10 - ex;
                se = se > 100 ? 100 : (se < -100 ? -100 : se);
                if (!(m > 0.f) || !(m < INFINITY)) se = 0;
                if (q8) {  // Q8_K codes of this 256-value block of h (q8_code), staged with scale 1
                    const float is = m > 0.f ? 127.f / m : 0.f;
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[c] = q8_code(v[c], is);
                    se = 0;
                }
                const float scl = ldexpf(1.f, se);
                const int s = lane >> 3, gg = (lane & 7) >> 1, half = lane & 1;
                float part_sum = 0.f;
                f16 *fr = &afrag[wave][uh][(s * 4 + gg) * 16];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float y = v[c] * scl;
                    const f16 hi = (f16)y;
                    const int el = perm8(4 * half + c);
                    fr[el] = hi;
                    fr[8 + el] = (f16)(y - (float)hi);
                    part_sum += y;
                }
                // the 8 lanes of the k-step: lane ^ 1, lane ^ 2, then the other
                // quad (same sums, in the same order, as shuffles by xor)
                part_sum += dpp_f<kDppXor1>(part_sum);
                part_sum += dpp_f<kDppXor2>(part_sum);
                part_sum += dpp_f<kDppHalfMirror>(part_sum);
                if ((lane & 7) == 0) {
                    const f16 hs = (f16)part_sum;
                    axs[wave][uh][s] = hs;
                    axs[wave][uh][8 + s] = (f16)(part_sum - (float)hs);
                }
                if (lane == 0) asinv[wave][uh] = q8 ? m / 127.f : ldexpf(1.f, -se);
            }
            lds_wave_sync();

            // A rows 0 and 1: the pair's two units; other rows zero
            const bool a_ok = n < 2;
            auto afr = [&](int ss, f16x8 &hi, f16x8 &lo) {
                const f16 *ap = &afrag[wave][n & 1][(ss * 4 + g) * 16];
                const f16x8 hv8 = *(const f16x8 *)ap;
                const f16x8 lv8 = *(const f16x8 *)(ap + 8);
                hi = a_ok ? hv8 : f16x8{};
                lo = a_ok ? lv8 : f16x8{};
            };
            const f16x4 amv = *(const f16x4 *)&axs[wave][n & 1][4 * g];
            const float sv[4] = {g == 0 ? asinv[wave][0] : 0.f, g == 0 ? asinv[wave][1] : 0.f, 0.f, 0.f};
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_sb_fn(q0[i], q1[i], hdr[i], afr, a_ok ? amv : f16x4{}, sv, g, acc);
            // C[0][0..7] (unit 2P) and C[1][8..15] (unit 2P + 1, if it exists)
            if (g == 0) {
                const int u = 2 * P + mine;
                if (u < units) part[u][n & 7] = mine ? acc[1] : acc[0];
            }
            lds_wave_sync();
        }
    }
    __syncthreads();
    if (wave == 0) {
        // o = sum over slots j in slot order of w_j * y_j, y_j = slot j's sum
        // over its super-blocks in super-block order (row lane % 8)
        const int r8 = lane & 7;
        float o = 0.f;
        if (k <= 8 && nsb <= 8) {
            // every read issued together: lane group j = lane / 8 sums slot j
            // (entries past k or nsb read a valid entry and are replaced by
            // +0, which leaves each sum's bits unchanged)
            const int j = lane >> 3;
            float pv[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) pv[b] = part[min(j, k - 1) * nsb + min(b, nsb - 1)][r8];
            float y = 0.f;
#pragma unroll
            for (int b = 0; b < 8; ++b) y += (j < k && b < nsb) ? pv[b] : 0.f;
            float wv[8], yv[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                wv[jj] = __shfl(my_w, jj, kWave);  // 0 past k (my_w of lanes >= k)
                yv[jj] = __shfl(y, jj * 8 + r8, kWave);
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) o += wv[jj] * (jj < k ? yv[jj] : 0.f);
        } else {
            for (int jj = 0; jj < k; ++jj) {
                float y = 0.f;
                for (int b = 0; b < nsb; ++b) y += part[jj * nsb + b][r8];
                o += __shfl(my_w, jj, kWave) * y;
            }
        }
        if (lane < 8) {
            const size_t oi = (size_t)t * H + rg * kRowGroup + hf * 8 + lane;
            out[oi] = resid ? resid[oi] + o : o;  // resid: the block's residual add
        }
    }
}

}  // namespace moe
