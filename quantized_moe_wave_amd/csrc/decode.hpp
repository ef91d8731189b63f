// Small-batch (decode) path: T <= kSmallT tokens per call, three launches.
//
//   router_small_kernel       router logits (fp64) and x staging; the last
//                             workgroup to finish (device-scope counter) does
//                             the top-k, renormalisation and bucket layout of
//                             all T tokens
//   gateup_pair_kernel        one (token, slot) pair x one 16-row weight group
//                             per workgroup, the four waves splitting the
//                             reduction dimension
//   down_combine_small_kernel down projection of one token's k experts fused
//                             with the router-weighted sum (slot order)
//
// The hand-off to the last workgroup moves only the fp64 logits, through
// agent-scope atomic stores/loads (no cache maintenance).
//
// Same arithmetic as the general path (router.hpp, stage.hpp, expert.hpp); the
// layer's definition and the readings are cited there. Only the work split
// differs: at decode every stage is latency-bound, so the point is fewer
// launches and more independent loads in flight per wave.
#pragma once
#include "common.hpp"
#include "expert.hpp"
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

// ceil(E/4) workgroups of 256 threads, one expert per wave; every workgroup
// also stages a share of the T x super-block units of x. COHERENT: logits are
// stored with agent-scope atomic stores (read back by another workgroup of
// the same launch).
template <bool COHERENT>
__device__ __forceinline__ void logits_small_body(const float *__restrict__ x, const float *__restrict__ wr,
                                                  const float *__restrict__ bias, int T, int H, int E,
                                                  double *__restrict__ logits, f16 *__restrict__ x_hilo,
                                                  f16 *__restrict__ x_xs, float *__restrict__ x_sinv) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nsb = H / kQ4Weights;
    const int nw = gridDim.x * 4;

    for (int u = blockIdx.x * 4 + wave; u < T * nsb; u += nw) {
        const int t = u / nsb, b = u % nsb;
        stage_row_sb(x + (size_t)t * H, nsb, b, x_hilo + (size_t)t * 2 * H, x_xs + (size_t)t * nsb * 16,
                     x_sinv + (size_t)t * nsb);
    }

    // Loads are unconditional (chunk and token indices clamped) so that all of
    // a wave's loads are in flight together; out-of-range terms are skipped.
    for (int e = blockIdx.x * 4 + wave; e < E; e += nw) {
        double acc[kSmallT];
#pragma unroll
        for (int t = 0; t < kSmallT; ++t) acc[t] = 0.0;
        const float *wrow = wr + (size_t)e * H;
        for (int c0 = 0; c0 < nsb; c0 += 8) {
            float4 wv[8], xv[kSmallT][8];
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[i] = *(const float4 *)(wrow + min(c0 + i, nsb - 1) * kQ4Weights + lane * 4);
#pragma unroll
            for (int t = 0; t < kSmallT; ++t)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    xv[t][i] = *(const float4 *)(x + (size_t)min(t, T - 1) * H + min(c0 + i, nsb - 1) * kQ4Weights +
                                                 lane * 4);
#pragma unroll
            for (int t = 0; t < kSmallT; ++t) {
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
        for (int t = 0; t < kSmallT; ++t) {
            if (t < T) {
                double s = wave_sum(acc[t]);
                if (lane == 0) {
                    if (bias) s += (double)bias[e];
                    if (COHERENT)
                        __hip_atomic_store(&logits[(size_t)t * E + e], s, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    else
                        logits[(size_t)t * E + e] = s;
                }
            }
        }
    }
}

// Rank-based top-k of one token for a whole workgroup (E <= 256 = one
// candidate per thread): the k winners' experts and logits land in LDS at
// their slot. Same rule as the other selections: larger logit first, equal
// logits to the lower index; NaN counts as -inf.
template <bool COHERENT>
__device__ __forceinline__ void topk_block(const double *lrow, int E, int k, double *lg, int *sel_e,
                                           double *sel_v) {
    __shared__ float lgf[kRankMaxExperts];
    const int tid = threadIdx.x;
    for (int c = tid; c < E; c += 256) {
        // COHERENT: written by other workgroups of this launch (agent-scope load)
        const double v = COHERENT ? __hip_atomic_load(&lrow[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : lrow[c];
        const double vv = (v == v) ? v : -INFINITY;
        lg[c] = vv;
        lgf[c] = (float)vv;  // rounding is monotone: lgf[j] > lgf[c] implies lg[j] > lg[c]
    }
    __syncthreads();
    // E <= 128: two threads per candidate, each counting half of the logits;
    // E <= 256: one thread per candidate. The count runs on the fp32 copies;
    // where fp32 copies are equal (only then can they disagree with fp64) the
    // pair is decided in fp64 with the lower-index rule, so the ranks are
    // exactly the fp64 ranks.
    const int half = (E <= 128) ? 2 : 1;
    const int c = (half == 2) ? (tid >> 1) : tid;
    const int jb = (half == 2) ? (tid & 1) * ((E + 1) / 2) : 0;
    const int je = (half == 2) ? min(E, jb + (E + 1) / 2) : E;
    const bool live = c < E;
    const double v = live ? lg[c] : -INFINITY;
    const float vf = live ? lgf[c] : -INFINITY;
    int rank = 0;
    for (int j0 = jb; j0 < je; j0 += 16) {
        float a[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) a[q] = lgf[min(j0 + q, E - 1)];
        uint32_t tie = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const bool in = live && (j0 + q < je);
            rank += (int)(in & (a[q] > vf));
            tie |= (uint32_t)(in & (a[q] == vf) & (j0 + q != c)) << q;
        }
        if (__ballot(tie != 0)) {  // rare: settle equal fp32 copies in fp64
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if ((tie >> q) & 1) {
                    const double b = lg[j0 + q];
                    rank += (int)(b > v) | ((int)(b == v) & (int)(j0 + q < c));
                }
            }
        }
    }
    if (half == 2) rank += __shfl_xor(rank, 1, kWave);
    if (live && (half == 1 || (tid & 1) == 0) && rank < k) {
        sel_e[rank] = c;
        sel_v[rank] = v;
    }
    __syncthreads();
}

// Routing outputs of all T tokens: idx/w per token, then the stable bucket
// layout of the T*k <= 256 pairs.
template <bool COHERENT>
__device__ __forceinline__ void routing_outputs_small(const double *logits, int T, int E, int k, double *lg, int *sel_e,
                                                   double *sel_v, int32_t *idx_out, float *w_out, int32_t *counts,
                                                   int32_t *offsets, int32_t *entries, int32_t *pos) {
    __shared__ int sidx[kSmallT * kMaxTopK];
    __shared__ int cnt[kRankMaxExperts];
    __shared__ int off_l[kRankMaxExperts];
    __shared__ int red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int t = 0; t < T; ++t) {
        topk_block<COHERENT>(logits + (size_t)t * E, E, k, lg, sel_e, sel_v);
        if (wave == 0) {
            const double ex = (lane < k) ? exp(sel_v[lane] - sel_v[0]) : 0.0;
            const double z = wave_sum(ex);
            if (lane < k) {
                idx_out[(size_t)t * k + lane] = sel_e[lane];
                w_out[(size_t)t * k + lane] = (float)(ex / z);
                sidx[t * k + lane] = sel_e[lane];
            }
        }
        __syncthreads();
    }
    for (int e = tid; e < E; e += 256) cnt[e] = 0;
    __syncthreads();
    const int S = T * k;
    int my_e = -1, rank = 0;
    if (tid < S) {
        my_e = sidx[tid];
        for (int q = 0; q < tid; ++q) rank += (sidx[q] == my_e);
        atomicAdd(&cnt[my_e], 1);
    }
    __syncthreads();
    const int c = tid < E ? cnt[tid] : 0;
    int ctot;
    const int run = block_exclusive_scan(c, red, &ctot);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = run;
        off_l[tid] = run;
    }
    if (tid == 0) offsets[E] = ctot;
    __syncthreads();
    if (tid < S) {
        const int p = off_l[my_e] + rank;
        entries[p] = tid;
        pos[tid] = p;
    }
}

// Router of the small path: logits_small_body's work, then the last
// workgroup to finish (device-scope counter; the logits travel through
// agent-scope atomic stores and loads, so no cache maintenance is needed)
// writes the routing outputs of all T tokens.
__global__ __launch_bounds__(256) void router_small_kernel(
    const float *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias, int T, int H, int E,
    int k, double *__restrict__ logits, f16 *__restrict__ x_hilo, f16 *__restrict__ x_xs, float *__restrict__ x_sinv,
    uint32_t *__restrict__ counter, int32_t *__restrict__ idx_out, float *__restrict__ w_out,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ entries,
    int32_t *__restrict__ pos) {
    logits_small_body<true>(x, wr, bias, T, H, E, logits, x_hilo, x_xs, x_sinv);
    __shared__ int s_last;
    wait_own_stores();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (counter_arrive(counter) == gridDim.x - 1);
    __syncthreads();
    if (!s_last) return;
    __shared__ __attribute__((aligned(16))) double lg[kRankMaxExperts];
    __shared__ int sel_e[kMaxTopK];
    __shared__ double sel_v[kMaxTopK];
    routing_outputs_small<true>(logits, T, E, k, lg, sel_e, sel_v, idx_out, w_out, counts, offsets, entries, pos);
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kSmallMaxH = 4096;  // hidden sizes the small path stages in LDS

// One super-block of one 16x16 tile, added to acc:
//   P = sum over the 8 k-steps of A (hi, then lo) x B, B = sub-block scale x
//       quant (exact fp16) built from this lane's repacked quant words q0, q1;
//   Q = min-term MFMA of am (k-step sums, hi | lo) with the mins;
//   acc[i] += sv[i] * (d * P[i] - dmin * Q[i]) with d, dmin of this lane's
//   weight row (header hdr). afrag(s, hi, lo) supplies A's k-step s.
template <typename AF>
__device__ __forceinline__ void mma_sb_fn(const u32x4 &q0, const u32x4 &q1, const u32x4 &hdr, AF afrag, f16x4 am,
                                          const float sv[4], int g, f32x4 &acc) {
    uint32_t sc[2], mn[2];
    unpack_scales(hdr, sc, mn);
    const float dd = half_bits_to_float(hdr.x & 0xFFFFu);
    const float dmin = half_bits_to_float(hdr.x >> 16);
    f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const u32x4 &q = (s < 4) ? q0 : q1;
        const int cc = (s >> 1) & 1;
        const uint32_t dA = cc ? q.z : q.x;
        const uint32_t dB = cc ? q.w : q.y;
        const f16 scv = (f16)(float)byte_of(sc, s);
        const f16x2 sc2 = {scv, scv};
        const f16x2 neg2 = sc2 * (f16)(-1024.f);
        const f16x8 B = q_times_scale(dA, dB, s & 1, sc2, neg2);
        f16x8 ahi, alo;
        afrag(s, ahi, alo);
        P = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, B, P, 0, 0, 0);
        P = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, B, P, 0, 0, 0);
    }
    f16x4 Bm;
#pragma unroll
    for (int i = 0; i < 4; ++i) Bm[i] = (f16)(float)byte_of(mn, 4 * (g & 1) + i);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 Q = __builtin_amdgcn_mfma_f32_16x16x16f16(am, Bm, zero, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += sv[i] * (dd * P[i] - dmin * Q[i]);
}

// Grid (T*k pairs, I/8 row groups), 256 threads. Pair p = t*k + j: the
// workgroup stages token t's A row in LDS and computes the 8 gate + 8 up rows
// of row group rg of expert idx[p] for that single row (MFMA row 0), the four
// waves splitting the super-blocks. Output h[p][I] = SiLU(gate) * up.
__global__ __launch_bounds__(256) void gateup_pair_kernel(const uint8_t *__restrict__ GU, int ngroups, int nsb,
                                                          const int32_t *__restrict__ idx, int k,
                                                          const f16 *__restrict__ x_hilo, const f16 *__restrict__ x_xs,
                                                          const float *__restrict__ x_sinv, float *__restrict__ h,
                                                          int I) {
    __shared__ __attribute__((aligned(16))) f16 arow[2 * kSmallMaxH];
    __shared__ __attribute__((aligned(16))) f16 axs[kSmallMaxH / kQ4Weights * 16];
    __shared__ float asv[kSmallMaxH / kQ4Weights];
    __shared__ f32x4 red[4][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = blockIdx.x, t = p / k, rg = blockIdx.y;
    const int n = lane & 15, g = lane >> 4;
    const int H = nsb * kQ4Weights;
    const int e = idx[p];  // expert of pair p (one load, in flight with the row copy)

    // token t's staged row
    {
        const u32x4 *src = (const u32x4 *)(x_hilo + (size_t)t * 2 * H);
        u32x4 *dst = (u32x4 *)arow;
        for (int c = tid; c < H / 4; c += 256) dst[c] = src[c];
        for (int c = tid; c < nsb * 4; c += 256)
            ((u32x2 *)axs)[c] = ((const u32x2 *)(x_xs + (size_t)t * nsb * 16))[c];
        for (int c = tid; c < nsb; c += 256) asv[c] = x_sinv[(size_t)t * nsb + c];
    }
    __syncthreads();

    const uint8_t *wg = GU + (size_t)((size_t)e * ngroups + rg) * nsb * kGroupSbBytes;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const bool a_ok = (n == 0);  // the tile's only row
    // wave w takes super-blocks w, w+4, ...; two per pass, loads issued first
    for (int b0 = wave; b0 < nsb; b0 += 8) {
        u32x4 q0[2], q1[2], hd[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint8_t *blk = wg + (size_t)min(b0 + 4 * i, nsb - 1) * kGroupSbBytes;
            q0[i] = *(const u32x4 *)(blk + lane * 16);
            q1[i] = *(const u32x4 *)(blk + 1024 + lane * 16);
            hd[i] = *(const u32x4 *)(blk + kGroupQsBytes + n * 16);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int b = b0 + 4 * i;
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
    const float r = red[0][lane][0] + red[1][lane][0] + red[2][lane][0] + red[3][lane][0];
    const float u = __shfl_xor(r, 8, kWave);
    if (lane < 8) h[(size_t)p * I + rg * 8 + lane] = silu_f(r) * u;
}

constexpr int kDcWaves = 8;        // waves per down/combine workgroup
constexpr int kDcMaxUnits = 4;     // (slot, super-block) units a wave holds in flight

// Grid (H/16 row groups, T tokens), 512 threads. The k*nsb (slot j,
// super-block b) units of one token are spread over the waves; each unit
// stages its 256 h values (row t*k + j of gateup_pair_kernel's output) in LDS (power-of-two scale, fp16 hi/lo, sub-block
// sums), runs the row-0 MFMA tile against the down weights of expert idx[t][j]
// and leaves a 16-column partial in LDS. Then out[t][cols] =
// sum_j w[t][j] * sum_b partial[j][b] in slot order.
__global__ __launch_bounds__(kDcWaves * 64) void down_combine_small_kernel(
    const uint8_t *__restrict__ Wd, int ngroups, int nsb, const int32_t *__restrict__ idx,
    const float *__restrict__ w, int k, const float *__restrict__ h, int I,
    float *__restrict__ out, int H) {
    const int rg = blockIdx.x, t = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int units = k * nsb;
    __shared__ float part[kMaxTopK * 6][16];
    __shared__ __attribute__((aligned(16))) f16 afrag[kDcWaves][8 * 4 * 16];  // [k-step][g][hi 8 | lo 8]
    __shared__ __attribute__((aligned(16))) f16 axs[kDcWaves][16];
    __shared__ float asinv[kDcWaves];

    // the token's k experts, lane j holding slot j (one load); h rows are
    // pair-indexed (t*k + j)
    const int my_e = idx[(size_t)t * k + min(lane, k - 1)];
    for (int base = 0; base < units; base += kDcWaves * kDcMaxUnits) {
        u32x4 q0[kDcMaxUnits], q1[kDcMaxUnits], hdr[kDcMaxUnits];
        float4 hv[kDcMaxUnits];
#pragma unroll
        for (int i = 0; i < kDcMaxUnits; ++i) {
            const int u = min(base + i * kDcWaves + wave, units - 1);  // clamped: loads stay unconditional
            const int j = u / nsb, b = u % nsb;
            const int e = __shfl(my_e, j, kWave);
            const uint8_t *blk = Wd + ((size_t)((size_t)e * ngroups + rg) * nsb + b) * kGroupSbBytes;
            q0[i] = *(const u32x4 *)(blk + lane * 16);
            q1[i] = *(const u32x4 *)(blk + 1024 + lane * 16);
            hdr[i] = *(const u32x4 *)(blk + kGroupQsBytes + n * 16);
            hv[i] = *(const float4 *)(h + ((size_t)t * k + j) * I + b * kQ4Weights + lane * 4);
        }
#pragma unroll
        for (int i = 0; i < kDcMaxUnits; ++i) {
            const int u = base + i * kDcWaves + wave;
            if (u >= units) break;
            // stage: lane holds columns 4*lane .. +3 of this super-block
            float v[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
            float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
            m = wave_max(m);
            int ex = 0;
            if (m > 0.f) (void)frexpf(m, &ex);
            int se = 10 - ex;
            se = se > 100 ? 100 : (se < -100 ? -100 : se);
            if (!(m > 0.f) || !(m < INFINITY)) se = 0;
            const float scl = ldexpf(1.f, se);
            const int s = lane >> 3, gg = (lane & 7) >> 1, half = lane & 1;
            float part_sum = 0.f;
            f16 *fr = &afrag[wave][(s * 4 + gg) * 16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float y = v[c] * scl;
                const f16 hi = (f16)y;
                const int el = perm8(4 * half + c);
                fr[el] = hi;
                fr[8 + el] = (f16)(y - (float)hi);
                part_sum += y;
            }
            part_sum += __shfl_xor(part_sum, 1, kWave);
            part_sum += __shfl_xor(part_sum, 2, kWave);
            part_sum += __shfl_xor(part_sum, 4, kWave);
            if ((lane & 7) == 0) {
                const f16 hs = (f16)part_sum;
                axs[wave][s] = hs;
                axs[wave][8 + s] = (f16)(part_sum - (float)hs);
            }
            if (lane == 0) asinv[wave] = ldexpf(1.f, -se);
            lds_wave_sync();

            const bool a_ok = (n == 0);
            auto afr = [&](int ss, f16x8 &hi, f16x8 &lo) {
                const f16x8 hv8 = *(const f16x8 *)&afrag[wave][(ss * 4 + g) * 16];
                const f16x8 lv8 = *(const f16x8 *)&afrag[wave][(ss * 4 + g) * 16 + 8];
                hi = a_ok ? hv8 : f16x8{};
                lo = a_ok ? lv8 : f16x8{};
            };
            const f16x4 amv = *(const f16x4 *)&axs[wave][4 * g];
            const float sv[4] = {g == 0 ? asinv[wave] : 0.f, 0.f, 0.f, 0.f};
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_sb_fn(q0[i], q1[i], hdr[i], afr, a_ok ? amv : f16x4{}, sv, g, acc);
            if (lane < 16) part[u][n] = acc[0];  // row 0, column n
            lds_wave_sync();
        }
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        float o = 0.f;
        for (int j = 0; j < k; ++j) {
            float y = 0.f;
            for (int b = 0; b < nsb; ++b) y += part[j * nsb + b][threadIdx.x];
            o += w[(size_t)t * k + j] * y;
        }
        out[(size_t)t * H + rg * kRowGroup + threadIdx.x] = o;
    }
}

}  // namespace moe
