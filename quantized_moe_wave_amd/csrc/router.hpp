// Router: logits = W_r x (+ bias) in double, softmax over all experts, top-k,
// renormalisation of the k weights.
//
// Defined by: forward_qwen3_moe_cuda_traced.rs (doc of
// forward_qwen3_moe_cuda_traced_with_plan: the MoeRouter stage is a token's k
// router weights after a softmax over the experts and a renormalisation over
// the chosen k) and forward_qwen3_moe.rs step 2h (the chosen experts' outputs
// are weighted by those router weights). Readings: the choice is made on the
// logits (the softmax is monotone), larger first, equal logits to the lower
// expert index; w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max) over the
// chosen i (the softmax denominator over all experts cancels).
//
// Grid: (token groups of TT tokens) x (expert groups of 4*EV experts); block
// 256 = 4 waves, wave w owns experts w, w+4, ... of its group. Lanes split the
// hidden dimension; products and sums are in double (fp32 inputs widen
// exactly), so logits match an fp64 reference to ~1e-16 relative and the
// top-k choice is exact except for true near-ties.
// The last workgroup of a token group to finish (device-scope counter) runs
// the softmax/top-k for that group's tokens, one wave per token.
// That is router_kernel, for T <= 4 outside the decode path; more tokens take
// router_logits_kernel (fp64 MFMA tiles) and a top-k launch of their own
// (topk_token_kernel, or topk_kernel for long rows), below.
#pragma once
#include "common.hpp"
#include "norm.hpp"
#include "stage.hpp"

namespace moe {

constexpr int kRouterChunk = 256;  // hidden columns staged per step

constexpr int kRankMaxExperts = 256;  // rank-based selection up to this many experts

// Selection key of logit v of expert c < kRankMaxExperts: the fp64 bit pattern
// mapped to an unsigned order (sign bit set for non-negative values, all bits
// flipped for negative ones; -0 is first made +0), with its lowest 8 mantissa
// bits replaced by 255 - c. Keys are distinct, and key order is logit order,
// equal logits going to the lower index; logits whose gap is below 2^-44 of
// their magnitude (far inside the near-tie band) are also ordered by index.
// NaN must already be mapped to -inf. One 64-bit compare orders two keys.
__device__ __forceinline__ uint64_t rank_key(double v, int c) {
    const uint64_t b = (uint64_t)__double_as_longlong(v + 0.0);
    const uint64_t ord = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
    return (ord & ~0xFFull) | (uint64_t)(255 - c);
}

// One wave: top-k of one token's E <= 64 * PL (<= kRankMaxExperts) logits by
// rank. Each candidate c counts the keys (rank_key) above its own; the k
// candidates with rank < k are the chosen experts and rank is their slot. Same
// result as k rounds of argmax with the lower-index rule, without a serial
// chain of cross-lane steps. lds: this wave's scratch of 64 * PL + kMaxTopK
// doubles + kMaxTopK ints. Split in two: topk_rank_load (lane l's logits l,
// l + 64, ...) and topk_rank_select (the rest), so that a caller can issue
// other loads in between.
template <int PL, bool COHERENT>
__device__ __forceinline__ void topk_rank_load(const double *lrow, int E, double (&v)[PL]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        // COHERENT: the logits were written by other workgroups of this launch
        v[i] = COHERENT ? __hip_atomic_load(&lrow[min(c, E - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : lrow[min(c, E - 1)];
    }
}

template <int PL>
__device__ __forceinline__ void topk_rank_select(const double (&lv)[PL], int E, int k, int32_t *idx_row,
                                                 float *w_row, int *sidx, double *lds);

template <int PL, bool COHERENT = true>
__device__ __forceinline__ void topk_rank_wave(const double *lrow, int E, int k, int32_t *idx_row, float *w_row,
                                               int *sidx, double *lds) {
    double v[PL];
    topk_rank_load<PL, COHERENT>(lrow, E, v);
    topk_rank_select<PL>(v, E, k, idx_row, w_row, sidx, lds);
}

// The selection of topk_rank_wave from the loaded logits.
template <int PL>
__device__ __forceinline__ void topk_rank_select(const double (&lv)[PL], int E, int k, int32_t *idx_row,
                                                 float *w_row, int *sidx, double *lds) {
    const int lane = threadIdx.x & 63;
    uint64_t *keys = (uint64_t *)lds;
    double v[PL];
    uint64_t key[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        const double x = lv[i];
        v[i] = (c < E && x == x) ? x : -INFINITY;  // NaN never wins; entries >= E pad with -inf
        key[i] = rank_key(v[i], c);
        keys[c] = key[i];
    }
    lds_wave_sync();
    int rank[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) rank[i] = 0;
    // 16 keys per step, read as 8 broadcast 16-byte LDS loads issued together
    // (two steps unrolled: a full unroll hoists every read into registers)
#pragma unroll 2
    for (int j0 = 0; j0 < 64 * PL; j0 += 16) {
        uint64_t a[16];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const ulonglong2 p2 = *(const ulonglong2 *)&keys[j0 + 2 * q];
            a[2 * q] = p2.x;
            a[2 * q + 1] = p2.y;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q)
#pragma unroll
            for (int i = 0; i < PL; ++i) rank[i] += (int)(a[q] > key[i]);
    }
    // winners into LDS (value and expert at their slot), global stores last
    double *sel = lds + 64 * PL;  // after the 64*PL keys
    int *sel_i = (int *)(sel + kMaxTopK);
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        if (c < E && rank[i] < k) {
            sel[rank[i]] = v[i];
            sel_i[rank[i]] = c;
        }
    }
    lds_wave_sync();
    const double ex = (lane < k) ? exp(sel[lane] - sel[0]) : 0.0;
    const double z = wave_sum(ex);
    if (lane < k) {
        const int c = sel_i[lane];
        idx_row[lane] = c;
        w_row[lane] = (float)(ex / z);
        if (sidx) sidx[lane] = c;
    }
    lds_wave_sync();
}

// Top-k of one token on one wave; dispatches on the expert count.
__device__ __forceinline__ void topk_any_wave(const double *lrow, int E, int k, int32_t *idx_row, float *w_row,
                                              int *sidx, double *lds);

// One wave: top-k of one token's E logits (device memory written by other
// workgroups of this launch, read with agent-scope loads) and the renormalised
// weights. Lane j < k writes slot j; sidx (optional, LDS) receives the experts.
__device__ __forceinline__ void topk_wave(const double *lrow, int E, int k, int32_t *idx_row, float *w_row,
                                          int *sidx) {
    const int lane = threadIdx.x & 63;
    const int per_lane = (E + 63) / 64;
    double lv[kMaxExperts / 64];
    uint32_t taken = 0;
    // loads of a uniform number of chunks, clamped to a valid expert, so they
    // are all in flight together
    for (int i0 = 0; i0 < kMaxExperts / 64; i0 += 4) {
        if (i0 >= per_lane) break;
        double v4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v4[i] = __hip_atomic_load(&lrow[min(lane + 64 * (i0 + i), E - 1)], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * (i0 + i);
            lv[i0 + i] = (e < E && v4[i] == v4[i]) ? v4[i] : -INFINITY;  // NaN never wins
            if (e >= E) taken |= 1u << (i0 + i);
        }
    }
#pragma unroll
    for (int i = 0; i < kMaxExperts / 64; ++i) {
        if (i >= ((per_lane + 3) & ~3)) {
            lv[i] = -INFINITY;
            taken |= 1u << i;
        }
    }
    // Round j picks the largest untaken logit (lower index on ties); lane j
    // keeps round j's winner. An untaken -inf still beats "nothing", so a
    // valid expert is always chosen.
    double my_v = -INFINITY, top_v = -INFINITY;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
        double bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kMaxExperts / 64; ++i) {
            int e = lane + 64 * i;
            if (!((taken >> i) & 1) && (lv[i] > bv || (lv[i] == bv && e < bi))) {
                bv = lv[i];
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            double ov = __shfl_xor(bv, o, kWave);
            int oi = __shfl_xor(bi, o, kWave);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (j == 0) top_v = bv;
        if (lane == j) {
            my_v = bv;
            my_i = bi;
        }
    }
    double ex = (lane < k) ? exp(my_v - top_v) : 0.0;
    double z = wave_sum(ex);
    if (lane < k) {
        idx_row[lane] = my_i;
        w_row[lane] = (float)(ex / z);
        if (sidx) sidx[lane] = my_i;
    }
}


__device__ __forceinline__ void topk_any_wave(const double *lrow, int E, int k, int32_t *idx_row, float *w_row,
                                              int *sidx, double *lds) {
    if (E <= 64)
        topk_rank_wave<1>(lrow, E, k, idx_row, w_row, sidx, lds);
    else if (E <= 128)
        topk_rank_wave<2>(lrow, E, k, idx_row, w_row, sidx, lds);
    else if (E <= kRankMaxExperts)
        topk_rank_wave<4>(lrow, E, k, idx_row, w_row, sidx, lds);
    else
        topk_wave(lrow, E, k, idx_row, w_row, sidx);
}

template <int TT, int EV>
__global__ __launch_bounds__(256) void router_kernel(const float *__restrict__ x, const float *__restrict__ wr,
                                                     const float *__restrict__ bias, int T, int H, int E, int k,
                                                     double *__restrict__ logits, int32_t *__restrict__ idx_out,
                                                     float *__restrict__ w_out, uint32_t *__restrict__ counters) {
    __shared__ float xs[TT][kRouterChunk];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * TT;
    const int nt = min(TT, T - t0);
    const int e0 = blockIdx.y * 4 * EV;

    double acc[EV][TT];
#pragma unroll
    for (int v = 0; v < EV; ++v)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[v][t] = 0.0;

    for (int h0 = 0; h0 < H; h0 += kRouterChunk) {
        __syncthreads();
        for (int i = tid; i < TT * kRouterChunk; i += 256) {
            int t = i / kRouterChunk, c = i % kRouterChunk;
            xs[t][c] = (t < nt) ? x[(size_t)(t0 + t) * H + h0 + c] : 0.f;
        }
        __syncthreads();
        float4 xv[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) xv[t] = *(const float4 *)&xs[t][lane * 4];
#pragma unroll
        for (int v = 0; v < EV; ++v) {
            const int e = e0 + wave + 4 * v;
            if (e < E) {
                float4 wv = *(const float4 *)&wr[(size_t)e * H + h0 + lane * 4];
                double w0 = wv.x, w1 = wv.y, w2 = wv.z, w3 = wv.w;
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    double a = acc[v][t];
                    a = fma(w0, (double)xv[t].x, a);
                    a = fma(w1, (double)xv[t].y, a);
                    a = fma(w2, (double)xv[t].z, a);
                    a = fma(w3, (double)xv[t].w, a);
                    acc[v][t] = a;
                }
            }
        }
    }
#pragma unroll
    for (int v = 0; v < EV; ++v) {
        const int e = e0 + wave + 4 * v;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            double s = wave_sum(acc[v][t]);
            if (lane == 0 && e < E && t < nt) {
                if (bias) s += (double)bias[e];
                __hip_atomic_store(&logits[(size_t)(t0 + t) * E + e], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }

    // Last workgroup of this token group does the selection. Hand-off: every
    // wave waits until its logit stores have completed, the barrier orders
    // them before thread 0's counter update, which is a release at agent scope
    // (and an acquire, for the workgroup that arrives last); that workgroup's
    // threads pass the barrier and an agent-scope acquire fence before they
    // read the logits, so every other workgroup's stores happen before those
    // reads.
    wait_own_stores();
    __syncthreads();
    if (tid == 0) s_last = (counter_arrive_acq_rel(&counters[blockIdx.x]) == gridDim.y - 1);
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    __shared__ __attribute__((aligned(16))) double tk_lds[4][kRankMaxExperts + kMaxTopK + kMaxTopK / 2];
    for (int t = wave; t < nt; t += 4)
        topk_any_wave(logits + (size_t)(t0 + t) * E, E, k, idx_out + (size_t)(t0 + t) * k,
                      w_out + (size_t)(t0 + t) * k, nullptr, tk_lds[wave]);
    if (tid == 0) __hip_atomic_store(&counters[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Many tokens: logits on fp64 MFMA, then top-k in a second launch.
//
// v_mfma_f64_16x16x4_f64 takes fp64 operands and accumulates in fp64; the
// fp32 inputs widen exactly and their products are exact, so the logits are
// an fp64 sum of exact products (as in the plain definition) up to summation
// order.
//
// Workgroup tile: 32 tokens x 32 experts, NWV waves (8 where H allows, so
// that two waves share each SIMD and hide each other's load and MFMA
// latency); wave w sums the hidden columns [w*H/NWV, (w+1)*H/NWV) into 2 x 2
// MFMA tiles (16 tokens x 16 experts each), and the NWV partial tiles are
// added in wave order through LDS (a fixed order: results are reproducible).
// Column pairing: for 16 consecutive columns from k0, lane l (n = l%16,
// g = l/16) loads the 4 floats at k0 + 4g of its token row (A) and of its
// expert row (B); MFMA step i (0..3) uses element i, so lane group g covers
// column k0 + 4g + i in step i on both sides and every column is used once.
// MFMA layouts (64 lanes): A lane l = A[row l%16][k l/16], B lane l =
// B[k l/16][col l%16], D lane l element r = D[row l/16 + 4r][col l%16] (the
// fp64 shape interleaves rows unlike the fp32 16x16 shapes).
constexpr int kRlTok = 32, kRlExp = 32, kRlPf = 4;  // tile, and 16-column groups loaded ahead

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Split of H over blockIdx.z for small T: workgroup z covers columns
// [z*H/ks, (z+1)*H/ks) and writes its partial sums to part[z][T][E] (the
// bias in z = 0); the top-k launch adds the ks partials in z order. ks = 1 writes
// the logits directly. H/ks must be a multiple of 64 * NWV (each wave's share
// a whole number of kRlPf 16-column groups).
constexpr int kRlMaxSplit = 16;
constexpr int kRlPartDoubles = 256 * 1024;  // ks*T*E < 1024 * 256 for the ks the host picks

// NORM (the block's pre-FFN RMSNorm folded in, norm_w = its weight g): the
// kernel sums W_r[e] . (x * g) (each product x*g exact in double) and leaves
// the row's 1/rms factor, and the bias, to the top-k launch, which has the row:
// logit = (1/rms) * sum + bias. Equal to the sum over the rounded normalised
// row up to the rounding of its elements (a few 1e-8 of a logit).
template <int NWV, bool NORM>
__global__ __launch_bounds__(64 * NWV) void router_logits_kernel(const float *__restrict__ x,
                                                                 const float *__restrict__ wr,
                                                                 const float *__restrict__ bias, int T, int H, int E,
                                                                 double *__restrict__ logits, int ks,
                                                                 double *__restrict__ part_out,
                                                                 const float *__restrict__ norm_w) {
    __shared__ double part[NWV][2][2][4][64];  // [wave][token block][expert block][element][lane]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int t0 = blockIdx.x * kRlTok, e0 = blockIdx.y * kRlExp;
    const int kq = H / (NWV * ks);          // columns per wave (a multiple of 64)
    const int kbeg = blockIdx.z * (H / ks) + wave * kq;
    const int ngrp = kq >> 4;               // 16-column groups per wave

    // rows of this lane (clamped: rows past T or E load a valid row, never stored)
    const float *xr[2], *wrow[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        xr[b] = x + (size_t)min(t0 + 16 * b + n, T - 1) * H + kbeg + 4 * g;
        wrow[b] = wr + (size_t)min(e0 + 16 * b + n, E - 1) * H + kbeg + 4 * g;
    }

    f64x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};

    // register ring of kRlPf groups: group j sits in slot j % kRlPf
    const float *gcol = NORM ? norm_w + kbeg + 4 * g : nullptr;
    float4 ra[kRlPf][2], rb[kRlPf][2], rg[kRlPf];
    auto load_grp = [&](int j, float4 (&a)[2], float4 (&b)[2], float4 &gg) {
        const int jj = min(j, ngrp - 1);  // past the end: reload the last group (unused)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            a[t] = *(const float4 *)(xr[t] + 16 * jj);
            b[t] = *(const float4 *)(wrow[t] + 16 * jj);
        }
        if (NORM) gg = *(const float4 *)(gcol + 16 * jj);
    };
#pragma unroll
    for (int j = 0; j < kRlPf; ++j) load_grp(j, ra[j], rb[j], rg[j]);

    for (int j0 = 0; j0 < ngrp; j0 += kRlPf) {
#pragma unroll
        for (int u = 0; u < kRlPf; ++u) {
            const float4 a0 = ra[u][0], a1 = ra[u][1], b0 = rb[u][0], b1 = rb[u][1], g0 = rg[u];
            load_grp(j0 + u + kRlPf, ra[u], rb[u], rg[u]);
            const float av[2][4] = {{a0.x, a0.y, a0.z, a0.w}, {a1.x, a1.y, a1.z, a1.w}};
            const float bv[2][4] = {{b0.x, b0.y, b0.z, b0.w}, {b1.x, b1.y, b1.z, b1.w}};
            const float gv[4] = {g0.x, g0.y, g0.z, g0.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int eb = 0; eb < 2; ++eb)
                        acc[tb][eb] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                            NORM ? (double)av[tb][i] * (double)gv[i] : (double)av[tb][i], (double)bv[eb][i],
                            acc[tb][eb], 0, 0, 0);
        }
    }

#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int eb = 0; eb < 2; ++eb)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[wave][tb][eb][r][lane] = acc[tb][eb][r];
    __syncthreads();
    // 1024 outputs, 1024 / (64 NWV) per thread: combo c = (tb, eb, r, lane)
#pragma unroll
    for (int q = 0; q < 1024 / (64 * NWV); ++q) {
        const int c = threadIdx.x + 64 * NWV * q;
        const int l = c & 63, r = (c >> 6) & 3, eb = (c >> 8) & 1, tb = c >> 9;
        const int t = t0 + 16 * tb + (l >> 4) + 4 * r, e = e0 + 16 * eb + (l & 15);
        double v = part[0][tb][eb][r][l];
#pragma unroll
        for (int w = 1; w < NWV; ++w) v += part[w][tb][eb][r][l];
        if (t < T && e < E) {
            if (bias && blockIdx.z == 0) v += (double)bias[e];
            if (ks == 1)
                logits[(size_t)t * E + e] = v;
            else
                part_out[((size_t)blockIdx.z * T + t) * E + e] = v;
        }
    }
}

// Top-k and renormalised weights of 4 tokens per workgroup, one wave each,
// from logits written by the previous launch; E <= 64 * PL (E <= kRankMaxExperts;
// larger E takes topk_wide_kernel). ks > 1: the logits are first summed from
// the ks partials of router_logits_kernel (z order) and written back to logits.
// x non-null: the wave also stages its token's activation row (H columns) for
// the grouped GEMM, as stage_kernel would (independent of the routing); the
// row's loads are issued right after the logits' and land while the
// selection runs.
// NORM (router_logits_kernel<.., true> ran before; x then holds the block's
// residual stream, whose row must fit the registers; norm_w is the norm
// weight): the wave computes its
// row's 1/rms r from the row it stages, turns each sum into the logit
// r * sum + bias (written back for the debug copy) and stages the normalised
// row fp32(x * g * r) (products in double, as rmsnorm_kernel).
// q8: the staged row holds Q8_K codes per super-block (stage_row_store).
template <int PL, bool NORM>
__global__ __launch_bounds__(256) void topk_kernel(double *__restrict__ logits, int T, int E, int k,
                                                   int32_t *__restrict__ idx_out, float *__restrict__ w_out, int ks,
                                                   const double *__restrict__ part, const float *__restrict__ x,
                                                   int H, f16 *__restrict__ x_hilo, f16 *__restrict__ x_xs,
                                                   float *__restrict__ x_sinv, const float *__restrict__ norm_w,
                                                   double eps, const float *__restrict__ bias, int q8) {
    __shared__ __attribute__((aligned(16))) double tk_lds[4][64 * PL + kMaxTopK + kMaxTopK / 2];
    __shared__ __attribute__((aligned(16))) double sums[4][64 * PL];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * (blockDim.x >> 6) + wave;  // one token per wave, 1-4 waves per workgroup
    if (t >= T) return;
    const int nh = H / kQ4Weights;
    const bool row_in_regs = x && (nh + 1) / 2 <= kStageRegPairs;
    StagedRow sr;
    // the row's 1/rms first (it scales every logit), from a pass of its own
    // over the row, so that the row is held in registers only from the
    // selection on, as without the norm
    const double r = NORM ? row_inv_rms(x + (size_t)t * H, H, eps) : 1.0;
    const double *lrow = logits + (size_t)t * E;
    if (ks > 1) {
        for (int c = lane; c < E; c += 64) {
            // all partials in flight together (index clamped), added in z order
            double pv[kRlMaxSplit];
#pragma unroll
            for (int z = 0; z < kRlMaxSplit; ++z) pv[z] = part[((size_t)min(z, ks - 1) * T + t) * E + c];
            double v = pv[0];
#pragma unroll
            for (int z = 1; z < kRlMaxSplit; ++z)
                if (z < ks) v += pv[z];
            if (NORM) v = r * v + (bias ? (double)bias[c] : 0.0);
            sums[wave][c] = v;
            logits[(size_t)t * E + c] = v;
        }
        lds_wave_sync();
        lrow = sums[wave];
    } else if (NORM) {
        for (int c = lane; c < E; c += 64) {
            const double v = r * lrow[c] + (bias ? (double)bias[c] : 0.0);
            sums[wave][c] = v;
            logits[(size_t)t * E + c] = v;
        }
        lds_wave_sync();
        lrow = sums[wave];
    }
    double lv[PL];
    topk_rank_load<PL, false>(lrow, E, lv);
    if (row_in_regs) stage_row_load(x + (size_t)t * H, nh, sr);
    topk_rank_select<PL>(lv, E, k, idx_out + (size_t)t * k, w_out + (size_t)t * k, nullptr, tk_lds[wave]);
    if (NORM) {  // the weight row only now, so that it does not stay live across the selection
        asm volatile("" ::: "memory");
        StagedRow gr;
        stage_row_load(norm_w, nh, gr);
        staged_row_normalise(sr, gr, nh, r);
    }
    if (row_in_regs)
        stage_row_store(sr, nh, x_hilo + (size_t)t * (2 * H), x_xs + (size_t)t * nh * 16, x_sinv + (size_t)t * nh,
                        q8 != 0);
    else if (x)
        stage_row_wave(x + (size_t)t * H, nh, x_hilo + (size_t)t * (2 * H), x_xs + (size_t)t * nh * 16,
                       x_sinv + (size_t)t * nh, q8 != 0);
}

// topk_kernel with one token per workgroup of 4 waves, for rows that fit the
// registers ((H / 256 + 1) / 2 <= kStageRegPairs, x non-null): the same
// results, with the token's chain of dependent steps split four ways. Thread
// c sums expert c's ks partials (z order); the four waves rank the
// candidates together (thread (part, c) counts the keys of part's share of
// the experts above c's, the counts added in LDS); wave w holds and stages
// the row's super-block pairs w, w + 4, ... (the row's scale from the four
// waves' maxima). NORM: 1/rms from the sum of squares of the held parts
// (each square exact in double).
template <int PL, bool NORM>
__global__ __launch_bounds__(256) void topk_token_kernel(double *__restrict__ logits, int T, int E, int k,
                                                         int32_t *__restrict__ idx_out, float *__restrict__ w_out,
                                                         int ks, const double *__restrict__ part,
                                                         const float *__restrict__ x, int H, f16 *__restrict__ x_hilo,
                                                         f16 *__restrict__ x_xs, float *__restrict__ x_sinv,
                                                         const float *__restrict__ norm_w, double eps,
                                                         const float *__restrict__ bias, int q8) {
    constexpr int EP = 64 * PL;       // candidates, padded
    constexpr int NPART = 256 / EP;   // rank parts (4, 2 or 1)
    constexpr int SPAN = EP / NPART;  // keys counted per thread
    static_assert(SPAN % 16 == 0, "16 keys per step");
    __shared__ __attribute__((aligned(16))) uint64_t keys[EP];
    __shared__ int rk[NPART][EP];
    __shared__ double sel_v[kMaxTopK];
    __shared__ int sel_e[kMaxTopK];
    __shared__ double red_d[4];
    __shared__ float red_f[4];
    const int t = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (t >= T) return;
    const int nh = H / kQ4Weights;
    const float *xrow = x + (size_t)t * H;
    StagedPart sp;
    stage_pairs_load(xrow, nh, wave, 4, sp);

    // expert tid's logit: partials issued first, the row's 1/rms meanwhile
    const int c = tid;
    double pv[kRlMaxSplit];
    if (ks > 1) {
#pragma unroll
        for (int z = 0; z < kRlMaxSplit; ++z) pv[z] = part[((size_t)min(z, ks - 1) * T + t) * E + min(c, E - 1)];
    } else {
        pv[0] = logits[(size_t)t * E + min(c, E - 1)];
    }
    double r = 1.0;
    if (NORM) {
        const double ss = wave_sum(staged_pairs_sumsq(sp, nh));
        if (lane == 0) red_d[wave] = ss;
        __syncthreads();
        r = 1.0 / sqrt((red_d[0] + red_d[1] + red_d[2] + red_d[3]) / (double)H + eps);
    }
    double v = pv[0];
    if (ks > 1) {
#pragma unroll
        for (int z = 1; z < kRlMaxSplit; ++z)
            if (z < ks) v += pv[z];
    }
    if (NORM) v = r * v + (bias ? (double)bias[min(c, E - 1)] : 0.0);
    if (c < E && (ks > 1 || NORM)) logits[(size_t)t * E + c] = v;
    v = (c < E && v == v) ? v : -INFINITY;  // NaN never wins; entries >= E pad with -inf
    if (c < EP) keys[c] = rank_key(v, c);
    __syncthreads();

    // ranks: thread (prt, cand) counts the keys of [prt * SPAN, (prt + 1) * SPAN)
    // above cand's (prt is uniform per wave, so the key reads broadcast)
    const int prt = tid / EP, cand = tid % EP;
    const uint64_t key = keys[cand];
    int rank = 0;
#pragma unroll 2
    for (int j0 = prt * SPAN; j0 < (prt + 1) * SPAN; j0 += 16) {
        uint64_t a[16];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const ulonglong2 p2 = *(const ulonglong2 *)&keys[j0 + 2 * q];
            a[2 * q] = p2.x;
            a[2 * q + 1] = p2.y;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) rank += (int)(a[q] > key);
    }
    rk[prt][cand] = rank;
    __syncthreads();
    if (c < E) {  // prt == 0 here: cand == c, v is c's
        int rs = 0;
#pragma unroll
        for (int q = 0; q < NPART; ++q) rs += rk[q][c];
        if (rs < k) {
            sel_v[rs] = v;
            sel_e[rs] = c;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const double ex = (lane < k) ? exp(sel_v[lane] - sel_v[0]) : 0.0;
        const double z = wave_sum(ex);
        if (lane < k) {
            idx_out[(size_t)t * k + lane] = sel_e[lane];
            w_out[(size_t)t * k + lane] = (float)(ex / z);
        }
    }

    // the row: normalised (NORM), scaled by the row's power of two, stored
    if (NORM) {
        StagedPart gp;
        stage_pairs_load(norm_w, nh, wave, 4, gp);
        staged_pairs_normalise(sp, gp, nh, r);
    }
    int se = 0;
    if (!q8) {
        const float m = wave_max(staged_pairs_absmax(sp, nh));
        if (lane == 0) red_f[wave] = m;
        __syncthreads();
        se = stage_exponent(fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3])));
    }
    staged_pairs_emit(sp, nh, se, x_hilo + (size_t)t * (2 * H), x_xs + (size_t)t * nh * 16, x_sinv + (size_t)t * nh,
                      q8 != 0);
}

// topk_kernel for E > kRankMaxExperts (k rounds of wave argmax; ks = 1): a
// kernel of its own so that its registers do not weigh on the rank path.
__global__ __launch_bounds__(256) void topk_wide_kernel(const double *__restrict__ logits, int T, int E, int k,
                                                        int32_t *__restrict__ idx_out, float *__restrict__ w_out) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_wave(logits + (size_t)t * E, E, k, idx_out + (size_t)t * k, w_out + (size_t)t * k, nullptr);
}

}  // namespace moe
