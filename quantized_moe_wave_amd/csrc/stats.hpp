// Per-stage statistics of one token of a forward: the traced forward's
// per-stage summary (forward_qwen3_moe_cuda_traced.rs: per-layer activation
// statistics of the last token, and its MoeRouter and MoeFfnOut stages, used to
// find the first stage where a NaN or Inf enters). The page names the
// statistics type, not its fields; these are: number of values, NaN count,
// +-Inf count, and over the finite values min, max, mean and root mean square
// (0 when none is finite).
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kStatStages = 4;  // router logits, router weights, SwiGLU h, output row
constexpr int kStatFields = 7;

struct StatAcc {
    int nan, inf, fin;
    double mn, mx, sum, sq;
    __device__ void clear() {
        nan = inf = fin = 0;
        mn = mx = sum = sq = 0.0;
    }
    __device__ void add(double x) {
        if (x != x) {
            ++nan;
        } else if (__builtin_isinf(x)) {
            ++inf;
        } else {
            mn = fin ? fmin(mn, x) : x;
            mx = fin ? fmax(mx, x) : x;
            sum += x;
            sq += x * x;
            ++fin;
        }
    }
    __device__ void merge(const StatAcc &o) {
        if (o.fin) {
            mn = fin ? fmin(mn, o.mn) : o.mn;
            mx = fin ? fmax(mx, o.mx) : o.mx;
        }
        nan += o.nan;
        inf += o.inf;
        fin += o.fin;
        sum += o.sum;
        sq += o.sq;
    }
};

// One workgroup of 256 threads: thread i takes values i, i + 256, ...; the
// partial statistics are then merged in a fixed tree order (deterministic).
template <typename Get>
__device__ void block_stats(int n, Get get, double *dst) {
    __shared__ StatAcc part[256];
    StatAcc a;
    a.clear();
    for (int i = threadIdx.x; i < n; i += 256) a.add(get(i));
    part[threadIdx.x] = a;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            StatAcc b = part[threadIdx.x];
            b.merge(part[threadIdx.x + s]);
            part[threadIdx.x] = b;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const StatAcc &r = part[0];
        dst[0] = (double)n;
        dst[1] = (double)r.nan;
        dst[2] = (double)r.inf;
        dst[3] = r.fin ? r.mn : 0.0;
        dst[4] = r.fin ? r.mx : 0.0;
        dst[5] = r.fin ? r.sum / (double)r.fin : 0.0;
        dst[6] = r.fin ? sqrt(r.sq / (double)r.fin) : 0.0;
    }
}

// Grid kStatStages workgroups, one per stage, for token t. h rows of the
// token's slots j: hpos[t*k + j] when hpos is given (rows in bucket order),
// else t*k + j (pair order).
__global__ __launch_bounds__(256) void stage_stats_kernel(const double *__restrict__ logits,
                                                          const float *__restrict__ w, const float *__restrict__ h,
                                                          const int32_t *__restrict__ hpos,
                                                          const float *__restrict__ out, int t, int E, int k, int I,
                                                          int H, double *__restrict__ stats) {
    double *dst = stats + blockIdx.x * kStatFields;
    switch (blockIdx.x) {
    case 0:
        block_stats(E, [&](int i) { return logits[(size_t)t * E + i]; }, dst);
        break;
    case 1:
        block_stats(k, [&](int i) { return (double)w[(size_t)t * k + i]; }, dst);
        break;
    case 2:
        block_stats(k * I, [&](int i) {
            const int j = i / I;
            const size_t row = hpos ? (size_t)hpos[(size_t)t * k + j] : (size_t)t * k + j;
            return (double)h[row * I + (i - j * I)];
        }, dst);
        break;
    default:
        block_stats(H, [&](int i) { return (double)out[(size_t)t * H + i]; }, dst);
        break;
    }
}

}  // namespace moe
