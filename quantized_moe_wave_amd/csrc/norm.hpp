// Pre-FFN RMSNorm of the Qwen3-MoE block, ahead of the layer.
//
// forward_qwen3_moe.rs (prefill step 2f, decode step 2g, "Pre-FFN norm"): the
// block normalises the residual stream with the layer's ffn norm weight and
// the model's eps before the MoE layer; the op is named there (rms_norm), not
// written out, and is read as the standard RMSNorm
//   xn[t][i] = x[t][i] * g[i] / sqrt((1/H) * sum_c x[t][c]^2 + eps).
// The residual add after the layer (the block's "Residual" step) is folded
// into the kernels that write the layer's output (combine_kernel,
// down_combine_small_kernel).
#pragma once
#include "common.hpp"

namespace moe {

// One workgroup (256 threads) per token: the sum of squares of fp32 values in
// double (each square exact), rms in double, and each output element rounded
// to fp32 from x * g / rms computed in double. H % 4 == 0.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ x, const float *__restrict__ g, int H,
                                                       double eps, float *__restrict__ xn) {
    __shared__ double part[4];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float *row = x + (size_t)t * H;
    double ss = 0.0;
    for (int c = tid * 4; c < H; c += 1024) {
        const float4 v = *(const float4 *)(row + c);
        ss += (double)v.x * v.x;
        ss += (double)v.y * v.y;
        ss += (double)v.z * v.z;
        ss += (double)v.w * v.w;
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    const double tot = (part[0] + part[1]) + (part[2] + part[3]);
    const double rms = sqrt(tot / (double)H + eps);
    float *dst = xn + (size_t)t * H;
    for (int c = tid * 4; c < H; c += 1024) {
        const float4 v = *(const float4 *)(row + c);
        const float4 w = *(const float4 *)(g + c);
        float4 o;
        o.x = (float)((double)v.x * w.x / rms);
        o.y = (float)((double)v.y * w.y / rms);
        o.z = (float)((double)v.z * w.z / rms);
        o.w = (float)((double)v.w * w.w / rms);
        *(float4 *)(dst + c) = o;
    }
}

}  // namespace moe
