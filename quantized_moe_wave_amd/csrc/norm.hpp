// Pre-FFN RMSNorm of the Qwen3-MoE block, ahead of the layer.
//
// forward_qwen3_moe.rs (prefill step 2f, decode step 2g, "Pre-FFN norm"): the
// block normalises the residual stream with the layer's ffn norm weight and
// the model's eps before the MoE layer; the op is named there (rms_norm), not
// written out, and is read as the standard RMSNorm
//   xn[t][i] = x[t][i] * g[i] / sqrt((1/H) * sum_c x[t][c]^2 + eps).
// At most four tokens (the decode path) the norm is fused into the router
// launch (router_small_kernel: each wave recomputes its tokens' 1/rms and
// normalises the values it reads); otherwise rmsnorm_kernel writes the
// normalised rows ahead of the layer. The residual add after the layer (the
// block's "Residual" step) is folded into the kernels that write the layer's
// output (combine_kernel, down_combine_small_kernel).
#pragma once
#include "common.hpp"

namespace moe {

// 1 / sqrt(mean of squares + eps) of one row of H floats (H % 256 == 0), by one
// wave: squares summed in double (each exact), lane-strided, then across the
// wave. Every lane returns the value.
__device__ __forceinline__ double row_inv_rms(const float *__restrict__ row, int H, double eps) {
    const int lane = threadIdx.x & 63;
    double ss = 0.0;
    for (int c = lane * 4; c < H; c += 256) {
        const float4 v = *(const float4 *)(row + c);
        ss += (double)v.x * v.x;
        ss += (double)v.y * v.y;
        ss += (double)v.z * v.z;
        ss += (double)v.w * v.w;
    }
    return 1.0 / sqrt(wave_sum(ss) / (double)H + eps);
}

// One workgroup (256 threads) per token: the sum of squares of fp32 values in
// double (each square exact), 1/rms in double, and each output element rounded
// to fp32 from x * g * (1/rms) computed in double (as the decode path's fused
// norm does). H % 4 == 0.
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
    const double r = 1.0 / sqrt(tot / (double)H + eps);
    float *dst = xn + (size_t)t * H;
    for (int c = tid * 4; c < H; c += 1024) {
        const float4 v = *(const float4 *)(row + c);
        const float4 w = *(const float4 *)(g + c);
        float4 o;
        o.x = (float)((double)v.x * w.x * r);
        o.y = (float)((double)v.y * w.y * r);
        o.z = (float)((double)v.z * w.z * r);
        o.w = (float)((double)v.w * w.w * r);
        *(float4 *)(dst + c) = o;
    }
}

}  // namespace moe
