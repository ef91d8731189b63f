// Expert matmuls with fused Q4_K dequantisation on gfx950 MFMA.
//
// The pages' expert step (forward_qwen3_moe.rs module doc and step 2h): each
// chosen expert dequantises its Q4_K gate/up/down bytes inside its matvecs,
// applies SiLU(gate) * up, and projects back with down.
//
// Per Q4_K super-block (256 columns of the reduction dimension) a weight is
//     w = d * sc_j * q - dmin * m_j        (j = 32-column sub-block)
// so a row . activation product over the super-block is
//     d * sum_c (sc_j q_c) x_c  -  dmin * sum_j m_j (sum_{c in j} x_c).
// The first sum runs on v_mfma_f32_16x16x32_f16 with B = sc_j * q_c, an exact
// integer <= 945 in fp16, and A = the staged activation split hi + lo (two
// MFMAs into the same fp32 accumulator). The second is one
// v_mfma_f32_16x16x16_f16 per super-block with A = the 8 staged 32-column
// sums (hi | lo) and B = the 8 mins (exact). The epilogue of each super-block
// adds sinv * (d * P - dmin * Q) to the running fp32 result.
//
// Tile: 16 tokens (rows of A, one expert bucket tile) x 16 weight rows (one
// repacked row group) per wave; 4 waves per workgroup take 4 consecutive row
// groups of the same tile. Every wave walks the whole reduction dimension.
//
// MFMA register layouts used (16x16 tiles, 64 lanes, lane l):
//   A: row l%16, k-slot group l/16;  B: column l%16, same k-slot group;
//   D: column l%16, rows 4*(l/16) + 0..3.
// Within a k-step the pairing of A and B k-slots is all that matters, and both
// sides use the same slot -> column map (kPerm, common.hpp).
#pragma once
#include "common.hpp"

namespace moe {

__device__ __forceinline__ float silu_f(float z) { return z / (1.f + expf(-z)); }

// B fragment of one k-step: 8 quants (nibble `nib` of the 8 bytes in dA, dB)
// times the sub-block scale, as exact fp16 integers.
__device__ __forceinline__ f16x8 q_times_scale(uint32_t dA, uint32_t dB, int nib, f16x2 sc2, f16x2 neg2) {
    const uint32_t magic = 0x64006400u;  // fp16 1024.0 in both halves
    const int sh = nib * 4;
    const uint32_t p0 = ((dA >> sh) & 0x000F000Fu) | magic;        // bytes 0, 2
    const uint32_t p1 = ((dA >> (sh + 8)) & 0x000F000Fu) | magic;  // bytes 1, 3
    const uint32_t p2 = ((dB >> sh) & 0x000F000Fu) | magic;        // bytes 4, 6
    const uint32_t p3 = ((dB >> (sh + 8)) & 0x000F000Fu) | magic;  // bytes 5, 7
    // (1024 + q) * sc - 1024 * sc = q * sc, exact in one fused rounding
    const f16x2 r0 = __builtin_elementwise_fma(u32_as_f16x2(p0), sc2, neg2);
    const f16x2 r1 = __builtin_elementwise_fma(u32_as_f16x2(p1), sc2, neg2);
    const f16x2 r2 = __builtin_elementwise_fma(u32_as_f16x2(p2), sc2, neg2);
    const f16x2 r3 = __builtin_elementwise_fma(u32_as_f16x2(p3), sc2, neg2);
    f16x8 out;
    out[0] = r0[0]; out[1] = r0[1]; out[2] = r1[0]; out[3] = r1[1];
    out[4] = r2[0]; out[5] = r2[1]; out[6] = r3[0]; out[7] = r3[1];
    return out;
}

// The 8 six-bit scales (sc) and mins (mn) of a header, one byte each.
__device__ __forceinline__ void unpack_scales(u32x4 hdr, uint32_t sc[2], uint32_t mn[2]) {
    const uint32_t s0 = hdr.y, s1 = hdr.z, s2 = hdr.w;  // scale bytes 0-3, 4-7, 8-11
    sc[0] = s0 & 0x3F3F3F3Fu;
    mn[0] = s1 & 0x3F3F3F3Fu;
    sc[1] = (s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u);
    mn[1] = ((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u);
}

__device__ __forceinline__ uint32_t byte_of(const uint32_t w[2], int j) { return (w[j >> 2] >> (8 * (j & 3))) & 0xFFu; }

// GATEUP: W = repacked gate/up matrix (I/8 row groups, K = H); A rows are the
//   tokens of the tile's bucket entries; output h[slot][I] = SiLU(g) * u.
// !GATEUP: W = repacked down matrix (H/16 row groups, K = I); A rows are the
//   tile's slots; output Y[slot][H].
template <bool GATEUP>
__global__ __launch_bounds__(256) void expert_m16_kernel(const uint8_t *__restrict__ W, int ngroups, int nsb,
                                                         const int4 *__restrict__ tiles,
                                                         const int32_t *__restrict__ n_tiles,
                                                         const int32_t *__restrict__ entries, int k,
                                                         const f16 *__restrict__ a_hilo,
                                                         const f16 *__restrict__ a_xs,
                                                         const float *__restrict__ a_sinv,
                                                         float *__restrict__ outp, int out_ld) {
    const int tile = blockIdx.x;
    if (tile >= *n_tiles) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = blockIdx.y * 4 + wave;
    if (rg >= ngroups) return;
    const int4 ti = tiles[tile];
    const int e = ti.x, r0 = ti.y, rows = ti.z;
    const int n = lane & 15, g = lane >> 4;
    const int K = nsb * kQ4Weights;

    // A row of this lane, and the 4 output rows it accumulates.
    const bool a_ok = n < rows;
    const int a_row = a_ok ? (GATEUP ? entries[r0 + n] / k : r0 + n) : 0;
    int o_row[4];
    bool o_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        o_ok[i] = m < rows;
        o_row[i] = o_ok[i] ? (GATEUP ? entries[r0 + m] / k : r0 + m) : 0;
    }

    const uint8_t *wg = W + (size_t)((size_t)e * ngroups + rg) * nsb * kGroupSbBytes;
    const f16 *arow = a_hilo + (size_t)a_row * (2 * K) + g * 16;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < nsb; ++b) {
        const uint8_t *blk = wg + (size_t)b * kGroupSbBytes;
        const u32x4 q0 = *(const u32x4 *)(blk + lane * 16);
        const u32x4 q1 = *(const u32x4 *)(blk + 1024 + lane * 16);
        const u32x4 hdr = *(const u32x4 *)(blk + kGroupQsBytes + n * 16);
        uint32_t sc[2], mn[2];
        unpack_scales(hdr, sc, mn);
        const float d = half_bits_to_float(hdr.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hdr.x >> 16);

        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 &q = (s < 4) ? q0 : q1;
            const int cc = (s >> 1) & 1;   // chunk within the half
            const int nib = s & 1;         // low / high nibble
            const uint32_t dA = cc ? q.z : q.x;
            const uint32_t dB = cc ? q.w : q.y;
            const f16 scv = (f16)(float)byte_of(sc, s);
            const f16x2 sc2 = {scv, scv};
            const f16x2 neg2 = sc2 * (f16)(-1024.f);
            const f16x8 B = q_times_scale(dA, dB, nib, sc2, neg2);
            f16x8 Ahi = {}, Alo = {};
            if (a_ok) {
                const f16 *ap = arow + (size_t)(b * 8 + s) * 64;
                Ahi = *(const f16x8 *)ap;
                Alo = *(const f16x8 *)(ap + 8);
            }
            P = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, B, P, 0, 0, 0);
            P = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, B, P, 0, 0, 0);
        }
        // min term: A' = 4 of the 8 sub-block sums (hi for g < 2, lo for g >= 2),
        // B' = the matching 4 mins.
        f16x4 Am = {};
        if (a_ok) Am = *(const f16x4 *)(a_xs + ((size_t)a_row * nsb + b) * 16 + 4 * g);
        f16x4 Bm;
#pragma unroll
        for (int i = 0; i < 4; ++i) Bm[i] = (f16)(float)byte_of(mn, 4 * (g & 1) + i);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 Q = __builtin_amdgcn_mfma_f32_16x16x16f16(Am, Bm, zero, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sv = o_ok[i] ? a_sinv[(size_t)o_row[i] * nsb + b] : 0.f;
            acc[i] += sv * (d * P[i] - dmin * Q[i]);
        }
    }

    if (GATEUP) {
        // lanes n < 8 hold gate row 8rg+n, lanes n+8 the matching up row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float u = __shfl_xor(acc[i], 8, kWave);
            if (n < 8 && o_ok[i]) outp[(size_t)(r0 + 4 * g + i) * out_ld + rg * 8 + n] = silu_f(acc[i]) * u;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (o_ok[i]) outp[(size_t)(r0 + 4 * g + i) * out_ld + rg * kRowGroup + n] = acc[i];
    }
}

// out[t][:] = sum_{j=0..k-1} w[t][j] * Y[pos[t*k+j]][:], slot 0 first (fixed
// order, no atomics). Grid (ceil(H/1024), T), 256 threads x 4 columns.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ Y, const int32_t *__restrict__ pos,
                                                      const float *__restrict__ w, int H, int k,
                                                      float *__restrict__ out) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const float wj = w[(size_t)t * k + j];
        const float4 y = *(const float4 *)(Y + (size_t)pos[(size_t)t * k + j] * H + c);
        acc.x += wj * y.x;
        acc.y += wj * y.y;
        acc.z += wj * y.z;
        acc.w += wj * y.w;
    }
    *(float4 *)(out + (size_t)t * H + c) = acc;
}

}  // namespace moe
