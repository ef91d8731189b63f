// Q4_K-on-MFMA building blocks shared by the expert kernels (gemm.hpp,
// decode.hpp), and the combine kernel.
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

// Both k-steps held by the same 8 bytes dA, dB: the low nibbles (k-step with
// scale sc_lo) and the high nibbles (scale sc_hi), as exact fp16 sc * q in the
// element order of q_times_scale. A low nibble or-ed into fp16 1024.0 (0x6400)
// reads as 1024 + q; a high nibble left in place (bits 4-7) and or-ed into fp16
// 64.0 (0x5400) reads as 64 + q, since one mantissa unit of 64.0 is 1/16. One
// fma per pair then removes the offset and applies the scale, exactly.
// Masks and magic halves for q_times_scale_pair, held in VGPRs: with two
// literal operands (v_and_or_b32 takes at most one, and no two SGPRs) the
// compiler would split each and-or into two instructions.
struct NibbleConsts {
    uint32_t lo_mask, hi_mask, lo_magic, hi_magic;
};
__device__ __forceinline__ NibbleConsts nibble_consts() {
    NibbleConsts c;
    uint32_t a = 0x000F000Fu, b = 0x00F000F0u, m = 0x64006400u, h = 0x54005400u;
    asm volatile("" : "+v"(a), "+v"(b), "+v"(m), "+v"(h));
    c.lo_mask = a;
    c.hi_mask = b;
    c.lo_magic = m;
    c.hi_magic = h;
    return c;
}

__device__ __forceinline__ void q_times_scale_pair(uint32_t dA, uint32_t dB, f16 sc_lo, f16 sc_hi, f16x8 &blo,
                                                   f16x8 &bhi, const NibbleConsts &k) {
    const uint32_t a8 = dA >> 8, b8 = dB >> 8;
    const f16x2 s0 = {sc_lo, sc_lo}, n0 = s0 * (f16)(-1024.f);
    const f16x2 s1 = {sc_hi, sc_hi}, n1 = s1 * (f16)(-64.f);
    const f16x2 l0 = __builtin_elementwise_fma(u32_as_f16x2((dA & k.lo_mask) | k.lo_magic), s0, n0);  // bytes 0, 2
    const f16x2 l1 = __builtin_elementwise_fma(u32_as_f16x2((a8 & k.lo_mask) | k.lo_magic), s0, n0);  // bytes 1, 3
    const f16x2 l2 = __builtin_elementwise_fma(u32_as_f16x2((dB & k.lo_mask) | k.lo_magic), s0, n0);  // bytes 4, 6
    const f16x2 l3 = __builtin_elementwise_fma(u32_as_f16x2((b8 & k.lo_mask) | k.lo_magic), s0, n0);  // bytes 5, 7
    const f16x2 h0 = __builtin_elementwise_fma(u32_as_f16x2((dA & k.hi_mask) | k.hi_magic), s1, n1);
    const f16x2 h1 = __builtin_elementwise_fma(u32_as_f16x2((a8 & k.hi_mask) | k.hi_magic), s1, n1);
    const f16x2 h2 = __builtin_elementwise_fma(u32_as_f16x2((dB & k.hi_mask) | k.hi_magic), s1, n1);
    const f16x2 h3 = __builtin_elementwise_fma(u32_as_f16x2((b8 & k.hi_mask) | k.hi_magic), s1, n1);
    blo[0] = l0[0]; blo[1] = l0[1]; blo[2] = l1[0]; blo[3] = l1[1];
    blo[4] = l2[0]; blo[5] = l2[1]; blo[6] = l3[0]; blo[7] = l3[1];
    bhi[0] = h0[0]; bhi[1] = h0[1]; bhi[2] = h1[0]; bhi[3] = h1[1];
    bhi[4] = h2[0]; bhi[5] = h2[1]; bhi[6] = h3[0]; bhi[7] = h3[1];
}

// Scales of sub-blocks 2i and 2i + 1 (bytes 2(i%2), 2(i%2) + 1 of the word w
// holding four 6-bit scales) as the packed pair sp, and the offsets the two
// nibble halves remove, np = {-1024 sc_2i, -64 sc_2i+1} (see
// q_times_scale_pair): a byte under exponent byte 0x64 is the half
// 1024 + byte, so one permute, one packed subtract and one packed multiply
// give both, instead of two conversions and a multiply per scale.
__device__ __forceinline__ void scale_pair(uint32_t w, int i, f16x2 &sp, f16x2 &np) {
    const uint32_t raw = __builtin_amdgcn_perm(0x64646464u, w, (i & 1) ? 0x04030402u : 0x04010400u);
    const f16x2 k1024 = {(f16)1024.f, (f16)1024.f};
    const f16x2 off = {(f16)-1024.f, (f16)-64.f};
    sp = u32_as_f16x2(raw) - k1024;
    np = sp * off;
}

// One k-step of the 8 bytes dA, dB (NIB 0: low nibbles, 1: high), as in
// q_times_scale_pair.
// a8, b8: dA >> 8 and dB >> 8, which the two nibble halves of the same bytes
// can share.
template <int NIB>
__device__ __forceinline__ f16x8 q_times_scale_nib(uint32_t dA, uint32_t dB, uint32_t a8, uint32_t b8, f16 sc,
                                                   const NibbleConsts &k) {
    const uint32_t mask = NIB ? k.hi_mask : k.lo_mask, magic = NIB ? k.hi_magic : k.lo_magic;
    const f16x2 s2 = {sc, sc}, n2 = s2 * (f16)(NIB ? -64.f : -1024.f);
    const f16x2 r0 = __builtin_elementwise_fma(u32_as_f16x2((dA & mask) | magic), s2, n2);  // bytes 0, 2
    const f16x2 r1 = __builtin_elementwise_fma(u32_as_f16x2((a8 & mask) | magic), s2, n2);  // bytes 1, 3
    const f16x2 r2 = __builtin_elementwise_fma(u32_as_f16x2((dB & mask) | magic), s2, n2);  // bytes 4, 6
    const f16x2 r3 = __builtin_elementwise_fma(u32_as_f16x2((b8 & mask) | magic), s2, n2);  // bytes 5, 7
    f16x8 out;
    out[0] = r0[0]; out[1] = r0[1]; out[2] = r1[0]; out[3] = r1[1];
    out[4] = r2[0]; out[5] = r2[1]; out[6] = r3[0]; out[7] = r3[1];
    return out;
}

// q_times_scale_nib with the scale and offset already in fp16 (sc2 = {sc, sc},
// n2 = {-1024 sc, -1024 sc} for NIB 0, {-64 sc, -64 sc} for NIB 1).
template <int NIB>
__device__ __forceinline__ f16x8 q_times_scale_nib_sn(uint32_t dA, uint32_t dB, uint32_t a8, uint32_t b8, f16x2 sc2,
                                                      f16x2 n2, const NibbleConsts &k) {
    const uint32_t mask = NIB ? k.hi_mask : k.lo_mask, magic = NIB ? k.hi_magic : k.lo_magic;
    const f16x2 r0 = __builtin_elementwise_fma(u32_as_f16x2((dA & mask) | magic), sc2, n2);  // bytes 0, 2
    const f16x2 r1 = __builtin_elementwise_fma(u32_as_f16x2((a8 & mask) | magic), sc2, n2);  // bytes 1, 3
    const f16x2 r2 = __builtin_elementwise_fma(u32_as_f16x2((dB & mask) | magic), sc2, n2);  // bytes 4, 6
    const f16x2 r3 = __builtin_elementwise_fma(u32_as_f16x2((b8 & mask) | magic), sc2, n2);  // bytes 5, 7
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


// out[t][:] = sum_{j=0..k-1} w[t][j] * Y[pos[t*k+j]][:], slot 0 first (fixed
// order, no atomics). Grid (ceil(H/1024), T), 256 threads x 4 columns.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ Y, const int32_t *__restrict__ pos,
                                                      const float *__restrict__ w, int H, int k,
                                                      const float *__restrict__ resid, float *__restrict__ out) {
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
    if (resid) {  // the block's residual add: out = resid + (weighted sum)
        const float4 r = *(const float4 *)(resid + (size_t)t * H + c);
        acc.x = r.x + acc.x;
        acc.y = r.y + acc.y;
        acc.z = r.z + acc.z;
        acc.w = r.w + acc.w;
    }
    *(float4 *)(out + (size_t)t * H + c) = acc;
}

}  // namespace moe
