// Grouped GEMM over expert buckets: tiles of up to 64 rows (RB = 4) for
// buckets of more than kTileM entries, of up to 16 rows (RB = 1) for smaller.
//
// Same arithmetic as expert.hpp (see there for the passages it follows and
// for the precision scheme): per Q4_K super-block b of the reduction
// dimension, P = sum_k A_hi*B + A_lo*B on v_mfma_f32_16x16x32_f16 with
// B = sub-block scale x quant (exact fp16), Q = min-term MFMA, and
// acc += sinv_row * (d_col * P - dmin_col * Q) in fp32.
//
// Work split: a workgroup owns a (16*RB) x 256 output tile: up to 16*RB rows
// of one expert's bucket (the last tile of a bucket may be partial; its
// missing rows repeat the last row and are not stored) by 16 repacked 16-row
// weight groups. Each of its 4 waves computes all rows against 4 weight
// groups (RB x 4 MFMA tiles). The staged activations cost 4 bytes per element
// against 0.5625 for Q4_K weights, so the tile is wide in the weight
// dimension: every staged row fetched serves 256 weight rows, and the 4 waves
// share it through LDS.
//
// Tile order: workgroup L runs on XCD L % 8 (round-robin dispatch). XCD x
// owns the contiguous range of ceil(n/8) expert tiles starting at x*ceil(n/8)
// and walks it tile by tile, column block by column block (slot = L / 8 ->
// tile slot / ncb of the range, column block slot % ncb). The ncb column
// blocks of a tile run together and share its activation rows through the
// XCD's L2; tiles are in expert order, so the tiles of one expert run
// together too and share its weights.
//
// Data movement, all by direct global->LDS loads (no staging registers):
//   A (staged activations): a ring of kGemmRing LDS buffers, each a quarter
//   super-block (2 k-steps = 256 bytes of each of the 16*RB rows); slot j
//   of row r is stored at slot j ^ (r % 16) so that the 16 lanes reading one
//   k-step group of 16 rows hit 16 distinct 16-byte bank groups.
//   B (repacked quants + headers of the tile's 16 weight groups, 36 KB per
//   super-block): double-buffered per super-block.
//   k-step sums and 1/s of every row: double-buffered per super-block.
// Every wave issues the same loads in the same order, so "chunk c has landed"
// is a fixed s_waitcnt vmcnt(n) per wave (vmcnt(0) in the last super-block),
// followed by a barrier.
#pragma once
#include "common.hpp"
#include "expert.hpp"

namespace moe {

constexpr int kGemmGroups = 16;                             // weight groups per tile (256 columns)
constexpr int kGemmMinRows = kTileM + 1;                    // buckets this large take 64-row tiles
constexpr int kChunkBytes = 256;                            // bytes of one row per A chunk (2 k-steps)
constexpr int kGemmRing = 4;                                // A chunks: one in use, three in flight
static_assert(kGemmRing == 4, "ring slot of chunk 4b + q is q");
constexpr int kBBufBytes = kGemmGroups * kGroupSbBytes;     // 36 KB
constexpr int kBLoads = kBBufBytes / (4 * 1024);            // 16-byte loads per lane per super-block: 9
constexpr int kBXLoads = kBLoads + 2;                       // + k-step sums + 1/s
constexpr int kXsBufBytes = 4 * 1024;                       // 4 waves x 32 rows x 32 B (rows past the tile repeat)
constexpr int kSvBufBytes = 4 * 256;                        // 4 waves x 64 floats (waves 1-3 repeat wave 0)
static_assert(kBBufBytes % (4 * 1024) == 0, "B block must split evenly over 4 waves");

// Tile shape for RB 16-row blocks (RB = 1 or 4).
template <int RB>
struct GemmShape {
    static constexpr int M = 16 * RB;                      // rows per tile
    static constexpr int ABuf = M * kChunkBytes;           // one A chunk
    static constexpr int ALoads = ABuf / (4 * 1024);       // 16-byte loads per lane per chunk
    static constexpr size_t Lds = (size_t)kGemmRing * ABuf + 2 * kBBufBytes + 2 * kXsBufBytes + 2 * kSvBufBytes;
    static_assert(ABuf % (4 * 1024) == 0, "A chunk must split evenly over 4 waves");
    static_assert(Lds <= 160 * 1024, "LDS budget");
};
constexpr int kGemmM = GemmShape<4>::M;

// Upper bound on 64-row tiles for S bucket entries over E experts: each bucket
// of c >= kGemmMinRows entries takes ceil(c / kGemmM) <= c / kGemmM + 1 tiles.
__host__ __device__ inline int max_gemm_tiles(int S, int E) {
    const int big_buckets = S / kGemmMinRows < E ? S / kGemmMinRows : E;
    return S / kGemmM + big_buckets;
}
// Upper bound on 16-row tiles: one per bucket of fewer than kGemmMinRows entries.
__host__ __device__ inline int max_small_tiles(int S, int E) { return S < E ? S : E; }

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

// GATEUP: W = repacked gate/up (ngroups = I/8 groups of 8 gate + 8 up rows,
//   K = H); A rows are the tokens of the bucket entries; out h[slot][I].
// !GATEUP: W = repacked down (ngroups = H/16, K = I); A rows are the bucket
//   slots themselves; out Y[slot][H].
// tiles[t] = (expert, first bucket slot, rows), t < *n_tiles; ncb = ngroups /
// kGemmGroups column blocks; grid = 8 * ncb * ceil(max tiles / 8).
template <bool GATEUP, int RB>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void expert_gemm_kernel(const uint8_t *__restrict__ W, int ngroups, int nsb,
                                                            const int4 *__restrict__ tiles,
                                                            const int32_t *__restrict__ n_tiles,
                                                            const int32_t *__restrict__ entries, int k,
                                                            const f16 *__restrict__ a_hilo,
                                                            const f16 *__restrict__ a_xs,
                                                            const float *__restrict__ a_sinv,
                                                            float *__restrict__ outp, int out_ld) {
    using Sh = GemmShape<RB>;
    constexpr int kABufBytes = Sh::ABuf, kALoads = Sh::ALoads;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *abuf = smem;
    uint8_t *bbuf = abuf + kGemmRing * kABufBytes;
    uint8_t *xsbuf = bbuf + 2 * kBBufBytes;
    float *svbuf = (float *)(xsbuf + 2 * kXsBufBytes);

    const int ncb = ngroups / kGemmGroups;
    const int ntl = *n_tiles;
    const int per_xcd = (ntl + 7) >> 3;  // tiles per XCD (a contiguous range)
    const int slot_id = blockIdx.x >> 3;
    const int tile = (blockIdx.x & 7) * per_xcd + slot_id / ncb;
    const int cblk = slot_id % ncb;
    if (slot_id / ncb >= per_xcd || tile >= ntl) return;
    const u32x4 tr = *(const u32x4 *)&tiles[tile];
    const int e = (int)tr.x, r0 = (int)tr.y, rows = (int)tr.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int K = nsb * kQ4Weights;
    const int rg0 = cblk * kGemmGroups;

    // source row (token for GATEUP, bucket slot otherwise) of tile row r;
    // rows past the end of a partial tile repeat its last row
    auto src_row = [&](int r) {
        const int rr = min(r, rows - 1);
        return GATEUP ? entries[r0 + rr] / k : r0 + rr;
    };

    // ---- A gather offsets (halves): rows 4*kALoads*wave + 4*i + lane/16, slot
    // (lane%16) ^ (row%16) of each chunk (staged rows stay far below 2^32 halves)
    uint32_t arow_o[kALoads];
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
        const int r = 4 * kALoads * wave + 4 * i + (lane >> 4);
        const int sl = (lane & 15) ^ (r & 15);
        arow_o[i] = (uint32_t)src_row(r) * (uint32_t)(2 * K) + (uint32_t)sl * 8u;
    }
    // k-step sums: rows 32*(wave%2) + lane/2, half (lane&1); 1/s: row lane
    const f16 *xs_p = a_xs + (size_t)src_row(32 * (wave & 1) + (lane >> 1)) * nsb * 16 + (lane & 1) * 8;
    const float *sv_p = a_sinv + (size_t)src_row(lane) * nsb;
    // ---- B gather: flat 16-byte slot f = (wave*kBLoads + i)*64 + lane of the
    // tile's 16 x 2304 bytes of one super-block
    const uint8_t *wtile = W + ((size_t)e * ngroups + rg0) * nsb * kGroupSbBytes;
    uint32_t boff[kBLoads];
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
        const int f = (wave * kBLoads + i) * 64 + lane;
        boff[i] = (uint32_t)((f / 144) * nsb * kGroupSbBytes + (f % 144) * 16);
    }

    auto issue_a = [&](int c) {  // chunk c = 4*b + q into ring buffer c % kGemmRing   (kALoads loads)
        const int b = c >> 2, q = c & 3;
        uint8_t *dst = abuf + (c & (kGemmRing - 1)) * kABufBytes + (4 * kALoads * wave) * kChunkBytes;
#pragma unroll
        for (int i = 0; i < kALoads; ++i) load_lds16(a_hilo + arow_o[i] + b * 512 + q * 128, dst + i * 1024);
    };
    auto issue_bx = [&](int b) {  // B, k-step sums and 1/s of super-block b   (kBXLoads loads)
        uint8_t *bd = bbuf + (b & 1) * kBBufBytes + wave * kBLoads * 1024;
#pragma unroll
        for (int i = 0; i < kBLoads; ++i) load_lds16(wtile + boff[i] + (size_t)b * kGroupSbBytes, bd + i * 1024);
        load_lds16(xs_p + b * 16, xsbuf + (b & 1) * kXsBufBytes + wave * 1024);
        load_lds4(sv_p + b, svbuf + (b & 1) * 256 + 64 * wave);
    };

    const NibbleConsts nk = nibble_consts();
    f32x4 acc[RB][4], P[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
            P[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // Per-super-block constants of this lane's 4 weight groups: scales
    // (bytes 0-3 | 4-7), this lane's 4 mins 4(g%2) .. 4(g%2)+3 (register
    // values: an array indexed by g%2 would go to scratch), d and dmin.
    struct SbConsts {
        uint32_t sc_lo[4], sc_hi[4], mnsel[4];
        float dd[4], dmin[4];
    };
    auto read_consts = [&](int b, SbConsts &k) {
        const uint8_t *bb = bbuf + (b & 1) * kBBufBytes + wave * 4 * kGroupSbBytes;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const u32x4 hdr = *(const u32x4 *)(bb + cb * kGroupSbBytes + kGroupQsBytes + n * 16);
            k.sc_lo[cb] = hdr.y & 0x3F3F3F3Fu;
            k.sc_hi[cb] = (hdr.w & 0x0F0F0F0Fu) | ((hdr.y >> 2) & 0x30303030u);
            const uint32_t mn_lo = hdr.z & 0x3F3F3F3Fu;
            const uint32_t mn_hi = ((hdr.w >> 4) & 0x0F0F0F0Fu) | ((hdr.z >> 2) & 0x30303030u);
            k.mnsel[cb] = (g & 1) ? mn_hi : mn_lo;
            k.dd[cb] = half_bits_to_float(hdr.x & 0xFFFFu);
            k.dmin[cb] = half_bits_to_float(hdr.x >> 16);
        }
    };
    // Fragments of one half (k-step 2q + s2) of chunk c = 4b + q: the 8 A
    // fragments (hi, lo of 4 row blocks; ring slot c % 4) and the 4 B
    // fragments, built from the lane's 8 quant bytes of each of its 4 weight
    // groups (low nibbles for s2 = 0, high for s2 = 1).
    auto read_a_half = [&](int c, int s2, f16x8 (&Ah)[RB], f16x8 (&Al)[RB]) {
        const uint8_t *ab = abuf + (c & (kGemmRing - 1)) * kABufBytes;
        const int jh = (s2 * 8 + 2 * g) ^ n;
        const int jl = (s2 * 8 + 2 * g + 1) ^ n;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = rb * 16 + n;  // A row of this lane (r % 16 == n)
            Ah[rb] = *(const f16x8 *)(ab + r * kChunkBytes + jh * 16);
            Al[rb] = *(const f16x8 *)(ab + r * kChunkBytes + jl * 16);
        }
    };
    auto read_quants = [&](int c, u32x2 (&w)[4]) {
        const int q = c & 3;
        const uint8_t *bb = bbuf + ((c >> 2) & 1) * kBBufBytes + wave * 4 * kGroupSbBytes;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            w[cb] = *(const u32x2 *)(bb + cb * kGroupSbBytes + (q >> 1) * 1024 + lane * 16 + (q & 1) * 8);
    };
    auto build_b_half = [&](int q, int s2, const SbConsts &k, const u32x2 (&w)[4], f16x8 (&Bf)[4]) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const uint32_t scw = q < 2 ? k.sc_lo[cb] : k.sc_hi[cb];
            const f16 sc = (f16)(float)((scw >> (16 * (q & 1) + 8 * s2)) & 0xFFu);
            Bf[cb] = s2 ? q_times_scale_nib<1>(w[cb].x, w[cb].y, sc, nk) : q_times_scale_nib<0>(w[cb].x, w[cb].y, sc, nk);
        }
    };
    auto mfma_half = [&](const f16x8 (&Ah)[RB], const f16x8 (&Al)[RB], const f16x8 (&Bf)[4]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                P[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah[rb], Bf[cb], P[rb][cb], 0, 0, 0);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                P[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al[rb], Bf[cb], P[rb][cb], 0, 0, 0);
    };
    // scheduling pattern of a half (8*RB MFMAs): its LDS reads early, two per
    // MFMA, then the unpack VALU spread over the rest (masks: 0x100 LDS read,
    // 0x008 MFMA, 0x002 VALU)
    auto interleave = [&]() {
        constexpr int kDsGroups = RB == 4 ? 6 : 3;
        constexpr int kValuPer = RB == 4 ? 2 : 8;
#pragma unroll
        for (int i = 0; i < kDsGroups; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 8 * RB - kDsGroups; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);
        }
    };
    // the fragments filled in a half must exist at its end (the compiler
    // would otherwise sink their computation past the next barrier)
    auto pin = [&](f16x8 (&Ah)[RB], f16x8 (&Al)[RB], f16x8 (&Bf)[4]) {
#pragma unroll
        for (int j = 0; j < RB; ++j) asm volatile("" : "+v"(Ah[j]), "+v"(Al[j]));
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(Bf[j]));
    };

    // Pipeline (per wave, chunk c = 4b + q, two halves per chunk):
    //   half 0: MFMAs of (c, k-step 2q) from set 0 | fill set 1 with (c, 2q+1)
    //   wait until chunk c+1 has landed; barrier; issue BX(b+1) (q == 0;
    //     before A(4b+4), so that waiting for A(4b+4) covers it) and A(c+4)
    //     into the ring slot of chunk c, whose last reads were in half 0
    //   half 1: MFMAs of (c, 2q+1) from set 1 | fill set 0 with (c+1, 2q+2)
    // Prologue issue order: BX(0), A(0), A(1), A(2), A(3).
    const int nchunks = 4 * nsb;
    issue_bx(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < kGemmRing; ++c) {
        if (c < nchunks) issue_a(c);
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm<3 * kALoads>();  // BX(0) and A(0) landed: at most A(1..3) outstanding
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    SbConsts kc;
    f16x8 Ah0[RB], Al0[RB], B0[4], Ah1[RB], Al1[RB], B1[4];
    u32x2 wq[4];
    read_consts(0, kc);
    read_quants(0, wq);
    read_a_half(0, 0, Ah0, Al0);
    build_b_half(0, 0, kc, wq, B0);
    __builtin_amdgcn_sched_barrier(0);

    for (int b = 0; b < nsb; ++b) {
        SbConsts kn;  // constants of super-block b+1 (read at q == 3)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 4 * b + q;

            // half 0
            read_a_half(c, 1, Ah1, Al1);
            build_b_half(q, 1, kc, wq, B1);
            mfma_half(Ah0, Al0, B0);
            interleave();
            pin(Ah1, Al1, B1);
            __builtin_amdgcn_sched_barrier(0);

            // At most N loads of this wave issued after A(c+1) are in flight:
            // A(c+2), A(c+3), and, for q == 1, 2, BX(b+1). Near the end (some
            // of those never issued) wait for everything.
            if (c + 3 >= nchunks)
                wait_vm<0>();
            else if (q == 1 || q == 2)
                wait_vm<2 * kALoads + kBXLoads>();
            else
                wait_vm<2 * kALoads>();
            __builtin_amdgcn_s_waitcnt(0xC07F);  // own LDS reads done before their buffers are refilled
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (q == 0 && b + 1 < nsb) issue_bx(b + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (c + kGemmRing < nchunks) issue_a(c + kGemmRing);
            __builtin_amdgcn_sched_barrier(0);

            // half 1 (after the last chunk the fill reads stale but in-bounds
            // LDS and its results go unused; no branch keeps it in one block
            // with the MFMAs)
            {
                u32x2 wn[4];
                if (q == 3) read_consts(b + 1, kn);
                read_quants(c + 1, wn);
                read_a_half(c + 1, 0, Ah0, Al0);
                build_b_half((q + 1) & 3, 0, q == 3 ? kn : kc, wn, B0);
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) wq[cb] = wn[cb];
            }
            mfma_half(Ah1, Al1, B1);
            interleave();
            pin(Ah0, Al0, B0);
            __builtin_amdgcn_sched_barrier(0);
        }

        // super-block b complete: min term and epilogue (its k-step sums and
        // 1/s sit in buffer b % 2, which BX(b+2) refills only after the next
        // barrier)
        const uint8_t *xsb = xsbuf + (b & 1) * kXsBufBytes;
        const float *svb = svbuf + (b & 1) * 256;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = rb * 16 + n;
            const f16x4 Am = *(const f16x4 *)(xsb + r * 32 + g * 8);
            const f32x4 sv = *(const f32x4 *)(svb + rb * 16 + 4 * g);  // rows rb*16 + 4g + 0..3
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const uint32_t mw = kc.mnsel[cb];
                f16x4 Bm;
#pragma unroll
                for (int i = 0; i < 4; ++i) Bm[i] = (f16)(float)((mw >> (8 * i)) & 0xFFu);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 Q = __builtin_amdgcn_mfma_f32_16x16x16f16(Am, Bm, zero, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[rb][cb][i] += sv[i] * (kc.dd[cb] * P[rb][cb][i] - kc.dmin[cb] * Q[i]);
                P[rb][cb] = zero;
            }
        }
        kc = kn;
    }

    // results: tile rows rb*16 + 4g + i (stored if < rows), columns of weight
    // group rg0 + 4*wave + cb
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int rg = rg0 + 4 * wave + cb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr_row = rb * 16 + 4 * g + i;
                const size_t row = (size_t)r0 + tr_row;
                if (GATEUP) {
                    const float u = __shfl_xor(acc[rb][cb][i], 8, kWave);
                    if (n < 8 && tr_row < rows) outp[row * out_ld + rg * 8 + n] = silu_f(acc[rb][cb][i]) * u;
                } else {
                    if (tr_row < rows) outp[row * out_ld + rg * kRowGroup + n] = acc[rb][cb][i];
                }
            }
        }
    }
}

}  // namespace moe
