// Grouped GEMM over expert buckets: tiles of up to 64 rows (RB = 4) for
// buckets of more than kTileM entries, of up to 16 rows (RB = 1) for smaller.
//
// Arithmetic (expert.hpp cites the passages it follows): over Q4_K
// super-block b a weight is d_b * sc * q - dmin_b * m, so a weight row's
// product with an activation row over the super-block is d_b P_b - dmin_b Q_b:
//   P_b = sum_k A_k (sc q)_k on v_mfma_f32_16x16x32_f16, B = sc q exact in
//         fp16, A = the staged activation split hi + lo (two MFMAs);
//   Q_b = sum_j S_j m_j on v_mfma_f32_16x16x16_f16 (S_j the staged 32-column
//         sums, m_j the 6-bit mins, exact in fp16).
// The staged activations carry one power-of-two scale s per row, so the
// result is (1/s) sum_b (d_b P_b - dmin_b Q_b).
//
// One fp32 accumulator X per output holds that sum divided by the current
// super-block's d: during super-block b its MFMAs add P_b into X and its min
// term adds -(dmin_b / d_b) Q_b (at any point of b, X being in units of d_b
// throughout); between b and b+1, X is multiplied by d_b / d_{b+1} (after the
// last super-block by d_b, then by 1/s). A super-block row with d = 0 adds
// only its min term: its B is zeroed and its d taken as 1 in both ratios.
// Each rescale costs one fp32 rounding, far below the 1e-4 bar over a few
// dozen super-blocks. One accumulator instead of a per-super-block partial
// plus a running sum halves the accumulator registers (64-row tiles; the
// 16-row tiles of exact activations have registers to spare and use the
// partial plus running sum, kTwoAcc below).
//
// Work split: a workgroup of NW waves owns a (16*RB) x (16*NW*CW) output
// tile: up to 16*RB rows of one expert's bucket (the last tile of a bucket
// may be partial; its missing rows repeat the last row and are not stored) by
// NW*CW repacked 16-row weight groups. Each wave computes all rows against CW
// weight groups (RB x CW MFMA tiles). A staged activation costs 4 bytes per
// element against 0.5625 for a Q4_K weight, so the tile is wide in the weight
// dimension: each staged row fetched serves 16*NW*CW weight rows. The per-CU
// global->LDS rate (about 23 bytes per cycle on this part) bounds what the
// MFMAs can be fed: a 64 x 512 tile needs about 16 bytes per cycle of MFMA
// work, a 64 x 256 tile about 25. Big tiles run 8 waves of 64 x 64 (two per
// SIMD): while one wave waits (barrier, loads, LDS, the super-block
// boundary's VALU work) the other keeps the SIMD's matrix unit busy.
//
// Tile order: workgroup L runs on XCD L % 8 (round-robin dispatch). XCD x
// owns the contiguous range of ceil(n/8) expert tiles starting at x*ceil(n/8)
// and walks it tile by tile, column block by column block. The column blocks
// of a tile run together and share its activation rows through the XCD's L2;
// tiles are in expert order, so the tiles of one expert share its weights.
//
// Data movement, all by direct global->LDS loads (no staging registers), as
// raw buffer loads: each lane's fixed byte offset in a VGPR, the per-step
// offset in an SGPR, so no load costs address VALU in the main loop:
//   A (staged activations): a ring of 4 chunk buffers; chunk c = 4b + q is a
//   quarter super-block (2 k-steps = 256 bytes of each row); 16-byte slot j
//   of row r is stored at slot j ^ (r % 16), so that the 16 lanes reading one
//   k-step group of 16 rows hit 16 distinct bank groups.
//   Bq (quants): a ring of 2 half-super-block buffers (1 KB per weight group;
//   each wave loads exactly its own CW groups).
//   HX (headers d, dmin, scales, mins of the tile's groups, and the k-step
//   sums of its rows): double-buffered per super-block.
// Per wave, iteration c runs in two halves (k-steps 2q and 2q + 1): the MFMAs
// of one half run while the fragments of the next are read from LDS and
// unpacked into the other register set. Between the halves the wave waits for
// chunk c+1's loads, passes the barrier and issues the group
//     [HX(b+1) if q == 0] [Bq((c+3)/2) if c is odd] [A(c+4)]
// into buffers whose last readers have all passed that barrier. Every wave
// issues the same loads in the same order and they complete in order, so
// "chunk c+1 has landed" is a fixed vmcnt per q (see the wait below).
#pragma once
#include <type_traits>

#include "common.hpp"
#include "expert.hpp"

namespace moe {

constexpr int kGemmMinRows = kTileM + 1;  // buckets this large take 64-row tiles
constexpr int kChunkBytes = 256;          // bytes of one row per A chunk (2 k-steps)
constexpr int kGemmRing = 4;              // A chunk buffers
static_assert(kGemmRing == 4, "ring slot of chunk 4b + q is q");

// Tile shape: RB 16-row blocks, CW 16-column weight groups per wave, NW waves.
// Q8: the activations are Q8_K-style codes with a scale per row and
// super-block (one MFMA pass, and each wave keeps the tile rows' scales of
// the current and the next super-block).
template <int RB, int CW, int NW, bool Q8 = false>
struct GemmShape {
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static constexpr int M = 16 * RB;                       // rows per tile
    static constexpr int Groups = NW * CW;                  // weight groups per tile
    static constexpr int ABuf = M * kChunkBytes;            // one A chunk
    static constexpr int ALoads = ABuf / (NW * 1024);       // 16-byte loads per lane per chunk
    static constexpr int BqBuf = Groups * 1024;             // quants of one half super-block
    static constexpr int BLoads = CW;                       // each wave loads its own groups
    static constexpr int HdrBuf = Groups * 256;             // headers of one super-block
    // headers move as 16-byte loads where they split evenly over the waves,
    // else as 4-byte loads (a 16 x 128 tile's 2 KB over 4 waves, a 64 x 256
    // tile's 4 KB over 8)
    static constexpr int HdrLoadB = HdrBuf % (NW * 1024) == 0 ? 16 : 4;
    static constexpr int HdrLoads = HdrBuf / (NW * 64 * HdrLoadB);  // header loads per lane
    // k-step sums, 32 B per row: 8 waves, or 4 waves on 16-row tiles, load 4
    // bytes per lane (rows 8*wave + lane/8: 64 or 32 rows, the rows past the
    // tile's repeating its last); 4 waves on 64-row tiles load 16 (rows
    // 32*(wave%2) + lane/2; waves 2, 3 repeat waves 0, 1)
    static constexpr bool XsNarrow = NW == 8 || RB == 1;
    static constexpr int XsBuf = NW == 8 ? 2048 : (RB == 1 ? 1024 : 4096);
    static constexpr int HLoads = HdrLoads + 1;  // headers + the k-step sums
    static constexpr int DxBuf = Q8 ? NW * 256 : 0;          // Q8: 64 rows' scales, one copy per wave
    static constexpr int HxLoads = HLoads + (Q8 ? 1 : 0);    // loads of one HX group
    static constexpr size_t DxOff =
        (size_t)kGemmRing * ABuf + 2 * (size_t)BqBuf + 2 * (size_t)HdrBuf + 2 * (size_t)XsBuf;
    static constexpr size_t SvOff = DxOff + 2 * (size_t)DxBuf;
    static constexpr size_t Lds = SvOff + NW * 64 * sizeof(float);  // + 1/s of the rows, one copy per wave
    // output staging (after the main loop, over the same LDS): M rows of up to
    // 16 * Groups floats, padded by 4 floats against bank conflicts
    static constexpr int OutLd = 16 * Groups + 4;
    static_assert(ALoads >= 1 && ABuf % (NW * 1024) == 0 && HdrLoads >= 1 && HdrBuf % (NW * 64 * HdrLoadB) == 0,
                  "buffers must split evenly over the waves");
    static_assert((size_t)M * OutLd * sizeof(float) <= SvOff, "output staging must fit below the 1/s copies");
    static_assert(Lds <= 160 * 1024, "LDS budget");
};
constexpr int kGemmM = 64;  // rows of a big tile

// Weight groups per big tile over ngroups groups (a multiple of 16: I/8 for
// gate/up, H/16 for down): 32 (64 x 512 tiles) where the groups split into
// blocks of 32, else 16 (64 x 256; both 8 waves).
__host__ __device__ inline int gemm_big_groups(int ngroups) { return ngroups % 32 == 0 ? 32 : 16; }

// Upper bound on 64-row tiles for S bucket entries over E experts: each bucket
// of c >= kGemmMinRows entries takes ceil(c / kGemmM) <= c / kGemmM + 1 tiles.
__host__ __device__ inline int max_gemm_tiles(int S, int E) {
    const int big_buckets = S / kGemmMinRows < E ? S / kGemmMinRows : E;
    return S / kGemmM + big_buckets;
}
// Calls whose buckets average at most kTileM pairs (S <= E * kTileM) cut every
// bucket into 16-row tiles and launch no 64-row GEMM: there the 64-row launches
// would mostly find no tile, and a rare larger bucket costs a few more passes
// over its expert's weights.
__host__ __device__ inline bool all_small_tiles(int S, int E) { return S <= E * kTileM; }
// Upper bound on 16-row tiles: one per bucket of fewer than kGemmMinRows
// entries, or with all_small_tiles ceil(c / kTileM) <= c / kTileM + 1 per bucket.
__host__ __device__ inline int max_small_tiles(int S, int E) {
    const int buckets = S < E ? S : E;
    return all_small_tiles(S, E) ? S / kTileM + buckets : buckets;
}

__device__ __forceinline__ void load_lds16(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)lds_base, 4, 0, 0);
}

// Raw buffer loads into LDS: a buffer resource over base (stride 0, all of
// the first 4 GB valid; dword 3 = the gfx9 raw 32-bit format), a per-lane
// 32-bit byte offset and a uniform one (an SGPR: no per-load address VALU).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, -1, 0x00020000);
}
__device__ __forceinline__ void bload_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void bload_lds4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 4, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(N) only (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// SiLU with the hardware exp2 and reciprocal (about 2 ulp): z / (1 + e^-z)
__device__ __forceinline__ float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// GATEUP: W = repacked gate/up (ngroups = I/8 groups of 8 gate + 8 up rows,
//   K = H); A rows are the tokens of the bucket entries; out h[slot][I].
// !GATEUP: W = repacked down (ngroups = H/16, K = I); A rows are the bucket
//   slots themselves; out Y[slot][H].
// tiles[t] = (expert, first bucket slot, rows), t < *n_tiles. ngroups must be
// a multiple of 4*CW; ncb = ngroups / (4*CW) column blocks; grid = 8 * ncb *
// ceil(max tiles / 8). a_sinv holds 1/s of every row (nsb equal entries);
// with Q8 the row's Q8_K scale d of every super-block.
// Main loop of one output tile (everything up to the epilogue). The LDS
// buffers come in as separate restrict pointers, so the compiler knows which
// global->LDS load each LDS read depends on and adds no wait of its own
// beyond the fixed ones below (without that knowledge it drains every load in
// flight before each header read).
template <bool GATEUP, int RB, int CW, int NW, bool Q8>
__device__ __forceinline__ void gemm_mainloop(uint8_t *__restrict__ abuf, uint8_t *__restrict__ bqbuf,
                                              uint8_t *__restrict__ hbuf, uint8_t *__restrict__ xsbuf,
                                              float *__restrict__ dxbuf, float *__restrict__ svbuf,
                                              const uint8_t *__restrict__ W, int ngroups,
                                              int nsb, const int32_t *__restrict__ entries, int k,
                                              const f16 *__restrict__ a_hilo, const f16 *__restrict__ a_xs,
                                              const float *__restrict__ a_sinv, int e, int r0, int rows, int rg0,
                                              int wave, f32x4 (&X)[RB][CW], float (&fcur)[CW]) {
    using Sh = GemmShape<RB, CW, NW, Q8>;
    constexpr int kALoads = Sh::ALoads, kBLoads = Sh::BLoads, kHxLoads = Sh::HxLoads;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g = lane >> 4;
    const int K = nsb * kQ4Weights;

    // source row (token for GATEUP, bucket slot otherwise) of tile row r;
    // rows past the end of a partial tile repeat its last row
    auto src_row = [&](int r) {
        const int rr = min(r, rows - 1);
        return GATEUP ? entries[r0 + rr] / k : r0 + rr;
    };

    // ---- per-lane load offsets
    // A (halves): rows 4*(kALoads*wave + i) + lane/16, slot (lane%16) ^ (row%16)
    // (staged rows stay far below 2^32 halves)
    uint32_t arow_o[kALoads];  // bytes
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
        const int r = 4 * kALoads * wave + 4 * i + (lane >> 4);
        const int sl = (lane & 15) ^ (r & 15);
        arow_o[i] = (uint32_t)src_row(r) * (uint32_t)(4 * K) + (uint32_t)sl * 16u;
    }
    const __amdgpu_buffer_rsrc_t rs_a = buf_rsrc(a_hilo);
    // Bq: flat 16-byte slot f = (wave*kBLoads + i)*64 + lane of a half
    // super-block -> group f/64, 16-byte slot f%64 of its 1 KB
    const uint8_t *wtile = W + ((size_t)e * ngroups + rg0) * nsb * kGroupSbBytes;
    const __amdgpu_buffer_rsrc_t rs_w = buf_rsrc(wtile);
    uint32_t boff[kBLoads];
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
        const int f = (wave * kBLoads + i) * 64 + lane;
        boff[i] = (uint32_t)((f >> 6) * nsb * kGroupSbBytes + (f & 63) * 16);
    }
    // headers: flat HdrLoadB-byte slot f -> group f / (256 / HdrLoadB), piece
    // f % (256 / HdrLoadB) of its 256 bytes (after the group's 2 KB of quants)
    constexpr int kHdrLoads = Sh::HdrLoads, kHdrB = Sh::HdrLoadB, kHdrPer = 256 / kHdrB;
    uint32_t hoff[kHdrLoads];
#pragma unroll
    for (int i = 0; i < kHdrLoads; ++i) {
        const int f = (wave * kHdrLoads + i) * 64 + lane;
        hoff[i] = (uint32_t)((f / kHdrPer) * nsb * kGroupSbBytes + kGroupQsBytes + (f % kHdrPer) * kHdrB);
    }
    // k-step sums: XsNarrow: row 8*wave + lane/8, 4-byte piece lane%8;
    // else row 32*(wave%2) + lane/2, 16-byte half lane%2
    const uint32_t xs_o = 2u * (Sh::XsNarrow ? (uint32_t)src_row(8 * wave + (lane >> 3)) * nsb * 16 + (lane & 7) * 2
                                             : (uint32_t)src_row(32 * (wave & 1) + (lane >> 1)) * nsb * 16 + (lane & 1) * 8);
    const __amdgpu_buffer_rsrc_t rs_xs = buf_rsrc(a_xs);
    const uint32_t dx_o = Q8 ? (uint32_t)src_row(lane) * nsb * 4u : 0u;
    const __amdgpu_buffer_rsrc_t rs_dx = buf_rsrc(a_sinv);

    auto issue_a = [&](int c) {  // chunk c into ring slot c % 4   (kALoads loads)
        const int b = c >> 2, q = c & 3;
        uint8_t *dst = abuf + (c & (kGemmRing - 1)) * Sh::ABuf + (4 * kALoads * wave) * kChunkBytes;
#pragma unroll
        for (int i = 0; i < kALoads; ++i) bload_lds16(rs_a, arow_o[i], (uint32_t)(b * 1024 + q * 256), dst + i * 1024);
    };
    auto issue_bq = [&](int hs) {  // quants of half super-block hs into slot hs % 2   (kBLoads loads)
        uint8_t *dst = bqbuf + (hs & 1) * Sh::BqBuf + wave * kBLoads * 1024;
        const uint32_t src = (uint32_t)((hs >> 1) * kGroupSbBytes + (hs & 1) * 1024);
#pragma unroll
        for (int i = 0; i < kBLoads; ++i) bload_lds16(rs_w, boff[i], src, dst + i * 1024);
    };
    auto issue_hx = [&](int b) {  // headers + k-step sums (+ Q8 row scales) of super-block b into buffer b % 2   (kHxLoads loads)
        uint8_t *dst = hbuf + (b & 1) * Sh::HdrBuf + wave * kHdrLoads * 64 * kHdrB;
#pragma unroll
        for (int i = 0; i < kHdrLoads; ++i) {
            if (kHdrB == 16)
                bload_lds16(rs_w, hoff[i], (uint32_t)(b * kGroupSbBytes), dst + i * 1024);
            else
                bload_lds4(rs_w, hoff[i], (uint32_t)(b * kGroupSbBytes), dst + i * 256);
        }
        if (Sh::XsNarrow)
            bload_lds4(rs_xs, xs_o, (uint32_t)(b * 32), xsbuf + (b & 1) * Sh::XsBuf + wave * 256);
        else
            bload_lds16(rs_xs, xs_o, (uint32_t)(b * 32), xsbuf + (b & 1) * Sh::XsBuf + wave * 1024);
        if (Q8)  // the tile rows' scales of super-block b (row lane), one copy per wave
            bload_lds4(rs_dx, dx_o, (uint32_t)(b * 4), dxbuf + (b & 1) * (Sh::DxBuf / 4) + wave * 64);
    };

    // ---- sub-block scales of this lane's CW weight groups (row n) for the
    // current super-block: bytes 0-3 | 4-7, zero where d = 0 (d, dmin and the
    // mins are read again at the boundary, while the headers are still in LDS)
    struct Scales {
        uint32_t lo[CW], hi[CW];
    };
    auto read_scales = [&](int b, Scales &kk) {
        const uint8_t *hb = hbuf + (b & 1) * Sh::HdrBuf + wave * CW * 256;
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) {
            const u32x4 hdr = *(const u32x4 *)(hb + cb * 256 + n * 16);
            const bool live = (hdr.x & 0x7FFFu) != 0u;  // d != 0
            kk.lo[cb] = live ? (hdr.y & 0x3F3F3F3Fu) : 0u;
            kk.hi[cb] = live ? ((hdr.w & 0x0F0F0F0Fu) | ((hdr.y >> 2) & 0x30303030u)) : 0u;
        }
    };
    const NibbleConsts nk = nibble_consts();
    // A fragments of half s2 (k-step 2q + s2) of chunk c: hi and lo of RB row blocks
    auto read_a_half = [&](int c, int s2, f16x8 (&Ah)[RB], f16x8 (&Al)[RB]) {
        const uint8_t *ab = abuf + (c & (kGemmRing - 1)) * Sh::ABuf;
        const int jh = (s2 * 8 + 2 * g) ^ n;
        const int jl = (s2 * 8 + 2 * g + 1) ^ n;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = rb * 16 + n;  // A row of this lane (r % 16 == n)
            Ah[rb] = *(const f16x8 *)(ab + r * kChunkBytes + jh * 16);
            if (!Q8) Al[rb] = *(const f16x8 *)(ab + r * kChunkBytes + jl * 16);  // Q8 codes have no lo part
        }
    };
    // the lane's 16 quant bytes of half super-block hs (chunks 2hs, 2hs + 1:
    // bytes 0-7 and 8-15) in each of its groups, from slot hs % 2; one
    // 16-byte read per lane is free of bank conflicts, two 8-byte reads at a
    // 16-byte stride are not
    auto read_quants = [&](int hs, u32x4 (&w)[CW]) {
        const uint8_t *bq = bqbuf + (hs & 1) * Sh::BqBuf + wave * CW * 1024;
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) w[cb] = *(const u32x4 *)(bq + cb * 1024 + lane * 16);
    };
    // the chunk's 8 bytes and the same shifted right by 8 (shared by its two
    // nibble halves)
    auto quants_of = [&](const u32x4 (&w)[CW], bool odd, u32x4 (&o)[CW]) {
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) {
            const uint32_t a = odd ? w[cb].z : w[cb].x, b = odd ? w[cb].w : w[cb].y;
            o[cb] = u32x4{a, b, a >> 8, b >> 8};
        }
    };
    // fp16 scales and offsets of chunk q's two sub-blocks (2q, 2q + 1) in each
    // group: computed once per chunk, used by its two k-steps
    struct ScalePairs {
        f16x2 sp[CW], np[CW];
    };
    auto scale_pairs = [&](int q, const Scales &kk, ScalePairs &pp) {
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) scale_pair(q < 2 ? kk.lo[cb] : kk.hi[cb], q, pp.sp[cb], pp.np[cb]);
    };
    // B fragments of k-step 2q + s2: sub-block scale x quant (low nibbles for
    // s2 = 0, high for s2 = 1)
    auto build_b_half = [&](int s2, const ScalePairs &pp, const u32x4 (&w)[CW], f16x8 (&Bf)[CW]) {
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) {
            const f16 sc = s2 ? pp.sp[cb].y : pp.sp[cb].x, nc = s2 ? pp.np[cb].y : pp.np[cb].x;
            const f16x2 sc2 = {sc, sc}, n2 = {nc, nc};
            Bf[cb] = s2 ? q_times_scale_nib_sn<1>(w[cb].x, w[cb].y, w[cb].z, w[cb].w, sc2, n2, nk)
                        : q_times_scale_nib_sn<0>(w[cb].x, w[cb].y, w[cb].z, w[cb].w, sc2, n2, nk);
        }
    };

#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) X[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // 16-row tiles (exact activations): the registers allow the plain form,
    // each super-block's MFMA sum P in an accumulator of its own (started from
    // zero by the super-block's first MFMA) and X += d_b P_b once it is
    // complete (at the next super-block's start, and after the last); the
    // min term goes into X as -dmin_b Q_b. No d ratio, reciprocal or rescale:
    // ~9% of those tiles' VALU. 64-row tiles keep the rescaled single
    // accumulator (two would not fit two waves per SIMD), Q8 tiles too (their
    // row scales change per super-block).
    constexpr bool kTwoAcc = RB == 1 && !Q8;
    f32x4 P[CW];
#pragma unroll
    for (int cb = 0; cb < CW; ++cb) P[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mfma_half = [&](const f16x8 (&Ah)[RB], const f16x8 (&Al)[RB], const f16x8 (&Bf)[CW], bool first) {
        if constexpr (kTwoAcc) {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cb = 0; cb < CW; ++cb) P[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah[0], Bf[cb], first ? zero : P[cb], 0, 0, 0);
#pragma unroll
            for (int cb = 0; cb < CW; ++cb) P[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al[0], Bf[cb], P[cb], 0, 0, 0);
            return;
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < CW; ++cb)
                X[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah[rb], Bf[cb], X[rb][cb], 0, 0, 0);
        if (Q8) return;  // codes are exact in the hi part
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < CW; ++cb)
                X[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al[rb], Bf[cb], X[rb][cb], 0, 0, 0);
    };
    // scheduling pattern of a half (2*RB*CW MFMAs): its LDS reads early, two
    // per MFMA, then the unpack VALU spread over the rest, and nld global->LDS
    // loads spread evenly among those MFMAs so that the load pipe is fed
    // steadily instead of in one burst: one after every (slots / nld)-th MFMA,
    // or, with more loads than MFMAs left (16-row and Q8 tiles), ceil(nld /
    // slots) after each (masks: 0x100 LDS read, 0x008 MFMA, 0x002 VALU, 0x020
    // global load)
    auto interleave = [&](int nld) {
        constexpr int kM = (Q8 ? 1 : 2) * RB * CW;
        constexpr int kDs0 = ((Q8 ? 1 : 2) * RB + CW + 1) / 2;
        constexpr int kDs = kDs0 < kM ? kDs0 : kM - 1;  // at least one MFMA left for the VALU groups
        constexpr int kSlots = kM - kDs;
        constexpr int kValuPer = (CW * 10 + kSlots - 1) / kSlots + 1;
        constexpr int kMaxPer = 16;  // bound on loads per slot (nld <= 16 on every shape)
        const int every = nld > kSlots ? 1 : (nld > 0 ? kSlots / nld : kSlots);
        const int per = nld > kSlots ? (nld + kSlots - 1) / kSlots : 1;
#pragma unroll
        for (int i = 0; i < kDs; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);
            if (nld > 0 && i % every == every - 1) {
                const int first = (i / every) * per;
#pragma unroll
                for (int c = 0; c < kMaxPer; ++c)
                    if (c < per && first + c < nld) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
    };
    // the B fragments unpacked in a half must exist at its end (the compiler
    // would otherwise sink their computation past the next barrier); the A
    // fragments are plain LDS reads and are left unpinned, so that the wait
    // for them does not get hoisted in front of the MFMAs
    auto pin = [&](f16x8 (&Bf)[CW]) {
#pragma unroll
        for (int j = 0; j < CW; ++j) asm volatile("" : "+v"(Bf[j]));
    };

    // ---- prologue: the tile rows' scale of the last super-block (1/s, or
    // with Q8 its d; row lane, one copy per wave), then the issue groups of iterations -4 .. -1 (nchunks >= 4):
    // HX(0) A(0) | Bq(0) A(1) | A(2) | Bq(1) A(3)
    load_lds4(a_sinv + (size_t)src_row(lane) * nsb + (nsb - 1), svbuf + wave * 64);  // the last super-block's
    issue_hx(0);
    issue_a(0);
    __builtin_amdgcn_sched_barrier(0);
    issue_bq(0);
    issue_a(1);
    __builtin_amdgcn_sched_barrier(0);
    issue_a(2);
    __builtin_amdgcn_sched_barrier(0);
    issue_bq(1);
    issue_a(3);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<3 * kALoads + kBLoads>();  // chunk 0 landed: at most A(1), A(2), Bq(1), A(3) in flight
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    Scales kc;
    ScalePairs kp;  // of the chunk whose k-steps are being built
    f16x8 Ah0[RB], Al0[RB], B0[CW], Ah1[RB], Al1[RB], B1[CW];
    u32x4 wq[CW];
    u32x4 wfull[CW];  // quants of the current half super-block
    read_scales(0, kc);
    read_quants(0, wfull);
    quants_of(wfull, false, wq);
    read_a_half(0, 0, Ah0, Al0);
    scale_pairs(0, kc, kp);
    build_b_half(0, kp, wq, B0);
    __builtin_amdgcn_sched_barrier(0);

    // Super-block b's min term and its rescale are spread over its
    // iterations (the accumulator is in units of d_b all through b):
    //   q = 1, half 0: X -= (dmin_b / d_b) Q_b   (Q_b on the k-step sums;
    //                  the headers and sums of b stay in LDS until HX(b+2))
    //   q = 3, half 1: f = d_b / d_{b+1} (d_last after the last super-block)
    //   next q = 0, half 0: X *= f, tile by tile ahead of its MFMAs
    // A d of 0 counts as 1 (its scales are zeroed, only the min term is left).
#pragma unroll
    for (int cb = 0; cb < CW; ++cb) fcur[cb] = 1.f;
    auto min_term = [&](int b) {
        const uint8_t *xsb = xsbuf + (b & 1) * Sh::XsBuf;
        const uint8_t *hb = hbuf + (b & 1) * Sh::HdrBuf + wave * CW * 256;
        float r1[CW];
        f16x4 Bm[CW];
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) {
            const u32x4 hdr = *(const u32x4 *)(hb + cb * 256 + n * 16);
            if constexpr (kTwoAcc) {
                r1[cb] = half_bits_to_float(hdr.x >> 16);  // X is in absolute units: -dmin Q
            } else {
                float d = half_bits_to_float(hdr.x & 0xFFFFu);
                d = d != 0.f ? d : 1.f;
                // reciprocal to 1 ulp: far below the bar, and no division sequence
                r1[cb] = half_bits_to_float(hdr.x >> 16) * __builtin_amdgcn_rcpf(d);
            }
            const uint32_t mn_lo = hdr.z & 0x3F3F3F3Fu;
            const uint32_t mn_hi = ((hdr.w >> 4) & 0x0F0F0F0Fu) | ((hdr.z >> 2) & 0x30303030u);
            // this lane's mins 4(g%2) .. 4(g%2)+3 (a select of register
            // values: an array indexed by g%2 would go to scratch), as fp16:
            // byte m under exponent byte 0x64 is the half 1024 + m
            const uint32_t mw = (g & 1) ? mn_hi : mn_lo;
            const f16x2 k1024 = {(f16)1024.f, (f16)1024.f};
            const f16x2 m01 = u32_as_f16x2(__builtin_amdgcn_perm(0x64646464u, mw, 0x04010400u)) - k1024;
            const f16x2 m23 = u32_as_f16x2(__builtin_amdgcn_perm(0x64646464u, mw, 0x04030402u)) - k1024;
            Bm[cb] = f16x4{m01.x, m01.y, m23.x, m23.y};
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const f16x4 Am = *(const f16x4 *)(xsb + (rb * 16 + n) * 32 + g * 8);
#pragma unroll
            for (int cb = 0; cb < CW; ++cb) {
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 Q = __builtin_amdgcn_mfma_f32_16x16x16f16(Am, Bm[cb], zero, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) X[rb][cb][i] -= r1[cb] * Q[i];
            }
        }
    };
    auto next_factor = [&](int b, bool last) {
        const uint8_t *hb = hbuf + (b & 1) * Sh::HdrBuf + wave * CW * 256;
        const uint8_t *hn = hbuf + ((b + 1) & 1) * Sh::HdrBuf + wave * CW * 256;
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) {
            if constexpr (kTwoAcc) {  // d_b for the fold X += d_b P_b (d = 0 adds nothing)
                fcur[cb] = half_bits_to_float(*(const uint32_t *)(hb + cb * 256 + n * 16) & 0xFFFFu);
                continue;
            }
            float d = half_bits_to_float(*(const uint32_t *)(hb + cb * 256 + n * 16) & 0xFFFFu);
            float dn = half_bits_to_float(*(const uint32_t *)(hn + cb * 256 + n * 16) & 0xFFFFu);
            d = d != 0.f ? d : 1.f;
            dn = (dn != 0.f && !last) ? dn : 1.f;  // after the last super-block: stale LDS, dropped
            fcur[cb] = d * __builtin_amdgcn_rcpf(dn);
        }
    };

    // One super-block: 4 iterations. LOADS: every load of the issue groups
    // exists (b < nsb - 1), so each wait is a fixed count and the groups are
    // spread over the MFMAs of half 1. The last super-block issues nothing.
    auto sb_step = [&](int b, auto loads_tag) {
        constexpr bool LOADS = decltype(loads_tag)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 4 * b + q;

            // half 0: MFMAs of (c, 2q) from set 0 | fill set 1 with (c, 2q+1)
            if (q == 0) {
                // Q8: X is also in units of the row's scale D_b (its d, or 1
                // where d = 0: such a block adds nothing), so the rows' factor
                // D_{b-1} / D_b joins the columns' (both scales still in LDS:
                // HX(b+1) refills the older buffer after the next barrier)
                float fr[RB][4];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) fr[rb][i] = 1.f;
                if (Q8 && b > 0) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const f32x4 dp = *(const f32x4 *)(dxbuf + ((b - 1) & 1) * (Sh::DxBuf / 4) + wave * 64 + rb * 16 + 4 * g);
                        const f32x4 dc = *(const f32x4 *)(dxbuf + (b & 1) * (Sh::DxBuf / 4) + wave * 64 + rb * 16 + 4 * g);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            fr[rb][i] = (dp[i] != 0.f ? dp[i] : 1.f) * __builtin_amdgcn_rcpf(dc[i] != 0.f ? dc[i] : 1.f);
                    }
                }
                if constexpr (kTwoAcc) {  // the previous super-block's sum (none before the first: P = 0)
#pragma unroll
                    for (int cb = 0; cb < CW; ++cb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) X[0][cb][i] = __builtin_fmaf(fcur[cb], P[cb][i], X[0][cb][i]);
                } else {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int cb = 0; cb < CW; ++cb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) X[rb][cb][i] *= Q8 ? fcur[cb] * fr[rb][i] : fcur[cb];
                }
            }
            if (q == 1) min_term(b);
            read_a_half(c, 1, Ah1, Al1);
            build_b_half(1, kp, wq, B1);
            mfma_half(Ah0, Al0, B0, q == 0);
            interleave(0);
            pin(B1);
            __builtin_amdgcn_sched_barrier(0);

            // Chunk c+1 needs A(c+1), Bq((c+1)/2) and, at q == 3, HX(b+1).
            // What this wave issued after the last of those is the rest of
            // the issue groups of iterations c-2 | c-1:
            //   q = 0: A(c+2) | Bq, A(c+3)        q = 1: A(c+2) | HX, A(c+3)
            //   q = 2: HX, A(c+2) | Bq, A(c+3)    q = 3: A(c+2) | A(c+3)
            // In the last super-block (no loads) those groups are complete
            // only for q = 0; later waits take everything.
            if (q == 0)
                wait_vm<2 * kALoads + kBLoads>();
            else if (!LOADS)
                wait_vm<0>();
            else if (q == 1)
                wait_vm<2 * kALoads + kHxLoads>();
            else if (q == 2)
                wait_vm<2 * kALoads + kHxLoads + kBLoads>();
            else
                wait_vm<2 * kALoads>();
            __builtin_amdgcn_s_waitcnt(0xC07F);  // own LDS reads done before their buffers are refilled
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);

            // half 1: MFMAs of (c, 2q+1) from set 1 | fill set 0 with the
            // first k-step of chunk c+1 | the issue group of iteration c.
            // After the last chunk the fill reads stale but in-bounds LDS
            // and its results go unused.
            {
                u32x4 wn[CW];
                if (q == 3) {
                    read_scales(b + 1, kc);
                    next_factor(b, !LOADS);
                }
                if ((q & 1) != 0) read_quants((c + 1) >> 1, wfull);  // chunk c+1 starts a half super-block
                quants_of(wfull, ((q + 1) & 1) != 0, wn);
                read_a_half(c + 1, 0, Ah0, Al0);
                scale_pairs((q + 1) & 3, kc, kp);
                build_b_half(0, kp, wn, B0);
#pragma unroll
                for (int cb = 0; cb < CW; ++cb) wq[cb] = wn[cb];
            }
            if constexpr (LOADS) {
                if (q == 0) issue_hx(b + 1);
                if (q & 1) issue_bq((c + 3) / 2);
                issue_a(c + 4);
            }
            mfma_half(Ah1, Al1, B1, false);
            interleave(!LOADS ? 0 : q == 0 ? kHxLoads + kALoads : q == 2 ? kALoads : kBLoads + kALoads);
            pin(B0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int b = 0; b < nsb - 1; ++b) sb_step(b, std::integral_constant<bool, true>{});
    sb_step(nsb - 1, std::integral_constant<bool, false>{});
    wait_vm<0>();  // no load into LDS may still be in flight when the workgroup ends
    if constexpr (kTwoAcc) {  // the last super-block's sum; the epilogue's factor is then 1
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) X[0][cb][i] = __builtin_fmaf(fcur[cb], P[cb][i], X[0][cb][i]);
            fcur[cb] = 1.f;
        }
    }
}

// Last-round balance of a big-tile launch. Per XCD x the launch has n_x =
// tiles_x * ncb units (tile, column block of 2*16 weight groups at 8 waves),
// run one per CU, C CUs at a time; n_x % C units would make a last round that
// leaves most of the XCD idle. When those r_x units fit C as halves (2 r_x <=
// C), the launch skips them (mode 1) and a second launch runs each as two
// independent half-width units (mode 2: 64 x 256 tiles of 8 waves, each wave
// 64 x 32, two per SIMD like the main launch; a 4-wave 64 x 256 instance, one
// wave per SIMD, took 35 against 31 us for the 30b prefill's gate/up halves),
// so the last round is about half as long; outputs do not overlap, nothing
// is summed.
struct TailSplit {
    int per_xcd;  // tiles per XCD (a contiguous range of the tile list)
    int full_x;   // units the main launch runs
    int r_x;      // units split into halves (0: none)
};
__device__ __forceinline__ TailSplit tail_split(int ntl, int ncb, int x, int C) {
    TailSplit t;
    t.per_xcd = (ntl + 7) >> 3;
    const int n_x = max(0, min(t.per_xcd, ntl - x * t.per_xcd)) * ncb;
    const int r = C > 0 ? n_x % C : 0;
    t.r_x = (r > 0 && 2 * r <= C) ? r : 0;
    t.full_x = n_x - t.r_x;
    return t;
}

// Waves per SIMD the register budget is sized for: big tiles run one
// workgroup per CU (NW / 4 waves per SIMD); 16-row tiles as many workgroups
// as their LDS allows (two of 16 x 256; four of 16 x 128, three with the Q8
// row scales), so they must fit 256 or 128 registers (with a budget of 512
// the compiler parks values in accumulator registers and moves them back and
// forth).
template <int RB, int CW, int NW>
constexpr int gemm_waves_per_simd() { return RB == 1 ? (CW == 2 ? 4 : 2) : NW / 4; }

template <bool GATEUP, int RB, int CW, int NW, bool Q8 = false>
__global__ __launch_bounds__(64 * NW, 1) __attribute__((
    amdgpu_waves_per_eu(gemm_waves_per_simd<RB, CW, NW>(), gemm_waves_per_simd<RB, CW, NW>()))) void expert_gemm_kernel(
    const uint8_t *__restrict__ W, int ngroups, int nsb, const int4 *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ entries, int k, const f16 *__restrict__ a_hilo,
    const f16 *__restrict__ a_xs, const float *__restrict__ a_sinv, float *__restrict__ outp, int out_ld, int C,
    int mode) {
    using Sh = GemmShape<RB, CW, NW, Q8>;
    constexpr int NT = 64 * NW;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *abuf = smem;
    uint8_t *bqbuf = abuf + kGemmRing * Sh::ABuf;
    uint8_t *hbuf = bqbuf + 2 * Sh::BqBuf;
    uint8_t *xsbuf = hbuf + 2 * Sh::HdrBuf;
    float *dxbuf = (float *)(smem + Sh::DxOff);
    float *svbuf = (float *)(smem + Sh::SvOff);

    // unit of this workgroup (tail_split): mode 0 every unit of this launch,
    // 1 all but the XCD's split tail units, 2 (the half-width instance) the
    // halves of the 8-wave launch's split units
    const int ntl = *n_tiles;
    const int x = blockIdx.x & 7, sid = blockIdx.x >> 3;
    int tile, rg0;
    if (mode == 2) {
        const int ncb8 = ngroups / (2 * Sh::Groups);
        const TailSplit ts = tail_split(ntl, ncb8, x, C);
        if (sid >= 2 * ts.r_x) return;
        const int u = ts.full_x + (sid >> 1);
        tile = x * ts.per_xcd + u / ncb8;
        rg0 = (u % ncb8) * 2 * Sh::Groups + (sid & 1) * Sh::Groups;
    } else {
        const int ncb = ngroups / Sh::Groups;
        const TailSplit ts = tail_split(ntl, ncb, x, mode == 1 ? C : 0);
        if (sid >= ts.full_x) return;
        tile = x * ts.per_xcd + sid / ncb;
        rg0 = (sid % ncb) * Sh::Groups;
    }
    const u32x4 tr = *(const u32x4 *)&tiles[tile];
    const int e = (int)tr.x, r0 = (int)tr.y, rows = (int)tr.z;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: LDS addresses stay scalar
    const int n = lane & 15, g = lane >> 4;

    f32x4 X[RB][CW];
    float fcur[CW];
    gemm_mainloop<GATEUP, RB, CW, NW, Q8>(abuf, bqbuf, hbuf, xsbuf, dxbuf, svbuf, W, ngroups, nsb, entries, k, a_hilo, a_xs,
                                      a_sinv, e, r0, rows, rg0, wave, X, fcur);

    // results: X of tile rows rb*16 + 4g + i, columns of weight group
    // CW*wave + cb, times d of the last super-block and the row's scale (1/s,
    // or with Q8 its d of the last super-block); staged through LDS (once every wave
    // is done with the loop's buffers), then written row by row with 16-byte
    // stores (rows past the end of a partial tile are not stored)
    float sv[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = svbuf[wave * 64 + rb * 16 + 4 * g + i];
            sv[rb][i] = v != 0.f ? v : 1.f;  // Q8: an all-zero last block has d = 0 (its unit is 1)
        }
    __syncthreads();
    constexpr int OC = GATEUP ? Sh::Groups * 8 : Sh::Groups * kRowGroup;  // output columns of the tile
    float *stg = (float *)smem;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) {
            if (GATEUP) {
                // lanes n < 8 hold gate, lanes n + 8 up of column n of the
                // group's 8 h columns. For rows i and i+1 the two lanes swap
                // one value (gate of row i+1 for up of row i; a DPP rotate
                // by 8 within each 16-lane row), so that each computes one h:
                // lane n < 8 row i, lane n + 8 row i+1.
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float v0 = X[rb][cb][i] * (fcur[cb] * sv[rb][i]);
                    const float v1 = X[rb][cb][i + 1] * (fcur[cb] * sv[rb][i + 1]);
                    const bool gl = n < 8;
                    const float send = gl ? v1 : v0;
                    const float recv = __builtin_bit_cast(
                        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0x128, 0xF, 0xF, false));
                    const float gv = gl ? v0 : recv, uv = gl ? recv : v1;
                    const int row = rb * 16 + 4 * g + i + (gl ? 0 : 1);
                    stg[row * Sh::OutLd + (CW * wave + cb) * 8 + (n & 7)] = silu_fast(gv) * uv;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    stg[(rb * 16 + 4 * g + i) * Sh::OutLd + (CW * wave + cb) * kRowGroup + n] =
                        X[rb][cb][i] * (fcur[cb] * sv[rb][i]);
            }
        }
    }
    __syncthreads();
    constexpr int kV4 = OC / 4;  // 16-byte pieces per row
    float *obase = outp + (size_t)r0 * out_ld + (size_t)rg0 * (GATEUP ? 8 : kRowGroup);
    for (int idx = threadIdx.x; idx < Sh::M * kV4; idx += NT) {
        const int row = idx / kV4, c4 = idx % kV4;
        if (row < rows)
            *(f32x4 *)(obase + (size_t)row * out_ld + c4 * 4) = *(const f32x4 *)(stg + row * Sh::OutLd + c4 * 4);
    }
}

}  // namespace moe
