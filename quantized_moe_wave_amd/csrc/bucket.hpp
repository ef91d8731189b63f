// Expert bucketing: a stable counting sort of the T*k (token, slot) pairs by
// chosen expert, plus the list of expert tiles the MFMA kernels walk.
//
// The pages run the layer position by position (forward_qwen3_moe.rs step 2g
// loop; forward_qwen3_moe_cuda_traced.rs step 2g loop), which streams every
// chosen expert's weights once per token. Grouping the tokens of one expert so
// its weights stream once per tile is this library's replacement for that
// loop; the grouping does not change any token's result.
//
// Layout (bit-exact, deterministic): counts[e]; offsets[e] = sum of counts
// below e, offsets[E] = T*k; entries[offsets[e] + r] = t*k + j for the r-th
// pair in token order that chose e. A bucket of at least kGemmMinRows entries
// is cut into tiles of up to kGemmM rows for the grouped GEMM (big_tiles);
// a smaller one into tiles of up to kTileM rows (tiles). Tile records are
// (e, first entry, rows, 0), in expert order. n_tiles[0] = number of small
// tiles, n_tiles[1] = number of GEMM tiles.
//
// Grid: E workgroups (one per expert), 256 threads. Every workgroup builds the
// full histogram in LDS (integer atomics only), so no workgroup waits for
// another. Each thread holds runs of kBkPairs consecutive pairs in registers,
// loaded in one go, so a round costs one memory round trip.
#pragma once
#include "common.hpp"
#include "gemm.hpp"

namespace moe {

// GEMM tiles and 16-row tiles of a bucket of c entries.
__device__ __forceinline__ int gemm_tiles_of(int c) { return c >= kGemmMinRows ? (c + kGemmM - 1) / kGemmM : 0; }
__device__ __forceinline__ int small_tiles_of(int c) { return c >= kGemmMinRows ? 0 : (c + kTileM - 1) / kTileM; }

constexpr int kBkPairs = 32;  // consecutive (token, slot) pairs per thread per round

__global__ __launch_bounds__(256) void bucket_kernel(const int32_t *__restrict__ idx, int T, int k, int E,
                                                     int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                     int32_t *__restrict__ entries, int32_t *__restrict__ pos,
                                                     int4 *__restrict__ tiles, int4 *__restrict__ big_tiles,
                                                     int32_t *__restrict__ n_tiles) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int red[3][4];
    __shared__ int wave_tot[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = blockIdx.x;
    const int S = T * k;
    constexpr int kRound = 256 * kBkPairs;

    // this thread's pairs of a round, loaded together (16 bytes at a time
    // where aligned; pairs past S read as -1)
    const bool vec_ok = ((uintptr_t)idx & 15u) == 0;  // the caller's array may be only 4-byte aligned
    auto load_pairs = [&](int r0, int (&v)[kBkPairs]) {
        const int s0 = r0 + tid * kBkPairs;
#pragma unroll
        for (int i = 0; i < kBkPairs; i += 4) {
            if (vec_ok && s0 + i + 3 < S) {
                const int4 q = *(const int4 *)&idx[s0 + i];
                v[i] = q.x;
                v[i + 1] = q.y;
                v[i + 2] = q.z;
                v[i + 3] = q.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[i + j] = s0 + i + j < S ? idx[s0 + i + j] : -1;
            }
        }
    };

    for (int i = tid; i < E; i += 256) cnt[i] = 0;
    __syncthreads();
    for (int r0 = 0; r0 < S; r0 += kRound) {
        int v[kBkPairs];
        load_pairs(r0, v);
#pragma unroll
        for (int i = 0; i < kBkPairs; ++i)
            if (v[i] >= 0) atomicAdd(&cnt[v[i]], 1);
    }
    __syncthreads();

    // Entries and tiles below expert e.
    int below = 0, tiles_below = 0, big_below = 0, tiles_all = 0, big_all = 0;
    for (int i = tid; i < E; i += 256) {
        const int c = cnt[i];
        const int nb = gemm_tiles_of(c);
        const int ns = small_tiles_of(c);
        tiles_all += ns;
        big_all += nb;
        if (i < e) {
            below += c;
            tiles_below += ns;
            big_below += nb;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        below += __shfl_xor(below, o, kWave);
        tiles_below += __shfl_xor(tiles_below, o, kWave);
        big_below += __shfl_xor(big_below, o, kWave);
        tiles_all += __shfl_xor(tiles_all, o, kWave);
        big_all += __shfl_xor(big_all, o, kWave);
    }
    if (lane == 0) {
        red[0][wave] = below;
        red[1][wave] = tiles_below;
        red[2][wave] = big_below;
        wave_tot[0][wave] = tiles_all;
        wave_tot[1][wave] = big_all;
    }
    __syncthreads();
    const int off = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    const int toff = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    const int boff = red[2][0] + red[2][1] + red[2][2] + red[2][3];
    const int mine = cnt[e];
    const int nbig = gemm_tiles_of(mine);
    const int nsmall = small_tiles_of(mine);
    if (tid == 0) {
        counts[e] = mine;
        offsets[e] = off;
        if (e == E - 1) offsets[E] = off + mine;
        if (e == 0) {
            n_tiles[0] = wave_tot[0][0] + wave_tot[0][1] + wave_tot[0][2] + wave_tot[0][3];
            n_tiles[1] = wave_tot[1][0] + wave_tot[1][1] + wave_tot[1][2] + wave_tot[1][3];
        }
    }
    for (int i = tid; i < nbig; i += 256)
        big_tiles[boff + i] = make_int4(e, off + i * kGemmM, min(kGemmM, mine - i * kGemmM), 0);
    for (int i = tid; i < nsmall; i += 256)
        tiles[toff + i] = make_int4(e, off + i * kTileM, min(kTileM, mine - i * kTileM), 0);
    if (mine == 0) return;

    // Stable scatter: pairs in index order (= token order, a token choosing e
    // at most once). Each thread counts e among its consecutive pairs, a
    // workgroup scan places them, and the thread writes its matches in order.
    __syncthreads();  // wave_tot is reused below
    int base = off;
    for (int r0 = 0; r0 < S; r0 += kRound) {
        int v[kBkPairs];
        load_pairs(r0, v);
        int m = 0;
#pragma unroll
        for (int i = 0; i < kBkPairs; ++i) m += (int)(v[i] == e);
        int incl = m;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += y;
        }
        if (lane == 63) wave_tot[0][wave] = incl;
        __syncthreads();
        int before = incl - m;
        for (int w = 0; w < wave; ++w) before += wave_tot[0][w];
        const int total = wave_tot[0][0] + wave_tot[0][1] + wave_tot[0][2] + wave_tot[0][3];
        int p = base + before;
        const int s0 = r0 + tid * kBkPairs;
#pragma unroll
        for (int i = 0; i < kBkPairs; ++i) {
            if (v[i] == e) {
                entries[p] = s0 + i;
                pos[s0 + i] = p;
                ++p;
            }
        }
        base += total;
        __syncthreads();  // wave_tot is rewritten by the next round
    }
}

}  // namespace moe
