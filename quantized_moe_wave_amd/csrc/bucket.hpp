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
// another.
#pragma once
#include "common.hpp"
#include "gemm.hpp"

namespace moe {

// GEMM tiles and 16-row tiles of a bucket of c entries.
__device__ __forceinline__ int gemm_tiles_of(int c) { return c >= kGemmMinRows ? (c + kGemmM - 1) / kGemmM : 0; }
__device__ __forceinline__ int small_tiles_of(int c) { return c >= kGemmMinRows ? 0 : (c + kTileM - 1) / kTileM; }

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

    for (int i = tid; i < E; i += 256) cnt[i] = 0;
    __syncthreads();
    for (int s = tid; s < S; s += 256) atomicAdd(&cnt[idx[s]], 1);
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

    // Stable scatter: tokens in ascending order, 256 per pass.
    int base = off;
    for (int t0 = 0; t0 < T; t0 += 256) {
        const int t = t0 + tid;
        int j = -1;
        if (t < T) {
            for (int jj = 0; jj < k; ++jj)
                if (idx[(size_t)t * k + jj] == e) j = jj;
        }
        const bool flag = j >= 0;
        const uint64_t ball = __ballot(flag);
        const int rank_in_wave = __popcll(ball & ((1ull << lane) - 1ull));
        __syncthreads();
        if (lane == 0) wave_tot[0][wave] = __popcll(ball);
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wave; ++w) before += wave_tot[0][w];
        if (flag) {
            const int p = base + before + rank_in_wave;
            entries[p] = t * k + j;
            pos[(size_t)t * k + j] = p;
        }
        base += wave_tot[0][0] + wave_tot[0][1] + wave_tot[0][2] + wave_tot[0][3];
    }
}

}  // namespace moe
