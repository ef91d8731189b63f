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
// a smaller one into tiles of up to kTileM rows (tiles); in calls with
// all_small_tiles (gemm.hpp) every bucket into kTileM-row tiles. Tile records are
// (e, first entry, rows, 0), in expert order. n_tiles[0] = number of small
// tiles, n_tiles[1] = number of GEMM tiles.
//
// Up to kBk1MaxPairs pairs over at most kBk1MaxExperts experts: one launch of
// one workgroup (bucket_single_kernel, below); otherwise two launches over
// chunks of kBkChunk consecutive pairs (one pair per thread), with integer
// arithmetic only:
//   bucket_hist_kernel     the expert histogram of each chunk -> hist[chunk][E]
//   bucket_scatter_kernel  each chunk: totals and its prefix over earlier
//                          chunks from hist, the exclusive scan over experts,
//                          and the place of each of its pairs: the earlier
//                          pairs of the same expert in earlier chunks, in
//                          earlier waves of the chunk, and in lower lanes of
//                          the wave (lanes with equal keys found by ballots);
//                          chunk 0 also writes counts, offsets and the tiles.
// No workgroup reads all pairs, and no counter is contended by a hot expert
// (a wave adds one count per distinct expert it holds).
#pragma once
#include "common.hpp"
#include "gemm.hpp"

namespace moe {

// GEMM tiles and 16-row tiles of a bucket of c entries (all: all_small_tiles
// of the call, every bucket in 16-row tiles).
__device__ __forceinline__ int gemm_tiles_of(int c, bool all) {
    return !all && c >= kGemmMinRows ? (c + kGemmM - 1) / kGemmM : 0;
}
__device__ __forceinline__ int small_tiles_of(int c, bool all) {
    return all || c < kGemmMinRows ? (c + kTileM - 1) / kTileM : 0;
}

constexpr int kBkChunk = 256;  // pairs per chunk = threads per workgroup
constexpr int kBkLoads = 32;   // histogram entries a thread has in flight (64 chunks in one round)

__host__ __device__ inline int bucket_chunks(int S) { return (S + kBkChunk - 1) / kBkChunk; }

constexpr int kBkKeyBits = 11; // keys 0..kMaxExperts (kMaxExperts: "no pair")
static_assert(kMaxExperts < (1 << kBkKeyBits), "keys must fit the ballot match");

// Lanes of this wave whose key equals this lane's, keys of NB bits (every
// lane must call it).
template <int NB = kBkKeyBits>
__device__ __forceinline__ uint64_t lanes_with_key(uint32_t key) {
    uint64_t m = ~0ull;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint32_t bit = (key >> b) & 1u;
        const uint64_t set = __ballot(bit);
        m &= bit ? set : ~set;
    }
    return m;
}

__device__ __forceinline__ uint64_t lanes_below() {
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive scan over n <= 4 * 256 values v[0..n) in LDS by a 256-thread
// workgroup (thread t owns v[t*per .. t*per + per), per = ceil(n / 256)):
// out[i] = sum of v below i (out may alias v); returns the total. Two barriers.
// V = long long scans two 32-bit counts packed in one value (no carry out of
// the low half: its total stays below 2^32).
template <typename V>
__device__ __forceinline__ V block_scan_lds(const V *v, V *out, int n, V *red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n + 255) / 256;
    V loc[4] = {0, 0, 0, 0};
    V sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = tid * per + i;
        if (i < per && j < n) loc[i] = v[j];
        sum += loc[i];
    }
    V incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const V y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    V run = incl - sum;
    for (int w = 0; w < wave; ++w) run += red[w];
    const V total = red[0] + red[1] + red[2] + red[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = tid * per + i;
        if (i < per && j < n) out[j] = run;
        run += loc[i];
    }
    __syncthreads();
    return total;
}

// Grid: bucket_chunks(S) workgroups of kBkChunk threads.
__global__ __launch_bounds__(kBkChunk) void bucket_hist_kernel(const int32_t *__restrict__ idx, int S, int E,
                                                              int32_t *__restrict__ hist) {
    __shared__ int cnt[kMaxExperts];
    const int tid = threadIdx.x;
    const int s = blockIdx.x * kBkChunk + tid;
    const uint32_t key = s < S ? (uint32_t)idx[s] : (uint32_t)kMaxExperts;
    for (int e = tid; e < E; e += kBkChunk) cnt[e] = 0;
    __syncthreads();
    const uint64_t m = lanes_with_key(key);
    if (key < (uint32_t)E && (m & lanes_below()) == 0) atomicAdd(&cnt[key], __popcll(m));
    __syncthreads();
    for (int e = tid; e < E; e += kBkChunk) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Grid: bucket_chunks(S) workgroups of kBkChunk threads.
__global__ __launch_bounds__(kBkChunk) void bucket_scatter_kernel(
    const int32_t *__restrict__ idx, int S, int E, const int32_t *__restrict__ hist, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ entries, int32_t *__restrict__ pos, int4 *__restrict__ tiles,
    int4 *__restrict__ big_tiles, int32_t *__restrict__ n_tiles) {
    __shared__ int tot[kMaxExperts];   // pairs per expert
    __shared__ int base[kMaxExperts];  // its first entry, then + pairs of earlier chunks
    __shared__ int wcnt[4][kMaxExperts];
    __shared__ int red[4];
    const int tid = threadIdx.x, wave = tid >> 6;
    const int chunk = blockIdx.x, nchunks = gridDim.x;
    const int s = chunk * kBkChunk + tid;
    // this thread's pair and its lanes of equal key, ahead of the hist reads
    const uint32_t key = s < S ? (uint32_t)idx[s] : (uint32_t)kMaxExperts;
    for (int e = tid; e < E; e += kBkChunk) {
        tot[e] = 0;
        base[e] = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) wcnt[w][e] = 0;
    }
    __syncthreads();
    // totals and the prefix over earlier chunks: for E <= 256 the 256 / E
    // threads of expert e take every (256 / E)-th chunk, kBkLoads loads in
    // flight per thread, and add their sums in LDS (integer atomics); more
    // experts loop over them
    const int tpe = E <= kBkChunk ? kBkChunk / E : 1;
    if (tid < tpe * E) {
        for (int e = tid % E; e < E; e += kBkChunk) {
            int sum_t = 0, sum_p = 0;
            for (int c0 = tid / E * (E <= kBkChunk); c0 < nchunks; c0 += tpe * kBkLoads) {
                // loads unconditional (chunk clamped), so that no branch splits
                // them and all are in flight together
                int v[kBkLoads];
#pragma unroll
                for (int i = 0; i < kBkLoads; ++i) v[i] = hist[(size_t)min(c0 + i * tpe, nchunks - 1) * E + e];
#pragma unroll
                for (int i = 0; i < kBkLoads; ++i) {
                    const int c = c0 + i * tpe;
                    sum_t += c < nchunks ? v[i] : 0;
                    sum_p += c < chunk ? v[i] : 0;
                }
            }
            atomicAdd(&tot[e], sum_t);
            atomicAdd(&base[e], sum_p);
        }
    }
    const uint64_t m = lanes_with_key(key);
    if (key < (uint32_t)E && (m & lanes_below()) == 0) wcnt[wave][key] = __popcll(m);
    __syncthreads();
    // first entry of every expert: exclusive scan of the totals; chunk 0 also
    // scans the tile counts here, so that no barrier follows a global store
    // (each would wait for the stores to complete)
    __shared__ int off_l[kMaxExperts];
    __shared__ long long toff[kMaxExperts];  // chunk 0: first 16-row tile (low half), first 64-row tile (high)
    __shared__ long long red2[4];
    block_scan_lds(tot, off_l, E, red);
    const bool all = all_small_tiles(S, E);
    int ns = 0, nb = 0;
    if (chunk == 0) {
        for (int e = tid; e < E; e += kBkChunk)
            toff[e] = (long long)small_tiles_of(tot[e], all) + ((long long)gemm_tiles_of(tot[e], all) << 32);
        __syncthreads();
        const long long n2 = block_scan_lds(toff, toff, E, red2);
        ns = (int)(n2 & 0xFFFFFFFFll);
        nb = (int)(n2 >> 32);
    }
    if (key < (uint32_t)E) {
        int r = __popcll(m & lanes_below());
        for (int w = 0; w < wave; ++w) r += wcnt[w][key];
        const int p = off_l[key] + base[key] + r;
        entries[p] = s;
        pos[s] = p;
    }
    if (chunk != 0) return;
    // chunk 0: counts, offsets and the tile lists
    for (int e = tid; e < E; e += kBkChunk) {
        const int c = tot[e], off = off_l[e];
        counts[e] = c;
        offsets[e] = off;
        const int nsm = small_tiles_of(c, all), nbg = gemm_tiles_of(c, all);
        const int so = (int)(toff[e] & 0xFFFFFFFFll), bo = (int)(toff[e] >> 32);
        for (int i = 0; i < nbg; ++i)
            big_tiles[bo + i] = make_int4(e, off + i * kGemmM, min(kGemmM, c - i * kGemmM), 0);
        for (int i = 0; i < nsm; ++i)
            tiles[so + i] = make_int4(e, off + i * kTileM, min(kTileM, c - i * kTileM), 0);
    }
    if (tid == 0) {
        offsets[E] = S;
        n_tiles[0] = ns;
        n_tiles[1] = nb;
    }
}

// Single-workgroup bucketing for small calls: the same layout in one launch,
// for S <= kBk1MaxPairs pairs over E <= kBk1MaxExperts experts (at a few
// thousand pairs two launches cost more than the work; at tens of thousands
// one CU's equal-key matching costs more than the second launch). Wave w owns
// the pairs [w*G*64, (w+1)*G*64), G = ceil(S / (64 * kBk1Waves)) groups of 64
// (its keys loaded up front). Pass 1 counts each wave's pairs per expert (per
// group one LDS add per distinct expert, by its lowest lane); the totals'
// exclusive scan over experts gives each expert's first entry, and within an
// expert the waves follow in order, so each (wave, expert) count becomes that
// wave's first entry for the expert. Pass 2 walks the groups again: a pair's
// entry is its wave's next entry for its expert plus the number of equal keys
// in lower lanes, and the lowest lane advances the wave's next entry. Then
// counts, offsets and the tile lists, as bucket_scatter_kernel's chunk 0.
constexpr int kBk1Waves = 16;
constexpr int kBk1MaxExperts = 256;
constexpr int kBk1MaxPairs = 4096;
constexpr int kBk1MaxGroups = kBk1MaxPairs / (kBk1Waves * 64);  // 64-pair groups per wave

// Exclusive scan of one value per thread over a workgroup of kBk1Waves waves;
// *total = the sum. Two barriers (red: kBk1Waves ints).
__device__ __forceinline__ int bk1_scan(int v, int *red, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kBk1Waves; ++w) {
        before += w < wave ? red[w] : 0;
        all += red[w];
    }
    *total = all;
    __syncthreads();
    return before + incl - v;
}

// Grid: one workgroup of kBk1Waves * 64 threads; 1 <= S <= kBk1MaxPairs.
// NB: key bits, 8 for E <= 255 (no pair = 255), 9 for E = 256 (no pair = 511):
// the equal-key match costs one ballot per bit, per 64 pairs, in both passes.
template <int NB>
__global__ __launch_bounds__(kBk1Waves * 64) void bucket_single_kernel(
    const int32_t *__restrict__ idx, int S, int E, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ entries, int32_t *__restrict__ pos, int4 *__restrict__ tiles, int4 *__restrict__ big_tiles,
    int32_t *__restrict__ n_tiles) {
    __shared__ int wh[kBk1Waves][kBk1MaxExperts];  // per (wave, expert): count, then next entry
    __shared__ int tot[kBk1MaxExperts], off_l[kBk1MaxExperts];
    __shared__ int red[kBk1Waves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = (S + kBk1Waves * 64 - 1) / (kBk1Waves * 64);
    const int s0 = wave * G * 64 + lane;
    // loads unconditional (index clamped) so that all of them are in flight together
    uint32_t keys[kBk1MaxGroups];
#pragma unroll
    for (int i = 0; i < kBk1MaxGroups; ++i) keys[i] = (uint32_t)idx[min(s0 + i * 64, S - 1)];
    static_assert((1 << NB) - 1 >= kBk1MaxExperts - 1, "keys must fit");
#pragma unroll
    for (int i = 0; i < kBk1MaxGroups; ++i)
        if (!(i < G && s0 + i * 64 < S)) keys[i] = (1u << NB) - 1u;  // no pair: above every expert of E < 2^NB
    for (int i = tid; i < kBk1Waves * kBk1MaxExperts; i += kBk1Waves * 64) (&wh[0][0])[i] = 0;
    __syncthreads();
    // pass 1: counts per (wave, expert)
#pragma unroll
    for (int i = 0; i < kBk1MaxGroups; ++i) {
        if (i < G) {
            const uint32_t key = keys[i];
            const uint64_t m = lanes_with_key<NB>(key);
            if (key < (uint32_t)E && (m & lanes_below()) == 0) wh[wave][key] += __popcll(m);
        }
    }
    __syncthreads();
    // totals, their exclusive scan over experts, and each wave's first entry
    int t_e = 0;
    if (tid < E)
        for (int w = 0; w < kBk1Waves; ++w) t_e += wh[w][tid];
    int n_all;
    const int first = bk1_scan(t_e, red, &n_all);
    if (tid < E) {
        tot[tid] = t_e;
        off_l[tid] = first;
        int run = first;
        for (int w = 0; w < kBk1Waves; ++w) {
            const int c = wh[w][tid];
            wh[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    // pass 2: places, in pair order within each wave
#pragma unroll
    for (int i = 0; i < kBk1MaxGroups; ++i) {
        if (i < G) {
            const uint32_t key = keys[i];
            const uint64_t m = lanes_with_key<NB>(key);
            if (key < (uint32_t)E) {
                const int base = wh[wave][key];
                const int p = base + __popcll(m & lanes_below());
                const int s = s0 + i * 64;
                entries[p] = s;
                pos[s] = p;
                if ((m & lanes_below()) == 0) wh[wave][key] = base + __popcll(m);
            }
        }
    }
    // counts, offsets and the tile lists
    const int c_e = tid < E ? tot[tid] : 0;
    if (tid < E) {
        counts[tid] = c_e;
        offsets[tid] = off_l[tid];
    }
    if (tid == 0) offsets[E] = S;
    int ns, nb;
    const bool all = all_small_tiles(S, E);
    const int so = bk1_scan(tid < E ? small_tiles_of(c_e, all) : 0, red, &ns);
    const int bo = bk1_scan(tid < E ? gemm_tiles_of(c_e, all) : 0, red, &nb);
    if (tid < E) {
        const int o = off_l[tid];
        for (int i = 0; i < gemm_tiles_of(c_e, all); ++i)
            big_tiles[bo + i] = make_int4(tid, o + i * kGemmM, min(kGemmM, c_e - i * kGemmM), 0);
        for (int i = 0; i < small_tiles_of(c_e, all); ++i)
            tiles[so + i] = make_int4(tid, o + i * kTileM, min(kTileM, c_e - i * kTileM), 0);
    }
    if (tid == 0) {
        n_tiles[0] = ns;
        n_tiles[1] = nb;
    }
}

}  // namespace moe
