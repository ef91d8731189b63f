// Host side of the C ABI declared in include/moe_ffn.h: validation, weight
// repack, workspace, and the per-call launch sequence.
//
// forward(T) enqueues, all on the caller's stream, with no host wait (T <= 4
// with shapes that fit: the three decode launches of decode.hpp instead):
//   1. router_kernel   logits (fp64), top-k, renormalised weights (T <= 4
//                      outside the decode path), or router_logits_kernel +
//                      topk_token_kernel (topk_kernel for rows longer than
//                      16 super-blocks), the latter also staging the x rows
//   2. bucket_single_kernel (one workgroup; up to 4096 pairs over at most
//                      256 experts), else bucket_hist_kernel +
//                      bucket_scatter_kernel: stable counting sort of
//                      (token, slot) by expert + tiles
//   3. stage_kernel    x rows -> scaled fp16 hi/lo + sub-block sums (only
//                      where step 1 did not stage them)
//   4. expert GATEUP   gate/up Q4_K MFMA + SiLU(g)*u -> h[slot][I]
//   5. stage_kernel    h rows -> staged
//   6. expert DOWN     down Q4_K MFMA -> Y[slot][H]
//   7. combine_kernel  out[t] = sum_j w[t][j] * Y[pos[t][j]]
// forward_block(T) folds the pre-FFN RMSNorm into the router launches (decode:
// the router launch normalises the values it reads; general path: the router
// sums W_r . (x * g) and the top-k launch applies 1/rms and stages the
// normalised row), or, where that does not fit, first runs rmsnorm_kernel
// (hidden -> normalised rows in the workspace); the last kernel adds hidden
// to its output.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe_ffn.h"
#include "bucket.hpp"
#include "common.hpp"
#include "decode.hpp"
#include "expert.hpp"
#include "gemm.hpp"
#include "norm.hpp"
#include "repack.hpp"
#include "router.hpp"
#include "stage.hpp"
#include "stats.hpp"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

#define HIP_TRY(expr)                                                                        \
    do {                                                                                     \
        hipError_t e_ = (expr);                                                              \
        if (e_ != hipSuccess)                                                                \
            return fail(e_ == hipErrorOutOfMemory ? MOE_ERR_OOM : MOE_ERR_DEVICE, "%s: %s (%s)", \
                        #expr, hipGetErrorString(e_), __func__);                             \
    } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace for up to cap tokens (S = cap * k slots).
struct Workspace {
    double *logits = nullptr;     // [T][E]
    double *lpart = nullptr;      // [kRlPartDoubles] partial logits of the split router
    int32_t *idx = nullptr;       // [T][k] (used when the caller passes no router_idx)
    float *w = nullptr;           // [T][k] (used when the caller passes no router_out)
    uint32_t *rcount = nullptr;   // [token groups] router completion counters (kept at zero)
    int32_t *counts = nullptr;    // [E]
    int32_t *offsets = nullptr;   // [E+1]
    int32_t *entries = nullptr;   // [S]
    int32_t *pos = nullptr;       // [S]
    int4 *tiles = nullptr;        // [max tiles] 16-row tiles
    int4 *big_tiles = nullptr;    // [max_gemm_tiles] GEMM tiles (up to 64 rows)
    int32_t *n_tiles = nullptr;   // [2] small, big
    int32_t *hist = nullptr;      // [bucket_chunks(S)][E] per-chunk expert histogram
    f16 *x_hilo = nullptr;        // [T][2H]
    f16 *x_xs = nullptr;          // [T][H/256][16]
    float *x_sinv = nullptr;      // [T][H/256]
    float *h = nullptr;           // [S][I]
    f16 *h_hilo = nullptr;        // [S][2I]
    f16 *h_xs = nullptr;          // [S][I/256][16]
    float *h_sinv = nullptr;      // [S][I/256]
    float *Y = nullptr;           // [S][H]
    float *xn = nullptr;          // [T][H] the block's normalised rows (moe_ffn_forward_block)
    int32_t *dsel = nullptr;      // [S] decode path: expert of each (token, slot) pair
    float *dw = nullptr;          // [S] decode path: its renormalised router weight
};

// 16-row tiles: buckets of fewer than kGemmMinRows (<= 16) entries, one tile
// each, or in calls with all_small_tiles every bucket. Room for the 16-row tile list of any call of up to S pairs: max_small_tiles
// over S' <= S (calls with all_small_tiles take up to S'/kTileM + E tiles).
int max_tiles(int S, int E) {
    const int s16 = S < E * kTileM ? S : E * kTileM;
    return s16 / kTileM + (S < E ? S : E);
}
static_assert(kGemmMinRows <= kTileM + 1, "a small bucket must fit one 16-row tile");

enum Stage {
    kStRouter = 0,
    kStTopk,
    kStBucket,
    kStStageX,
    kStGateUp,
    kStGateUpBig,
    kStStageH,
    kStDown,
    kStDownBig,
    kStCombine,
    kStGateUpTail,
    kStDownTail,
    kStNorm,
    kStBucketScatter,
    kStCount
};
const char *const kStageNames[kStCount] = {"router",      "topk",    "bucket",   "stage_x",  "gate_up",
                                           "gate_up_big", "stage_h", "down",     "down_big", "combine",
                                           "gate_up_tail", "down_tail", "norm", "bucket_scatter"};

// Start/stop events of profiled stages. A profiled kernel is launched with
// hipExtLaunchKernelGGL, which timestamps the kernel's own start and end.
struct Profiler {
    uint32_t mask = 0;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs[kStCount];
    size_t used[kStCount] = {};
    // Next free event pair of stage s, or {nullptr, nullptr} if s is not profiled.
    std::pair<hipEvent_t, hipEvent_t> next(int s) {
        if (!((mask >> s) & 1)) return {nullptr, nullptr};
        if (used[s] == pairs[s].size()) {
            hipEvent_t a = nullptr, b = nullptr;
            if (hipEventCreate(&a) != hipSuccess) return {nullptr, nullptr};
            if (hipEventCreate(&b) != hipSuccess) {
                (void)hipEventDestroy(a);
                return {nullptr, nullptr};
            }
            pairs[s].push_back({a, b});
        }
        return pairs[s][used[s]++];
    }
    ~Profiler() {
        for (auto &v : pairs)
            for (auto &p : v) {
                (void)hipEventDestroy(p.first);
                (void)hipEventDestroy(p.second);
            }
    }
};

// Launch kernel on st with dynamic LDS; if stage s is profiled, bracket it
// with its events.
template <typename... KArgs, typename... Args>
void launch_lds(Profiler &pf, int s, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                Args... args) {
    auto ev = pf.next(s);
    if (ev.first)
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, ev.first, ev.second, 0,
                              static_cast<KArgs>(args)...);
    else
        kernel<<<grid, block, lds, st>>>(static_cast<KArgs>(args)...);
}

// Launch kernel on st; if stage s is profiled, bracket it with its events.
template <typename... KArgs, typename... Args>
void launch(Profiler &pf, int s, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st, Args... args) {
    auto ev = pf.next(s);
    if (ev.first)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.first, ev.second, 0, static_cast<KArgs>(args)...);
    else
        kernel<<<grid, block, 0, st>>>(static_cast<KArgs>(args)...);
}

}  // namespace

struct moe_ffn_s {
    moe_ffn_shape sh{};
    int device = -1;
    int cus_per_xcd = 0;     // compute units per XCD (0: the big GEMMs' last round is not split)
    uint8_t *gu = nullptr;   // repacked gate/up
    uint8_t *dn = nullptr;   // repacked down
    float *rw = nullptr;     // [E][H]
    float *rb = nullptr;     // [E] or null
    float *norm_w = nullptr; // [H] pre-FFN norm weight (moe_ffn_set_norm), or null
    float norm_eps = 0.f;
    void *ws_base = nullptr;
    int cap = 0;             // tokens the workspace holds
    Workspace ws;
    int last_T = 0;
    bool last_decode = false;  // whether the most recent forward took the decode path (h rows in pair order)
    Workspace *last_ws = nullptr;  // workspace of the most recent forward (ws, or scratch_ws)
    Profiler prof;
    uint8_t *scratch = nullptr;    // this device's copy of the no-alloc scratch (device address)
    Workspace scratch_ws;          // layout of the most recent no-alloc forward over it
};

// Scratch of moe_ffn_forward_noalloc: the workspace of every call of that
// entry point on a device, so that it allocates nothing. Each device holds its
// own copy of the array (from the library's load until the process ends); in
// host code its name is only a stand-in, and the device address of this
// device's copy comes from hipGetSymbolAddress (scratch_address, called once
// per device by moe_ffn_create with that device current).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's scratch (dev: the current device).
hipError_t scratch_address(int dev, uint8_t **out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_addr[dev] = (uint8_t *)p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

__global__ void zero_u32_kernel(uint32_t *__restrict__ p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

bool is_device_ptr(const void *p) {
    if (!p) return false;
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged;
}

moe_status check_shape(const moe_ffn_shape *s) {
    if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    const int H = s->hidden_dim, E = s->num_experts, k = s->num_experts_per_tok, I = s->moe_intermediate;
    if (E <= 0 || k <= 0 || I <= 0)
        return fail(MOE_ERR_INVALID_SHAPE,
                    "incomplete MoE shape: num_experts=%d num_experts_per_tok=%d moe_intermediate=%d (all must be > 0)",
                    E, k, I);
    if (k > E) return fail(MOE_ERR_INVALID_SHAPE, "num_experts_per_tok (%d) exceeds num_experts (%d)", k, E);
    if (H <= 0 || H % kQ4Weights || I % kQ4Weights)
        return fail(MOE_ERR_INVALID_SHAPE, "hidden_dim (%d) and moe_intermediate (%d) must be positive multiples of 256",
                    H, I);
    if (E > kMaxExperts || k > kMaxTopK)
        return fail(MOE_ERR_INVALID_SHAPE, "num_experts (%d) must be <= %d and num_experts_per_tok (%d) <= %d", E,
                    kMaxExperts, k, kMaxTopK);
    if ((long long)H * I > (1ll << 31) / 4 || (long long)E * H * I / 256 * 144 > (1ll << 40))
        return fail(MOE_ERR_INVALID_SHAPE, "shape too large");
    return MOE_OK;
}

size_t gate_bytes_of(const moe_ffn_shape &s) {
    return (size_t)s.num_experts * s.moe_intermediate * (s.hidden_dim / kQ4Weights) * kQ4Bytes;
}
size_t down_bytes_of(const moe_ffn_shape &s) {
    return (size_t)s.num_experts * s.hidden_dim * (s.moe_intermediate / kQ4Weights) * kQ4Bytes;
}

// Carve the workspace for cap tokens out of one allocation; returns its size.
size_t layout_ws(const moe_ffn_shape &s, int cap, char *base, Workspace *w) {
    const size_t T = cap, E = s.num_experts, k = s.num_experts_per_tok, H = s.hidden_dim, I = s.moe_intermediate;
    const size_t S = T * k, nh = H / kQ4Weights, ni = I / kQ4Weights;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char *p = base ? base + off : nullptr;
        off = align_up(off + bytes);
        return p;
    };
    w->logits = (double *)take(T * E * 8);
    w->lpart = (double *)take((size_t)kRlPartDoubles * 8);
    w->idx = (int32_t *)take(S * 4);
    w->w = (float *)take(S * 4);
    w->rcount = (uint32_t *)take(T * 4);
    w->counts = (int32_t *)take(E * 4);
    w->offsets = (int32_t *)take((E + 1) * 4);
    w->entries = (int32_t *)take(S * 4);
    w->pos = (int32_t *)take(S * 4);
    w->tiles = (int4 *)take((size_t)max_tiles((int)S, (int)E) * sizeof(int4));
    w->big_tiles = (int4 *)take((size_t)max_gemm_tiles((int)S, (int)E) * sizeof(int4));
    w->n_tiles = (int32_t *)take(8);
    w->hist = (int32_t *)take((size_t)bucket_chunks((int)S) * E * 4);
    w->x_hilo = (f16 *)take(T * 2 * H * 2);
    w->x_xs = (f16 *)take(T * nh * 16 * 2);
    w->x_sinv = (float *)take(T * nh * 4);
    w->h = (float *)take(S * I * 4);
    w->h_hilo = (f16 *)take(S * 2 * I * 2);
    w->h_xs = (f16 *)take(S * ni * 16 * 2);
    w->h_sinv = (float *)take(S * ni * 4);
    w->Y = (float *)take(S * H * 4);
    w->xn = (float *)take(T * H * 4);
    w->dsel = (int32_t *)take(S * 4);
    w->dw = (float *)take(S * 4);
    return off;
}

moe_status ensure_ws(moe_ffn_t h, int T, hipStream_t st) {
    if (T <= h->cap) return MOE_OK;
    Workspace w;
    const size_t bytes = layout_ws(h->sh, T, nullptr, &w);
    HIP_TRY(hipStreamSynchronize(st));
    if (h->ws_base) {
        HIP_TRY(hipFree(h->ws_base));
        h->ws_base = nullptr;
        h->cap = 0;
    }
    void *base = nullptr;
    HIP_TRY(hipMalloc(&base, bytes));
    layout_ws(h->sh, T, (char *)base, &w);
    // router completion counters must start at zero; the kernel returns them to zero
    hipError_t e = hipMemsetAsync(w.rcount, 0, (size_t)T * 4, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        (void)hipFree(base);
        return fail(MOE_ERR_DEVICE, "workspace init failed: %s", hipGetErrorString(e));
    }
    h->ws_base = base;
    h->ws = w;
    h->cap = T;
    return MOE_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + nb && pb < pa + na;
}

template <int TT, int EV>
void launch_router(moe_ffn_t h, Workspace &ws, Profiler &pf, int T, const float *x, int32_t *idx, float *w,
                   hipStream_t st) {
    const moe_ffn_shape &s = h->sh;
    dim3 grid((T + TT - 1) / TT, (s.num_experts + 4 * EV - 1) / (4 * EV));
    launch(pf, kStRouter, router_kernel<TT, EV>, grid, dim3(256), st, x, h->rw, h->rb, T, s.hidden_dim,
           s.num_experts, s.num_experts_per_tok, ws.logits, idx, w, ws.rcount);
}

// Argument checks shared by the forward entry points (x is the layer's input,
// or the block's residual stream).
moe_status check_call(moe_ffn_t h, int32_t T, const float *x, float *out, float *router_out, int32_t *router_idx) {
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (T < 1) return fail(MOE_ERR_INVALID_SHAPE, "token count must be >= 1 (got %d)", T);
    const moe_ffn_shape &s = h->sh;
    const int k = s.num_experts_per_tok, H = s.hidden_dim, I = s.moe_intermediate;
    // the grouped GEMMs address staged rows with 32-bit byte offsets
    if ((uint64_t)T * 4 * H >= (1ull << 32) || (uint64_t)T * k * 4 * I >= (1ull << 32))
        return fail(MOE_ERR_INVALID_SHAPE, "token count %d too large for this layer (T*4*H and T*k*4*I must be < 2^32)",
                    T);
    if (!x || !out) return fail(MOE_ERR_INVALID_ARG, "x and out must not be NULL");
    if (!is_device_ptr(x) || !is_device_ptr(out) || (router_out && !is_device_ptr(router_out)) ||
        (router_idx && !is_device_ptr(router_idx)))
        return fail(MOE_ERR_INVALID_ARG, "x, out, router_out, router_idx must be device pointers");
    const size_t xb = (size_t)T * H * 4, kb = (size_t)T * k * 4;
    if (overlaps(x, xb, out, xb)) return fail(MOE_ERR_INVALID_ARG, "out overlaps x");
    if (router_out && (overlaps(router_out, kb, x, xb) || overlaps(router_out, kb, out, xb)))
        return fail(MOE_ERR_INVALID_ARG, "router_out overlaps x or out");
    if (router_idx && (overlaps(router_idx, kb, x, xb) || overlaps(router_idx, kb, out, xb) ||
                       (router_out && overlaps(router_idx, kb, router_out, kb))))
        return fail(MOE_ERR_INVALID_ARG, "router_idx overlaps another buffer");
    return MOE_OK;
}

// Whether T tokens take the decode path (decode.hpp): few tokens, and shapes
// whose staged row, ranking and per-token down units fit its kernels.
bool decode_path(const moe_ffn_shape &s, int T) {
    const int H = s.hidden_dim, E = s.num_experts, k = s.num_experts_per_tok, ni = s.moe_intermediate / kQ4Weights;
    return T <= kSmallT && H <= kSmallMaxH && E <= kRankMaxExperts && k * ni <= kMaxTopK * 6;
}

// Whether the block's RMSNorm folds into the general path's router and top-k
// launches: the MFMA router with the rank top-k after it, and rows that fit
// the top-k wave's registers.
bool fold_norm_general(const moe_ffn_shape &s, int T) {
    const int nh = s.hidden_dim / kQ4Weights;
    return T > 4 && s.num_experts <= kRankMaxExperts && (nh + 1) / 2 <= kStageRegPairs;
}

// Dynamic LDS limits of the grouped GEMM instances (above the default).
template <bool Q8>
hipError_t gemm_lds_limits() {
    const hipError_t a[6] = {
        hipFuncSetAttribute((const void *)expert_gemm_kernel<true, 4, 2, 8, Q8>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)GemmShape<4, 2, 8, Q8>::Lds),
        hipFuncSetAttribute((const void *)expert_gemm_kernel<false, 4, 2, 8, Q8>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)GemmShape<4, 2, 8, Q8>::Lds),
        hipFuncSetAttribute((const void *)expert_gemm_kernel<true, 4, 4, 8, Q8>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)GemmShape<4, 4, 8, Q8>::Lds),
        hipFuncSetAttribute((const void *)expert_gemm_kernel<false, 4, 4, 8, Q8>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)GemmShape<4, 4, 8, Q8>::Lds),
        hipFuncSetAttribute((const void *)expert_gemm_kernel<true, 1, 2, 4, Q8>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)GemmShape<1, 2, 4, Q8>::Lds),
        hipFuncSetAttribute((const void *)expert_gemm_kernel<false, 1, 2, 4, Q8>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)GemmShape<1, 2, 4, Q8>::Lds)};
    for (hipError_t e : a)
        if (e != hipSuccess) return e;
    return hipSuccess;
}

// The expert matmuls of the general path: gate/up grouped GEMMs into h, h
// staged, down grouped GEMMs into Y. Q8: Q8_K-style activation codes (x staged
// so by the caller, h here), one MFMA pass.
template <bool Q8>
void expert_gemms(moe_ffn_t h, Workspace &w, Profiler &pf, int32_t T, hipStream_t st) {
    const moe_ffn_shape &s = h->sh;
    const int E = s.num_experts, k = s.num_experts_per_tok, H = s.hidden_dim, I = s.moe_intermediate;
    const int S = T * k;
    const int nh = H / kQ4Weights, ni = I / kQ4Weights;
    // Grouped GEMM grids: 8 XCD lanes x column blocks x ceil(max tiles / 8)
    // (see gemm.hpp); 16-row x 128-column tiles (4 waves, four workgroups per
    // CU) for buckets of at most 16 entries, 64-row x 512-column tiles (8
    // waves of 64 x 64) for larger ones, or 64 x 256 (8 waves of 64 x 32)
    // where the weight groups do not split into blocks of 32.
    const int gu_groups = I / 8, dn_groups = H / kRowGroup;
    const int ms8 = (max_small_tiles(S, E) + 7) / 8, mg8 = (max_gemm_tiles(S, E) + 7) / 8;
    using Small = GemmShape<1, 2, 4, Q8>;
    using Big = GemmShape<4, 4, 8, Q8>;
    using Half = GemmShape<4, 2, 8, Q8>;
    // big tiles: the 8-wave launch leaves each XCD's split tail units (see
    // tail_split in gemm.hpp) to a second 8-wave launch that runs them as
    // 64 x 256 halves (each wave 64 x 32, two waves per SIMD);
    // only where there are enough pairs for several big tiles per XCD (with
    // few or none the extra launch costs more than it saves)
    const int C = S >= (size_t)E * kGemmMinRows ? h->cus_per_xcd : 0;
    launch_lds(pf, kStGateUp, expert_gemm_kernel<true, 1, 2, 4, Q8>, dim3(8 * (gu_groups / Small::Groups) * ms8),
               dim3(256), Small::Lds, st, h->gu, gu_groups, nh, w.tiles, w.n_tiles, w.entries, k, w.x_hilo,
               w.x_xs, w.x_sinv, w.h, I, 0, 0);
    const bool big = S >= kGemmMinRows && !all_small_tiles(S, E);  // else no 64-row tile exists
    if (big) {
        launch_lds(pf, kStGateUpBig, expert_gemm_kernel<true, 4, 4, 8, Q8>, dim3(8 * (gu_groups / Big::Groups) * mg8),
                   dim3(512), Big::Lds, st, h->gu, gu_groups, nh, w.big_tiles, w.n_tiles + 1, w.entries, k,
                   w.x_hilo, w.x_xs, w.x_sinv, w.h, I, C, 1);
        if (C > 0)
            launch_lds(pf, kStGateUpTail, expert_gemm_kernel<true, 4, 2, 8, Q8>, dim3(8 * C), dim3(512), Half::Lds, st,
                       h->gu, gu_groups, nh, w.big_tiles, w.n_tiles + 1, w.entries, k, w.x_hilo, w.x_xs, w.x_sinv,
                       w.h, I, C, 2);
    }

    launch(pf, kStStageH, stage_kernel, dim3((unsigned)((S + 3) / 4)), dim3(256), st, w.h, S, I, I, w.h_hilo, w.h_xs,
           w.h_sinv, (int)Q8);

    launch_lds(pf, kStDown, expert_gemm_kernel<false, 1, 2, 4, Q8>, dim3(8 * (dn_groups / Small::Groups) * ms8),
               dim3(256), Small::Lds, st, h->dn, dn_groups, ni, w.tiles, w.n_tiles, w.entries, k, w.h_hilo,
               w.h_xs, w.h_sinv, w.Y, H, 0, 0);
    if (big) {
        if (gemm_big_groups(dn_groups) == Big::Groups) {
            launch_lds(pf, kStDownBig, expert_gemm_kernel<false, 4, 4, 8, Q8>,
                       dim3(8 * (dn_groups / Big::Groups) * mg8), dim3(512), Big::Lds, st, h->dn, dn_groups, ni,
                       w.big_tiles, w.n_tiles + 1, w.entries, k, w.h_hilo, w.h_xs, w.h_sinv, w.Y, H, C, 1);
            if (C > 0)
                launch_lds(pf, kStDownTail, expert_gemm_kernel<false, 4, 2, 8, Q8>, dim3(8 * C), dim3(512), Half::Lds,
                           st, h->dn, dn_groups, ni, w.big_tiles, w.n_tiles + 1, w.entries, k, w.h_hilo, w.h_xs,
                           w.h_sinv, w.Y, H, C, 2);
        } else {
            launch_lds(pf, kStDownBig, expert_gemm_kernel<false, 4, 2, 8, Q8>,
                       dim3(8 * (dn_groups / Half::Groups) * mg8), dim3(512), Half::Lds, st, h->dn, dn_groups, ni,
                       w.big_tiles, w.n_tiles + 1, w.entries, k, w.h_hilo, w.h_xs, w.h_sinv, w.Y, H, 0, 0);
        }
    }

}

// The layer on T tokens of x (already checked); resid, if not null, is added
// to the output by the kernel that writes it (the block's residual add).
// norm_w (decode path only): x is the residual stream and the router launch
// applies the block's RMSNorm (weight norm_w, eps) to every value it reads.
// q8: the experts' matvecs take Q8_K-style codes of x and h (the staging
// launches store the codes instead; the grouped GEMMs run one MFMA pass).
// w: the workspace of this call, laid out for at least T tokens (the handle's
// own, or the no-alloc variant's scratch); pf: the stage profiler to use.
moe_status forward_layer(moe_ffn_t h, Workspace &w, Profiler &pf, int32_t T, const float *x, float *out,
                         float *router_out, int32_t *router_idx, const float *resid, const float *norm_w, double eps,
                         int q8, hipStream_t st) {
    const moe_ffn_shape &s = h->sh;
    const int E = s.num_experts, k = s.num_experts_per_tok, H = s.hidden_dim, I = s.moe_intermediate;
    int32_t *idx = router_idx ? router_idx : w.idx;
    float *wt = router_out ? router_out : w.w;
    const int S = T * k;
    const int nh = H / kQ4Weights, ni = I / kQ4Weights;

    if (norm_w && !decode_path(s, T) && !fold_norm_general(s, T))
        return fail(MOE_ERR_INVALID_ARG, "internal: fused norm where the router cannot take it");
    if (decode_path(s, T)) {
        // decode path: three launches (see decode.hpp)
        auto rk = T == 1 ? router_small_kernel<1> : T == 2 ? router_small_kernel<2> : T == 3 ? router_small_kernel<3>
                                                                                       : router_small_kernel<4>;
        launch(pf, kStRouter, rk, dim3(E + T * nh), dim3(64), st, x, h->rw, h->rb, T, H, E,
               w.logits, w.x_hilo, w.x_xs, w.x_sinv, norm_w, eps, q8);
        launch(pf, kStGateUp, gateup_pair_kernel, dim3(S, I / 8), dim3(kGpWaves * 64), st, h->gu, I / 8, nh, w.logits, E, k,
               w.x_hilo, w.x_xs, w.x_sinv, w.h, I, w.dsel, w.dw);
        launch(pf, kStDown, down_combine_small_kernel, dim3(2 * (H / kRowGroup) + 1, T), dim3(kDcWaves * 64), st, h->dn,
               H / kRowGroup, ni, w.logits, E, T, k, w.h, I, w.dsel, w.dw, resid, out, H, idx, wt, w.counts, w.offsets,
               w.entries, w.pos, q8);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
        h->last_T = T;
        h->last_decode = true;
        h->last_ws = &w;
        return MOE_OK;
    }
    bool staged_x = false;
    if (T == 1) {
        launch_router<1, 1>(h, w, pf, T, x, idx, wt, st);
    } else if (T <= 4) {
        launch_router<4, 1>(h, w, pf, T, x, idx, wt, st);
    } else {
        // few token tiles: split H over more workgroups, up to 256 of them
        // (partials summed in split order by the top-k kernel; rtiles * ks <=
        // 256 keeps ks*T*E <= 1024 * rtiles * ks <= kRlPartDoubles; 235b
        // shape at T = 512: 26.8 -> 16.4 us against a split up to 128)
        // many token tiles: 8 waves per workgroup (two per SIMD) where each
        // wave's share of H is whole 64-column groups; few: 4 waves, and the
        // split over workgroups below supplies the parallelism
        const int rtiles = ((T + kRlTok - 1) / kRlTok) * ((E + kRlExp - 1) / kRlExp);
        const int nwv = H % 512 == 0 && rtiles >= 128 ? 8 : 4;
        int ks = 1;
        if (E <= kRankMaxExperts)
            while (ks < kRlMaxSplit && rtiles * 2 * ks <= 256 && (H / (64 * nwv)) % (2 * ks) == 0) ks *= 2;
        if (ks > 1 && (size_t)ks * T * E > (size_t)kRlPartDoubles)  // ks = 1 writes the logits directly
            return fail(MOE_ERR_INVALID_ARG, "internal: router split %d exceeds the partial-logit buffer", ks);
        const dim3 rgrid((T + kRlTok - 1) / kRlTok, (E + kRlExp - 1) / kRlExp, ks);
        // with the block's norm folded in, the router leaves 1/rms and the
        // bias to the top-k launch
        const float *rbias = norm_w ? nullptr : h->rb;
        if (nwv == 8)
            launch(pf, kStRouter, norm_w ? router_logits_kernel<8, true> : router_logits_kernel<8, false>, rgrid,
                   dim3(512), st, x, h->rw, rbias, T, H, E, w.logits, ks, w.lpart, norm_w);
        else
            launch(pf, kStRouter, norm_w ? router_logits_kernel<4, true> : router_logits_kernel<4, false>, rgrid,
                   dim3(256), st, x, h->rw, rbias, T, H, E, w.logits, ks, w.lpart, norm_w);
        if (E <= kRankMaxExperts) {
            // the top-k launch also stages x (normalised, with the block's
            // norm): one token per workgroup of 4 waves where the row fits
            // their registers, else one per wave
            const bool per_token = (nh + 1) / 2 <= kStageRegPairs;
            auto topk = per_token
                            ? (norm_w ? (E <= 64 ? topk_token_kernel<1, true> : E <= 128 ? topk_token_kernel<2, true>
                                                                                         : topk_token_kernel<4, true>)
                                      : (E <= 64 ? topk_token_kernel<1, false> : E <= 128 ? topk_token_kernel<2, false>
                                                                                          : topk_token_kernel<4, false>))
                            : (norm_w ? (E <= 64 ? topk_kernel<1, true> : E <= 128 ? topk_kernel<2, true>
                                                                                   : topk_kernel<4, true>)
                                      : (E <= 64 ? topk_kernel<1, false> : E <= 128 ? topk_kernel<2, false>
                                                                                    : topk_kernel<4, false>));
            launch(pf, kStTopk, topk, dim3(per_token ? T : (T + 3) / 4), dim3(256), st, w.logits, T, E, k, idx, wt, ks,
                   w.lpart, x, H, w.x_hilo, w.x_xs, w.x_sinv, norm_w, eps, norm_w ? h->rb : nullptr, q8);
            staged_x = true;
        } else {
            launch(pf, kStTopk, topk_wide_kernel, dim3((T + 3) / 4), dim3(256), st, w.logits, T, E, k, idx, wt);
        }
    }

    if (S <= kBk1MaxPairs && E <= kBk1MaxExperts) {
        launch(pf, kStBucket, E <= 255 ? bucket_single_kernel<8> : bucket_single_kernel<9>, dim3(1), dim3(kBk1Waves * 64), st, idx, S, E, w.counts, w.offsets,
               w.entries, w.pos, w.tiles, w.big_tiles, w.n_tiles);
    } else {
        const int nchunks = bucket_chunks(S);
        launch(pf, kStBucket, bucket_hist_kernel, dim3(nchunks), dim3(kBkChunk), st, idx, S, E, w.hist);
        launch(pf, kStBucketScatter, bucket_scatter_kernel, dim3(nchunks), dim3(kBkChunk), st, idx, S, E, w.hist,
               w.counts, w.offsets, w.entries, w.pos, w.tiles, w.big_tiles, w.n_tiles);
    }

    if (!staged_x)
        launch(pf, kStStageX, stage_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), st, x, T, H, H, w.x_hilo,
               w.x_xs, w.x_sinv, q8);

    if (q8)
        expert_gemms<true>(h, w, pf, T, st);
    else
        expert_gemms<false>(h, w, pf, T, st);

    launch(pf, kStCombine, combine_kernel, dim3((H + 1023) / 1024, T), dim3(256), st, w.Y, w.pos, wt, H, k, resid, out);

    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    h->last_T = T;
    h->last_decode = false;
    h->last_ws = &w;
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_ffn_abi_version(void) { return MOE_FFN_ABI_VERSION; }

const char *moe_ffn_last_error(void) { return g_err.c_str(); }

moe_status moe_ffn_create(const moe_ffn_shape *shape, const void *gate_q4k, size_t gate_bytes, const void *up_q4k,
                          size_t up_bytes, const void *down_q4k, size_t down_bytes, const float *router_w,
                          const float *router_bias, void *stream, moe_ffn_t *out) {
    g_err.clear();
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out handle pointer is NULL");
    *out = nullptr;
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_ffn_shape s = *shape;
    const size_t gb = gate_bytes_of(s), db = down_bytes_of(s);
    if (gate_bytes != gb || up_bytes != gb || down_bytes != db)
        return fail(MOE_ERR_BLOB_SIZE, "blob sizes gate=%zu up=%zu down=%zu, shape needs gate=up=%zu down=%zu",
                    gate_bytes, up_bytes, down_bytes, gb, db);
    if (!gate_q4k || !up_q4k || !down_q4k || !router_w)
        return fail(MOE_ERR_INVALID_ARG, "gate, up, down and router_w must not be NULL");
    if (!is_device_ptr(gate_q4k) || !is_device_ptr(up_q4k) || !is_device_ptr(down_q4k) || !is_device_ptr(router_w) ||
        (router_bias && !is_device_ptr(router_bias)))
        return fail(MOE_ERR_INVALID_ARG, "weights must be device pointers");
    hipStream_t hs = (hipStream_t)stream;
    {
        hipError_t e = gemm_lds_limits<false>();
        if (e == hipSuccess) e = gemm_lds_limits<true>();
        if (e != hipSuccess)
            return fail(MOE_ERR_DEVICE, "cannot raise the GEMM kernels' LDS limit to %zu bytes: %s",
                        GemmShape<4, 4, 8, true>::Lds, hipGetErrorString(e));
    }
    moe_ffn_t h = new moe_ffn_s();
    h->sh = s;
    auto cleanup = [&](moe_status r) {
        moe_ffn_destroy(h);
        return r;
    };
    if (hipGetDevice(&h->device) != hipSuccess) return cleanup(fail(MOE_ERR_DEVICE, "hipGetDevice failed"));
    {
        // the big GEMMs' tail split assumes workgroups spread round-robin over 8 XCDs of equal size
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, h->device) != hipSuccess)
            return cleanup(fail(MOE_ERR_DEVICE, "hipGetDeviceProperties failed"));
        h->cus_per_xcd = prop.multiProcessorCount % 8 == 0 ? prop.multiProcessorCount / 8 : 0;
    }
    {
        const hipError_t e = scratch_address(h->device, &h->scratch);
        if (e != hipSuccess)
            return cleanup(fail(MOE_ERR_DEVICE, "hipGetSymbolAddress of the no-alloc scratch failed on device %d: %s",
                                h->device, hipGetErrorString(e)));
    }
    const int E = s.num_experts, H = s.hidden_dim, I = s.moe_intermediate;
    if (hipMalloc(&h->gu, 2 * gb) != hipSuccess || hipMalloc(&h->dn, db) != hipSuccess ||
        hipMalloc(&h->rw, (size_t)E * H * 4) != hipSuccess ||
        (router_bias && hipMalloc(&h->rb, (size_t)E * 4) != hipSuccess))
        return cleanup(fail(MOE_ERR_OOM, "weight allocation failed (%zu bytes)", 2 * gb + db));
    hipError_t e = hipMemcpyAsync(h->rw, router_w, (size_t)E * H * 4, hipMemcpyDeviceToDevice, hs);
    if (e == hipSuccess && router_bias) e = hipMemcpyAsync(h->rb, router_bias, (size_t)E * 4, hipMemcpyDeviceToDevice, hs);
    if (e != hipSuccess) return cleanup(fail(MOE_ERR_DEVICE, "router copy failed: %s", hipGetErrorString(e)));
    const int nh = H / kQ4Weights, ni = I / kQ4Weights;
    auto rep = [&](const void *src, uint8_t *dst, int rows, int nsb, int kind) {
        const long total = (long)E * rows * nsb;
        repack_kernel<<<(unsigned)((total + 255) / 256), 256, 0, hs>>>((const uint8_t *)src, dst, E, rows, nsb, kind);
    };
    rep(gate_q4k, h->gu, I, nh, 0);
    rep(up_q4k, h->gu, I, nh, 1);
    rep(down_q4k, h->dn, H, ni, 2);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return cleanup(fail(MOE_ERR_DEVICE, "weight repack failed: %s", hipGetErrorString(e)));
    *out = h;
    return MOE_OK;
}

moe_status moe_ffn_reserve(moe_ffn_t h, int32_t max_tokens, void *stream) {
    g_err.clear();
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (max_tokens < 1) return fail(MOE_ERR_INVALID_SHAPE, "max_tokens must be >= 1 (got %d)", max_tokens);
    return ensure_ws(h, max_tokens, (hipStream_t)stream);
}

moe_status moe_ffn_forward(moe_ffn_t h, int32_t T, const float *x, float *out, float *router_out,
                           int32_t *router_idx, void *stream) {
    g_err.clear();
    moe_status r = check_call(h, T, x, out, router_out, router_idx);
    if (r == MOE_OK) r = ensure_ws(h, T, (hipStream_t)stream);
    if (r != MOE_OK) return r;
    return forward_layer(h, h->ws, h->prof, T, x, out, router_out, router_idx, nullptr, nullptr, 0.0, 0,
                         (hipStream_t)stream);
}

moe_status moe_ffn_forward_noalloc(moe_ffn_t h, int32_t T, const float *x, float *out, float *router_out,
                                   int32_t *router_idx, void *stream) {
    g_err.clear();
    moe_status r = check_call(h, T, x, out, router_out, router_idx);
    if (r != MOE_OK) return r;
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (dev != h->device)
        return fail(MOE_ERR_INVALID_ARG, "the current device (%d) is not the handle's device (%d)", dev, h->device);
    Workspace w;
    const size_t need = layout_ws(h->sh, T, nullptr, &w);
    if (need > kScratchBytes) {
        int tmax = T;
        while (tmax > 1 && layout_ws(h->sh, tmax, nullptr, &w) > kScratchBytes) tmax = tmax * 3 / 4;
        while (layout_ws(h->sh, tmax + 1, nullptr, &w) <= kScratchBytes) ++tmax;
        return fail(MOE_ERR_INVALID_SHAPE,
                    "T = %d needs %zu bytes of scratch; the no-alloc variant has %zu (at most %d tokens of this layer)",
                    T, need, kScratchBytes, layout_ws(h->sh, 1, nullptr, &w) <= kScratchBytes ? tmax : 0);
    }
    layout_ws(h->sh, T, (char *)h->scratch, &w);
    h->scratch_ws = w;
    hipStream_t st = (hipStream_t)stream;
    // the router's completion counters (used by router_kernel, T <= 4 off the
    // decode path) must start at zero: clear them, whatever an earlier call
    // left in the shared scratch
    if (T <= 4 && !decode_path(h->sh, T)) zero_u32_kernel<<<1, 256, 0, st>>>(h->scratch_ws.rcount, T);
    static Profiler no_profile;  // never enabled: no events are created or recorded
    return forward_layer(h, h->scratch_ws, no_profile, T, x, out, router_out, router_idx, nullptr, nullptr, 0.0, 0,
                         st);
}

moe_status moe_ffn_forward_q8(moe_ffn_t h, int32_t T, const float *x, float *out, float *router_out,
                              int32_t *router_idx, void *stream) {
    g_err.clear();
    moe_status r = check_call(h, T, x, out, router_out, router_idx);
    if (r != MOE_OK) return r;
    r = ensure_ws(h, T, (hipStream_t)stream);
    if (r != MOE_OK) return r;
    return forward_layer(h, h->ws, h->prof, T, x, out, router_out, router_idx, nullptr, nullptr, 0.0, 1,
                         (hipStream_t)stream);
}

moe_status moe_ffn_set_norm(moe_ffn_t h, const float *norm_w, float eps, void *stream) {
    g_err.clear();
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (!norm_w) return fail(MOE_ERR_INVALID_ARG, "norm_w must not be NULL");
    if (!(eps >= 0.f) || !(eps < INFINITY)) return fail(MOE_ERR_INVALID_ARG, "eps must be finite and >= 0");
    hipStream_t st = (hipStream_t)stream;
    const size_t bytes = (size_t)h->sh.hidden_dim * 4;
    if (!h->norm_w) {
        void *p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess) {
            (void)hipGetLastError();
            return fail(MOE_ERR_OOM, "could not allocate %zu bytes for the norm weight", bytes);
        }
        h->norm_w = (float *)p;
    }
    HIP_TRY(hipMemcpyAsync(h->norm_w, norm_w, bytes, hipMemcpyDefault, st));
    HIP_TRY(hipStreamSynchronize(st));
    h->norm_eps = eps;
    return MOE_OK;
}

moe_status moe_ffn_forward_block(moe_ffn_t h, int32_t T, const float *hidden, float *out, float *router_out,
                                 int32_t *router_idx, void *stream) {
    g_err.clear();
    moe_status r = check_call(h, T, hidden, out, router_out, router_idx);
    if (r != MOE_OK) return r;
    if (!h->norm_w) return fail(MOE_ERR_INVALID_ARG, "no norm weight on this handle (call moe_ffn_set_norm first)");
    hipStream_t st = (hipStream_t)stream;
    r = ensure_ws(h, T, st);
    if (r != MOE_OK) return r;
    // decode path: the norm is fused into its router launch; general path:
    // into the router and top-k launches (where they can take it)
    if (decode_path(h->sh, T) || fold_norm_general(h->sh, T))
        return forward_layer(h, h->ws, h->prof, T, hidden, out, router_out, router_idx, hidden, h->norm_w,
                             (double)h->norm_eps, 0, st);
    launch(h->prof, kStNorm, rmsnorm_kernel, dim3(T), dim3(256), st, hidden, h->norm_w, h->sh.hidden_dim,
           (double)h->norm_eps, h->ws.xn);
    return forward_layer(h, h->ws, h->prof, T, h->ws.xn, out, router_out, router_idx, hidden, nullptr, 0.0, 0, st);
}

moe_status moe_ffn_debug_routing(moe_ffn_t h, double *logits, int32_t *counts, int32_t *offsets, int32_t *entries,
                                 void *stream) {
    g_err.clear();
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (h->last_T < 1) return fail(MOE_ERR_INVALID_ARG, "no forward has run on this handle");
    if ((logits && !is_device_ptr(logits)) || (counts && !is_device_ptr(counts)) ||
        (offsets && !is_device_ptr(offsets)) || (entries && !is_device_ptr(entries)))
        return fail(MOE_ERR_INVALID_ARG, "debug outputs must be device pointers");
    hipStream_t st = (hipStream_t)stream;
    const size_t T = h->last_T, E = h->sh.num_experts, k = h->sh.num_experts_per_tok;
    const Workspace &w = *h->last_ws;
    if (logits) HIP_TRY(hipMemcpyAsync(logits, w.logits, T * E * 8, hipMemcpyDeviceToDevice, st));
    if (counts) HIP_TRY(hipMemcpyAsync(counts, w.counts, E * 4, hipMemcpyDeviceToDevice, st));
    if (offsets) HIP_TRY(hipMemcpyAsync(offsets, w.offsets, (E + 1) * 4, hipMemcpyDeviceToDevice, st));
    if (entries) HIP_TRY(hipMemcpyAsync(entries, w.entries, T * k * 4, hipMemcpyDeviceToDevice, st));
    return MOE_OK;
}

moe_status moe_ffn_debug_stats(moe_ffn_t h, int32_t token, const float *out, const float *router_out,
                               double *stats, void *stream) {
    g_err.clear();
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (h->last_T < 1) return fail(MOE_ERR_INVALID_ARG, "no forward has run on this handle");
    if (token < 0 || token >= h->last_T)
        return fail(MOE_ERR_INVALID_ARG, "token %d outside the last forward's 0..%d", token, h->last_T - 1);
    if (!is_device_ptr(out) || !is_device_ptr(stats) || (router_out && !is_device_ptr(router_out)))
        return fail(MOE_ERR_INVALID_ARG, "out, stats and router_out must be device pointers");
    const moe_ffn_shape &s = h->sh;
    const Workspace &w = *h->last_ws;
    hipLaunchKernelGGL(stage_stats_kernel, dim3(kStatStages), dim3(256), 0, (hipStream_t)stream, w.logits,
                       router_out ? router_out : w.w, w.h, h->last_decode ? nullptr : w.pos, out,
                       (int)token, s.num_experts, s.num_experts_per_tok, s.moe_intermediate, s.hidden_dim, stats);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
}

moe_status moe_ffn_profile(moe_ffn_t h, uint32_t stage_mask) {
    g_err.clear();
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    h->prof.mask = stage_mask & ((1u << kStCount) - 1u);
    return MOE_OK;
}

moe_status moe_ffn_profile_read(moe_ffn_t h, double *ms, int32_t *launches) {
    g_err.clear();
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (!ms || !launches) return fail(MOE_ERR_INVALID_ARG, "ms and launches must not be NULL");
    Profiler &p = h->prof;
    for (int s = 0; s < kStCount; ++s) {
        for (size_t i = 0; i < p.used[s]; ++i) {
            HIP_TRY(hipEventSynchronize(p.pairs[s][i].second));
            float e = 0.f;
            HIP_TRY(hipEventElapsedTime(&e, p.pairs[s][i].first, p.pairs[s][i].second));
            ms[s] += e;
            launches[s] += 1;
        }
        p.used[s] = 0;
    }
    return MOE_OK;
}

int32_t moe_ffn_stage_count(void) { return kStCount; }

const char *moe_ffn_stage_name(int32_t stage) { return (stage >= 0 && stage < kStCount) ? kStageNames[stage] : nullptr; }

moe_status moe_ffn_destroy(moe_ffn_t h) {
    if (!h) return MOE_OK;
    (void)hipDeviceSynchronize();
    if (h->gu) (void)hipFree(h->gu);
    if (h->dn) (void)hipFree(h->dn);
    if (h->rw) (void)hipFree(h->rw);
    if (h->rb) (void)hipFree(h->rb);
    if (h->norm_w) (void)hipFree(h->norm_w);
    if (h->ws_base) (void)hipFree(h->ws_base);
    delete h;
    return MOE_OK;
}

}  // extern "C"
