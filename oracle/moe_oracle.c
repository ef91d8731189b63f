/*
 * Plain fp64 CPU oracle of the routed-expert MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header, table or constant with the HIP
 * library; both sides read the same seeded inputs and nothing else.
 *
 * What is computed, and where the pages define it (docs.rs source pages of the
 * aprender-serve crate):
 *   - forward_qwen3_moe.rs, decode step 2h (MoE FFN) comment: for one position
 *     the layer returns a hidden_dim vector; each chosen expert applies a SwiGLU
 *     of its gate and up projections followed by its down projection, and the
 *     expert results are summed with router weights that come from a softmax
 *     followed by a renormalisation over the chosen k. The module doc adds that
 *     each chosen expert's matrix-vector products dequantise its Q4_K bytes as
 *     they go.
 *   - forward_qwen3_moe_cuda_traced.rs, doc of ..._traced_with_plan: the
 *     MoeRouter stage holds the k router weights of the last token after that
 *     softmax and renormalisation; MoeFfnOut holds its hidden_dim output.
 *   - forward_qwen3_moe.rs, prefill step 2g: positions are sent through the
 *     layer one at a time, so each token is routed and computed on its own.
 * Readings where the pages are silent (each listed in the design notes):
 *   - Q4_K super-block layout: the public GGUF/ggml Q4_K block (the pages only
 *     name the format, in the Q4_K_M model file name).
 *   - top-k is taken on the logits (softmax is monotone), larger first, exact
 *     ties to the lower expert index; outputs are listed in that order.
 *   - renormalisation: w_j = p_{e_j} / sum_i p_{e_i} over the k selected, with
 *     p the softmax over all experts.
 *   - SiLU is applied to the gate projection, SiLU(z) = z / (1 + exp(-z)).
 *   - matrices are [out][in] row-major, Q4_K blocks along the input dimension.
 *
 * Every floating-point step is done in IEEE double. Inputs (fp32 activations
 * and router weights, fp16 block scales, small integers) are widened exactly,
 * and a dequantised weight d*sc*q - dmin*m is exact in double.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 * Threads only split independent tokens or rows; no result depends on them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MO_Q4K_BYTES 144
#define MO_Q4K_WEIGHTS 256

/* ---------------------------------------------------------------- threads */

int mo_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------- binary16 */

/* IEEE 754 binary16 to double: 1 sign bit, 5 exponent bits (bias 15), 10
 * fraction bits; exponent 0 holds subnormals frac * 2^-24. */
double mo_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(frac + 1024), expo - 25);
    }
    return sign ? -v : v;
}

/* ------------------------------------------------------------------ Q4_K */

/* Fields of one 144-byte Q4_K super-block (public GGUF k-quant format):
 *   bytes 0-1   d     (fp16, little endian)  super-block scale
 *   bytes 2-3   dmin  (fp16)                 super-block min scale
 *   bytes 4-15  twelve bytes holding eight 6-bit scales and eight 6-bit mins
 *   bytes 16-143 128 bytes of 4-bit quants
 * Sub-block j (32 weights) for j < 4: scale = low 6 bits of scale byte j,
 * min = low 6 bits of scale byte j+4. For j >= 4: the low 4 bits come from
 * scale byte j+4 (low nibble for the scale, high nibble for the min) and the
 * top 2 bits from the top 2 bits of scale byte j-4 (scale) or byte j (min).
 * Quants: weight 64c + l (c = 0..3, l = 0..31) is the low nibble of quant byte
 * 32c + l, and weight 64c + 32 + l is the high nibble of the same byte.
 * Weight value = d * scale_j * q - dmin * min_j with j = weight / 32. */
void mo_q4k_fields(const uint8_t *blk, double *d, double *dmin, int32_t sc[8], int32_t mn[8],
                   int32_t q[256]) {
    const uint8_t *s = blk + 4;
    const uint8_t *qs = blk + 16;
    *d = mo_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    *dmin = mo_half_to_double((uint16_t)(blk[2] | (blk[3] << 8)));
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            mn[j] = s[j + 4] & 63;
        } else {
            sc[j] = (s[j + 4] & 0x0f) | ((s[j - 4] >> 6) << 4);
            mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
    }
    for (int c = 0; c < 4; ++c) {
        for (int l = 0; l < 32; ++l) {
            q[64 * c + l] = qs[32 * c + l] & 0x0f;
            q[64 * c + 32 + l] = qs[32 * c + l] >> 4;
        }
    }
}

void mo_q4k_dequant_block(const uint8_t *blk, double out[256]) {
    double d, dmin;
    int32_t sc[8], mn[8], q[256];
    mo_q4k_fields(blk, &d, &dmin, sc, mn, q);
    for (int i = 0; i < 256; ++i) {
        int j = i / 32;
        out[i] = d * (double)sc[j] * (double)q[i] - dmin * (double)mn[j];
    }
}

/* Dequantise a [rows][cols] matrix stored as rows of cols/256 blocks. */
void mo_q4k_dequant_matrix(const uint8_t *blob, int64_t rows, int64_t cols, double *out) {
    int64_t nb = cols / MO_Q4K_WEIGHTS;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            mo_q4k_dequant_block(blob + (r * nb + b) * MO_Q4K_BYTES, out + r * cols + b * MO_Q4K_WEIGHTS);
        }
    }
}

/* ----------------------------------------------------------------- router */

/* logits[t][e] = sum_h W[e][h] * x[t][h] (+ bias[e]), in double. */
void mo_router_logits(int32_t T, int32_t H, int32_t E, const float *x, const float *w,
                      const float *bias, double *logits) {
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; ++h) acc += (double)w[(int64_t)e * H + h] * (double)x[(int64_t)t * H + h];
            if (bias) acc += (double)bias[e];
            logits[(int64_t)t * E + e] = acc;
        }
    }
}

/* k passes of argmax over the experts not yet chosen; a later expert replaces
 * the running best only if its logit is strictly larger, so exact ties go to
 * the lower index. */
void mo_topk(int32_t T, int32_t E, int32_t k, const double *logits, int32_t *idx) {
    for (int32_t t = 0; t < T; ++t) {
        const double *l = logits + (int64_t)t * E;
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int32_t i = 0; i < j; ++i) taken |= (idx[(int64_t)t * k + i] == e);
                if (taken) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            idx[(int64_t)t * k + j] = best;
        }
    }
}

/* Softmax over all E experts (max-subtracted), then the k chosen
 * probabilities divided by their own sum. */
void mo_router_weights(int32_t T, int32_t E, int32_t k, const double *logits, const int32_t *idx,
                       double *wout) {
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    for (int32_t t = 0; t < T; ++t) {
        const double *l = logits + (int64_t)t * E;
        double mx = l[0];
        for (int32_t e = 1; e < E; ++e)
            if (l[e] > mx) mx = l[e];
        double z = 0.0;
        for (int32_t e = 0; e < E; ++e) {
            p[e] = exp(l[e] - mx);
            z += p[e];
        }
        for (int32_t e = 0; e < E; ++e) p[e] /= z;
        double s = 0.0;
        for (int32_t j = 0; j < k; ++j) s += p[idx[(int64_t)t * k + j]];
        for (int32_t j = 0; j < k; ++j) wout[(int64_t)t * k + j] = p[idx[(int64_t)t * k + j]] / s;
    }
    free(p);
}

/* -------------------------------------------------------------- bucketing */

/* Stable counting sort of the T*k (token, slot) pairs by expert:
 * counts[e], offsets[e] = sum of counts below e (offsets[E] = T*k),
 * entries[offsets[e] + r] = t*k + j for the r-th pair (in token order) that
 * chose e, and pos[t*k + j] = its place in entries. */
void mo_bucket(int32_t T, int32_t k, int32_t E, const int32_t *idx, int32_t *counts, int32_t *offsets,
               int32_t *entries, int32_t *pos) {
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t s = 0; s < (int64_t)T * k; ++s) counts[idx[s]] += 1;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = idx[(int64_t)t * k + j];
            int32_t p = offsets[e] + fill[e]++;
            entries[p] = t * k + j;
            pos[(int64_t)t * k + j] = p;
        }
    }
    free(fill);
}

/* ------------------------------------------------------------ expert FFN */

double mo_silu(double z) { return z / (1.0 + exp(-z)); }

/* Q8_K-style activation quantisation (the int8-activation CPU path the
 * dispatch page compares against, qwen3_moe_dispatch.rs; the pages name it
 * without its arithmetic, so this reading is taken): per block of 256 fp32
 * values, amax = max |v|; if amax is 0 then d = 0 and every q = 0, else
 * q = rint(v * (127 / amax)) (round half to even), clamped to [-127, 127], and
 * d = amax / 127, with every step in fp32 (the precision that decides the
 * integer codes). The block then stands for the values d * q. n % 256 == 0. */
void mo_q8k_quantize(int64_t n, const float *v, float *d, int8_t *q) {
    for (int64_t b = 0; b < n / 256; ++b) {
        const float *vb = v + b * 256;
        float amax = 0.0f;
        for (int i = 0; i < 256; ++i) {
            const float a = fabsf(vb[i]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            d[b] = 0.0f;
            for (int i = 0; i < 256; ++i) q[b * 256 + i] = 0;
            continue;
        }
        const float iscale = 127.0f / amax;
        for (int i = 0; i < 256; ++i) {
            float r = rintf(vb[i] * iscale);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[b * 256 + i] = (int8_t)r;
        }
        d[b] = amax / 127.0f;
    }
}

/* x (n fp32 values) replaced by its Q8_K values d * q, in double. */
static int q8k_round_trip(int64_t n, const float *x, double *out) {
    float *d = (float *)malloc(sizeof(float) * (size_t)(n / 256));
    int8_t *q = (int8_t *)malloc((size_t)n);
    if (!d || !q) {
        free(d); free(q);
        return -1;
    }
    mo_q8k_quantize(n, x, d, q);
    for (int64_t i = 0; i < n; ++i) out[i] = (double)d[i / 256] * (double)q[i];
    free(d); free(q);
    return 0;
}

/* One expert on one activation row, with dequantised fp64 matrices
 * Wg, Wu [I][H] and Wd [H][I]:
 *   g = Wg x, u = Wu x, h = SiLU(g) * u, y = Wd h.
 * q8: h enters the down projection as its Q8_K values (h rounded to fp32, then
 * mo_q8k_quantize), as the int8-activation path feeds each matvec. */
static int expert_dense_impl(int32_t H, int32_t I, const double *Wg, const double *Wu, const double *Wd,
                             const double *x, double *y, double *g_out, double *u_out, double *h_out, int q8) {
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    float *hf = q8 ? (float *)malloc(sizeof(float) * (size_t)I) : NULL;
    if (!h || (q8 && !hf)) {
        free(h); free(hf);
        return -1;
    }
    for (int32_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int32_t c = 0; c < H; ++c) {
            g += Wg[(int64_t)i * H + c] * x[c];
            u += Wu[(int64_t)i * H + c] * x[c];
        }
        h[i] = mo_silu(g) * u;
        if (g_out) g_out[i] = g;
        if (u_out) u_out[i] = u;
        if (h_out) h_out[i] = h[i];
    }
    if (q8) {
        for (int32_t i = 0; i < I; ++i) hf[i] = (float)h[i];
        if (q8k_round_trip(I, hf, h) != 0) {
            free(h); free(hf);
            return -1;
        }
    }
    for (int32_t n = 0; n < H; ++n) {
        double acc = 0.0;
        for (int32_t i = 0; i < I; ++i) acc += Wd[(int64_t)n * I + i] * h[i];
        y[n] = acc;
    }
    free(h); free(hf);
    return 0;
}

void mo_expert_dense(int32_t H, int32_t I, const double *Wg, const double *Wu, const double *Wd,
                     const double *x, double *y, double *g_out, double *u_out, double *h_out) {
    (void)expert_dense_impl(H, I, Wg, Wu, Wd, x, y, g_out, u_out, h_out, 0);
}

/* Same, straight from one expert's Q4_K blobs (gate/up [I][H/256] blocks,
 * down [H][I/256] blocks) and an fp32 activation row. */
int mo_expert_q4k(int32_t H, int32_t I, const uint8_t *gate, const uint8_t *up, const uint8_t *down,
                  const float *x, double *y, double *g, double *u, double *h) {
    double *Wg = (double *)malloc(sizeof(double) * (size_t)I * H);
    double *Wu = (double *)malloc(sizeof(double) * (size_t)I * H);
    double *Wd = (double *)malloc(sizeof(double) * (size_t)H * I);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    if (!Wg || !Wu || !Wd || !xd) {
        free(Wg); free(Wu); free(Wd); free(xd);
        return -1;
    }
    mo_q4k_dequant_matrix(gate, I, H, Wg);
    mo_q4k_dequant_matrix(up, I, H, Wu);
    mo_q4k_dequant_matrix(down, H, I, Wd);
    for (int32_t c = 0; c < H; ++c) xd[c] = (double)x[c];
    mo_expert_dense(H, I, Wg, Wu, Wd, xd, y, g, u, h);
    free(Wg); free(Wu); free(Wd); free(xd);
    return 0;
}

/* ---------------------------------------------------------------- forward */

/* The whole layer for T tokens.
 *   x [T][H] fp32, router_w [E][H] fp32, bias [E] fp32 or NULL,
 *   gate, up [E][I][H/256][144], down [E][H][I/256][144] bytes.
 * Router (logits, top-k, weights) runs for all T tokens. The expert part runs
 * for the n_sel tokens listed in sel (all tokens if sel is NULL) and writes
 * out[n_sel][H] in the order of sel.
 * If idx_in is given it replaces the top-k choice (the weights are still the
 * renormalised softmax at those experts); idx_out/w_out/logits_out may be
 * NULL. Returns 0, or -1 on allocation failure / bad arguments. */
static int forward_impl(int32_t H, int32_t E, int32_t k, int32_t I, int32_t T, const float *x,
                        const float *router_w, const float *bias, const uint8_t *gate, const uint8_t *up,
                        const uint8_t *down, const int32_t *sel, int32_t n_sel, const int32_t *idx_in, double *out,
                        int32_t *idx_out, double *w_out, double *logits_out, int q8) {
    if (H <= 0 || E <= 0 || k <= 0 || k > E || I <= 0 || T <= 0 || H % 256 || I % 256) return -1;
    int64_t nsel = sel ? n_sel : T;
    double *logits = (double *)malloc(sizeof(double) * (size_t)T * E);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * k);
    double *w = (double *)malloc(sizeof(double) * (size_t)T * k);
    double *Y = (double *)malloc(sizeof(double) * (size_t)nsel * k * H);
    double *Wg = (double *)malloc(sizeof(double) * (size_t)I * H);
    double *Wu = (double *)malloc(sizeof(double) * (size_t)I * H);
    double *Wd = (double *)malloc(sizeof(double) * (size_t)H * I);
    int rc = 0;
    if (!logits || !idx || !w || !Y || !Wg || !Wu || !Wd) {
        rc = -1;
        goto done;
    }
    mo_router_logits(T, H, E, x, router_w, bias, logits);
    if (idx_in) {
        memcpy(idx, idx_in, sizeof(int32_t) * (size_t)T * k);
        for (int64_t s = 0; s < (int64_t)T * k; ++s)
            if (idx[s] < 0 || idx[s] >= E) { rc = -1; goto done; }
    } else {
        mo_topk(T, E, k, logits, idx);
    }
    mo_router_weights(T, E, k, logits, idx, w);

    const int64_t nbh = H / 256, nbi = I / 256;
    const int64_t gate_stride = (int64_t)I * nbh * 144, down_stride = (int64_t)H * nbi * 144;
    /* Expert by expert: dequantise its three matrices once, then run every
     * selected (token, slot) pair that chose it. */
    for (int32_t e = 0; e < E; ++e) {
        int used = 0;
        for (int64_t s = 0; s < nsel && !used; ++s) {
            int32_t t = sel ? sel[s] : (int32_t)s;
            for (int32_t j = 0; j < k; ++j) used |= (idx[(int64_t)t * k + j] == e);
        }
        if (!used) continue;
        mo_q4k_dequant_matrix(gate + e * gate_stride, I, H, Wg);
        mo_q4k_dequant_matrix(up + e * gate_stride, I, H, Wu);
        mo_q4k_dequant_matrix(down + e * down_stride, H, I, Wd);
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t s = 0; s < nsel; ++s) {
            int32_t t = sel ? sel[s] : (int32_t)s;
            for (int32_t j = 0; j < k; ++j) {
                if (idx[(int64_t)t * k + j] != e) continue;
                double *xd = (double *)malloc(sizeof(double) * (size_t)H);
                int bad = !xd;
                if (!bad && q8) {
                    bad = q8k_round_trip(H, x + (int64_t)t * H, xd) != 0;
                } else if (!bad) {
                    for (int32_t c = 0; c < H; ++c) xd[c] = (double)x[(int64_t)t * H + c];
                }
                if (!bad) bad = expert_dense_impl(H, I, Wg, Wu, Wd, xd, Y + (s * k + j) * H, NULL, NULL, NULL, q8);
                if (bad) {
#pragma omp atomic write
                    rc = -1;
                }
                free(xd);
            }
        }
    }
    /* Router-weighted sum over the k slots, slot 0 first. */
    for (int64_t s = 0; s < nsel; ++s) {
        int32_t t = sel ? sel[s] : (int32_t)s;
        for (int32_t n = 0; n < H; ++n) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) acc += w[(int64_t)t * k + j] * Y[(s * k + j) * H + n];
            out[s * H + n] = acc;
        }
    }
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)T * k);
    if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)T * k);
    if (logits_out) memcpy(logits_out, logits, sizeof(double) * (size_t)T * E);
done:
    free(logits); free(idx); free(w); free(Y); free(Wg); free(Wu); free(Wd);
    return rc;
}

/* ------------------------------------------------- the block around the layer */

/* Pre-FFN norm (forward_qwen3_moe.rs: prefill step 2f and decode step 2g,
 * "Pre-FFN norm"): the block normalises the residual stream with the layer's
 * ffn norm weight and the model's eps before the MoE layer. The pages call the
 * op (rms_norm) without writing out its formula; the standard RMSNorm is taken:
 *   y[t][i] = x[t][i] * g[i] / sqrt((1/H) * sum_c x[t][c]^2 + eps). */
void mo_rms_norm(int32_t T, int32_t H, const float *x, const float *g, double eps, double *y) {
    for (int64_t t = 0; t < T; ++t) {
        const float *row = x + t * H;
        double ss = 0.0;
        for (int32_t c = 0; c < H; ++c) ss += (double)row[c] * (double)row[c];
        const double rms = sqrt(ss / (double)H + eps);
        for (int32_t c = 0; c < H; ++c) y[t * H + c] = (double)row[c] * (double)g[c] / rms;
    }
}

/* Residual after the layer (forward_qwen3_moe.rs: the "Residual" step after
 * prefill step 2g, decode step 2i): the layer's output is added to the
 * residual stream it was computed from, out = hidden + ffn. */
void mo_add_residual(int64_t n, const float *hidden, const double *ffn, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (double)hidden[i] + ffn[i];
}

/* ------------------------------------------------------ per-stage statistics */

/* Statistics of one stage's values, the traced forward's per-stage summary
 * (forward_qwen3_moe_cuda_traced.rs: per-layer activation statistics of the
 * last token, used to find the first stage where a NaN or Inf enters; the page
 * names the statistics type but not its fields). Fields taken:
 *   s[0] number of values, s[1] NaN count, s[2] +-Inf count, and over the
 *   finite values only: s[3] min, s[4] max, s[5] mean, s[6] root mean square
 *   (all four 0 when no value is finite). */
void mo_stage_stats(int64_t n, const double *v, double s[7]) {
    int64_t nan = 0, inf = 0, fin = 0;
    double mn = 0.0, mx = 0.0, sum = 0.0, sq = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double x = v[i];
        if (x != x) {
            ++nan;
        } else if (x == INFINITY || x == -INFINITY) {
            ++inf;
        } else {
            if (fin == 0 || x < mn) mn = x;
            if (fin == 0 || x > mx) mx = x;
            sum += x;
            sq += x * x;
            ++fin;
        }
    }
    s[0] = (double)n;
    s[1] = (double)nan;
    s[2] = (double)inf;
    s[3] = mn;
    s[4] = mx;
    s[5] = fin ? sum / (double)fin : 0.0;
    s[6] = fin ? sqrt(sq / (double)fin) : 0.0;
}

/* The layer (described above). */
int mo_forward(int32_t H, int32_t E, int32_t k, int32_t I, int32_t T, const float *x, const float *router_w,
               const float *bias, const uint8_t *gate, const uint8_t *up, const uint8_t *down,
               const int32_t *sel, int32_t n_sel, const int32_t *idx_in, double *out, int32_t *idx_out,
               double *w_out, double *logits_out) {
    return forward_impl(H, E, k, I, T, x, router_w, bias, gate, up, down, sel, n_sel, idx_in, out, idx_out, w_out,
                        logits_out, 0);
}

/* The layer (arguments as mo_forward) with the routed experts' matvecs fed
 * Q8_K-quantised activations: each token's x row, and each expert's h, enter
 * as their mo_q8k_quantize values; the router runs on the fp32 x. */
int mo_forward_q8(int32_t H, int32_t E, int32_t k, int32_t I, int32_t T, const float *x, const float *router_w,
                  const float *bias, const uint8_t *gate, const uint8_t *up, const uint8_t *down,
                  const int32_t *sel, int32_t n_sel, const int32_t *idx_in, double *out, int32_t *idx_out,
                  double *w_out, double *logits_out) {
    return forward_impl(H, E, k, I, T, x, router_w, bias, gate, up, down, sel, n_sel, idx_in, out, idx_out, w_out,
                        logits_out, 1);
}
