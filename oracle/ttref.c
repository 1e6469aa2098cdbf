/*
 * ttref -- the plain fp64 CPU oracle for one block-wise diffusion decoding step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header or constant with the HIP library; it decodes its own
 * inputs and follows the method's plain definition, in double precision, with no
 * tiling, no online softmax and no reordering beyond what the definition states.
 *
 * Sources (page title, then section):
 *   [GS]  "Nemotron-TwoTower: Diffusion Language Modeling with Pretrained Autoregressive
 *          Context" (gist.science explainer, English), Technical Summary.
 *   [SN]  snilld.dk, "NVIDIA aabner for hoej-throughput tekstgenerering med TwoTower
 *          diffusion over en frossen autoregressiv rygrad".
 *
 * Inputs are bf16 bit patterns (uint16) or fp32; every element is widened exactly to
 * double before any arithmetic.
 *
 * Readings where the pages are silent (each listed with its reason in the design notes):
 *   - one softmax spans the context keys and the block keys together;
 *   - no mask inside the block, every valid context key is visible to every block query;
 *   - no positional term, bias or softcap inside the attention; scale 1/sqrt(D);
 *   - KV head of query head h is floor(h / (Hq/Hkv));
 *   - confidence = largest softmax probability of the position's full-vocabulary
 *     distribution at temperature 1; the token is the lowest index attaining the max;
 *   - "above the threshold" is strict (conf > gamma);
 *   - if a sequence has masked positions but none clears gamma, its single most
 *     confident masked position is committed (ties: lowest position);
 *   - the denoiser's Mamba-2 scan is the Mamba-2 selective state-space recurrence (the
 *     pages name the layer type, not its equations), causal, started from the state seeded
 *     by the context tower;
 *   - adaLN is layer normalization without affine terms followed by (1 + scale) and shift,
 *     and a gated residual, with each layer's vectors the sum of one shared set per
 *     sequence (from the timestep) and the layer's own learned offsets ("adaLN-single").
 *
 * Parity pins: every function here is checked against library routines, closed forms
 * and invariants by the CPU test suite; no function is left unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TTREF_F32 0
#define TTREF_BF16 1
#define TTREF_F64 2 /* internal: logits the oracle computed itself */

#define TTREF_OK 0
#define TTREF_EINVAL 1
#define TTREF_ENOMEM 2

/* Exact widening of one element to double. */
static double ttref_load(const void *base, size_t idx, int dtype)
{
    if (dtype == TTREF_F32)
        return (double)((const float *)base)[idx];
    if (dtype == TTREF_F64)
        return ((const double *)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Number of host threads the oracle's parallel loops use (reported with its timings). */
int ttref_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Exported so that the tests can pin the decode itself against a library conversion. */
double ttref_decode(const void *base, size_t idx, int dtype)
{
    return ttref_load(base, idx, dtype);
}

/*
 * Denoiser block attention of one attention layer ([GS] Methodology > Architecture, and
 * Generation Process): each of the S block queries of sequence b and query head h attends,
 * in one softmax, to the context tower's same-layer keys K_ctx[b, 0:ctx_len[b], g] (past
 * blocks) followed by the block's own keys K_blk[b, 0:S, g] (bidirectional, unmasked).
 *
 *   s_j = (q . k_j) / sqrt(D)
 *   p_j = exp(s_j - max_k s_k) / sum_k exp(s_k - max_k s_k)
 *   out[b,i,h,:] = sum_j p_j v_j
 *
 * Layouts: q[B,S,Hq,D], k_blk/v_blk[B,S,Hkv,D], k_ctx/v_ctx[B,Lmax,Hkv,D], out[B,S,Hq,D]
 * (double). Context rows at or beyond ctx_len[b] are never read.
 */
int ttref_block_denoise_attn(int B, int S, int Hq, int Hkv, int D, int Lmax, int dtype,
                             const void *q, const void *k_blk, const void *v_blk,
                             const void *k_ctx, const void *v_ctx, const int32_t *ctx_len,
                             double *out)
{
    if (B < 0 || S < 1 || Hq < 1 || Hkv < 1 || D < 1 || Lmax < 0 || Hq % Hkv != 0)
        return TTREF_EINVAL;
    if (dtype != TTREF_F32 && dtype != TTREF_BF16)
        return TTREF_EINVAL;
    for (int b = 0; b < B; ++b)
        if (ctx_len[b] < 0 || ctx_len[b] > Lmax)
            return TTREF_EINVAL;
    const int G = Hq / Hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    int failed = 0;

#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < S; ++i)
            for (int h = 0; h < Hq; ++h) {
                const int g = h / G;
                const int nctx = ctx_len[b];
                const int n = nctx + S;
                double *s = (double *)malloc((size_t)n * sizeof(double));
                double *qv = (double *)malloc((size_t)D * sizeof(double));
                if (!s || !qv) {
                    free(s);
                    free(qv);
#pragma omp atomic write
                    failed = 1;
                    continue;
                }
                const size_t qoff = (((size_t)b * S + i) * Hq + h) * D;
                for (int d = 0; d < D; ++d)
                    qv[d] = ttref_load(q, qoff + d, dtype);
                /* scores over [context keys ; block keys] */
                for (int j = 0; j < n; ++j) {
                    const void *kbase;
                    size_t koff;
                    if (j < nctx) {
                        kbase = k_ctx;
                        koff = (((size_t)b * Lmax + j) * Hkv + g) * D;
                    } else {
                        kbase = k_blk;
                        koff = (((size_t)b * S + (j - nctx)) * Hkv + g) * D;
                    }
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += qv[d] * ttref_load(kbase, koff + d, dtype);
                    s[j] = dot * inv_sqrt_d;
                }
                /* softmax over all n keys */
                double mx = s[0];
                for (int j = 1; j < n; ++j)
                    if (s[j] > mx)
                        mx = s[j];
                double z = 0.0;
                for (int j = 0; j < n; ++j) {
                    s[j] = exp(s[j] - mx);
                    z += s[j];
                }
                for (int j = 0; j < n; ++j)
                    s[j] /= z;
                /* probability-weighted sum of the values */
                double *o = out + qoff;
                for (int d = 0; d < D; ++d)
                    o[d] = 0.0;
                for (int j = 0; j < n; ++j) {
                    const void *vbase;
                    size_t voff;
                    if (j < nctx) {
                        vbase = v_ctx;
                        voff = (((size_t)b * Lmax + j) * Hkv + g) * D;
                    } else {
                        vbase = v_blk;
                        voff = (((size_t)b * S + (j - nctx)) * Hkv + g) * D;
                    }
                    for (int d = 0; d < D; ++d)
                        o[d] += s[j] * ttref_load(vbase, voff + d, dtype);
                }
                free(s);
                free(qv);
            }
    return failed ? TTREF_ENOMEM : TTREF_OK;
}

/*
 * Confidence unmasking of one denoising step ([GS] Training and Conditioning > Sampling;
 * [SN] Blockwise generering i praksis): every still-masked position gets its greedy token
 * and a confidence; positions whose confidence is above gamma are committed, the rest stay
 * masked.
 *
 * For each masked (b,i), over the full vocabulary row l[0:V]:
 *   M = max_v l_v;   token = lowest v with l_v == M;   Z = sum_v exp(l_v - M);
 *   conf = 1 / Z   (the largest softmax probability);   committed = (conf > gamma).
 * If sequence b has masked positions and none is committed, the masked position with the
 * largest conf (lowest i on ties) is committed.
 * Unmasked positions: token = -1, committed = 0, conf = 0, Z = 0. Their rows are not read.
 * Outputs token_id[B,S] int32, committed[B,S] uint8; conf and Z ([B,S] double) may be NULL.
 */
static void ttref_commit_rows(int B, int S, int V, int dtype, const void *logits,
                              const uint8_t *mask, double gamma, int32_t *token_id,
                              uint8_t *committed, double *conf_out, double *z_out)
{
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        int any_masked = 0, any_committed = 0;
        int best_i = -1;
        double best_conf = -1.0;
        for (int i = 0; i < S; ++i) {
            const size_t r = (size_t)b * S + i;
            if (!mask[r]) {
                token_id[r] = -1;
                committed[r] = 0;
                if (conf_out)
                    conf_out[r] = 0.0;
                if (z_out)
                    z_out[r] = 0.0;
                continue;
            }
            any_masked = 1;
            const size_t off = r * (size_t)V;
            double m = ttref_load(logits, off, dtype);
            int tok = 0;
            for (int v = 1; v < V; ++v) {
                const double x = ttref_load(logits, off + v, dtype);
                if (x > m) {
                    m = x;
                    tok = v;
                }
            }
            double z = 0.0;
            for (int v = 0; v < V; ++v)
                z += exp(ttref_load(logits, off + v, dtype) - m);
            const double conf = 1.0 / z;
            token_id[r] = tok;
            committed[r] = (uint8_t)(conf > gamma);
            any_committed |= committed[r];
            if (conf_out)
                conf_out[r] = conf;
            if (z_out)
                z_out[r] = z;
            if (conf > best_conf) {
                best_conf = conf;
                best_i = i;
            }
        }
        if (any_masked && !any_committed)
            committed[(size_t)b * S + best_i] = 1;
    }
}

int ttref_commit(int B, int S, int V, int dtype, const void *logits, const uint8_t *mask,
                 double gamma, int32_t *token_id, uint8_t *committed, double *conf_out,
                 double *z_out)
{
    if (B < 0 || S < 1 || V < 1 || isnan(gamma))
        return TTREF_EINVAL;
    if (dtype != TTREF_F32 && dtype != TTREF_BF16)
        return TTREF_EINVAL;
    ttref_commit_rows(B, S, V, dtype, logits, mask, gamma, token_id, committed, conf_out, z_out);
    return TTREF_OK;
}

/*
 * The LM head followed by confidence unmasking ([GS] Training and Conditioning > Sampling:
 * all masked tokens are predicted at once from the denoiser's output; [SN] Blockwise
 * generering i praksis). The step's logits are the LM head's output for the hidden state
 * h[b,i,0:K] of every still-masked position (K = d_model) and the head's weight rows
 * w[v,0:K] (vocabulary-major, as the head's [V, K] matrix):
 *   l[b,i,v] = sum_k h[b,i,k] * w[v,k]
 * Each product of two bf16 values is exact in double and the sum runs over k in ascending
 * order in double. The commit rule of ttref_commit is then applied to these logits.
 * Hidden rows of unmasked positions are not read. Inputs are bf16 bit patterns.
 */
int ttref_lmhead_commit(int B, int S, int K, int V, const uint16_t *hidden,
                        const uint16_t *weight, const uint8_t *mask, double gamma,
                        int32_t *token_id, uint8_t *committed, double *conf_out, double *z_out)
{
    if (B < 0 || S < 1 || K < 1 || V < 1 || isnan(gamma))
        return TTREF_EINVAL;
    double *lg = (double *)malloc((size_t)S * V * sizeof(double));
    if (!lg)
        return TTREF_ENOMEM;
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < S; ++i) {
            const size_t r = (size_t)b * S + i;
            if (!mask[r])
                continue;
            const size_t hoff = r * (size_t)K;
#pragma omp parallel for schedule(static)
            for (int v = 0; v < V; ++v) {
                const size_t woff = (size_t)v * K;
                double dot = 0.0;
                for (int k = 0; k < K; ++k)
                    dot += ttref_load(hidden, hoff + k, TTREF_BF16) *
                           ttref_load(weight, woff + k, TTREF_BF16);
                lg[(size_t)i * V + v] = dot;
            }
        }
        ttref_commit_rows(1, S, V, TTREF_F64, lg, mask + (size_t)b * S, gamma,
                          token_id + (size_t)b * S, committed + (size_t)b * S,
                          conf_out ? conf_out + (size_t)b * S : NULL,
                          z_out ? z_out + (size_t)b * S : NULL);
    }
    free(lg);
    return TTREF_OK;
}

/*
 * The context cache update after a block is committed ([GS] Generation Process: once a
 * block is committed, the context tower updates its states with the new clean tokens;
 * [SN] "Blockwise generering i praksis": the context tower then updates its caches and
 * Mamba states, once per block). For one attention layer the block's new key and value
 * rows k_new, v_new [B,S,Hkv,D] are written at positions ctx_len[b] .. ctx_len[b]+S-1 of
 * that layer's cache k_ctx, v_ctx [B,Lmax,Hkv,D]; with bump != 0, ctx_len[b] then grows by
 * S (the last layer's call of a step bumps). A sequence whose block does not fit
 * (ctx_len[b] < 0 or ctx_len[b] + S > Lmax) is left as it is and gets skipped[b] = 1
 * (else 0). Element bits are copied unchanged: no arithmetic.
 */
int ttref_ctx_append(int B, int S, int Hkv, int D, int Lmax, int dtype, const void *k_new,
                     const void *v_new, void *k_ctx, void *v_ctx, int32_t *ctx_len, int bump,
                     uint8_t *skipped)
{
    if (B < 0 || S < 1 || Hkv < 1 || D < 1 || Lmax < 0)
        return TTREF_EINVAL;
    if (dtype != TTREF_F32 && dtype != TTREF_BF16)
        return TTREF_EINVAL;
    const size_t elt = dtype == TTREF_F32 ? 4 : 2;
    const size_t row = (size_t)Hkv * D * elt; /* bytes of one position, all KV heads */
    for (int b = 0; b < B; ++b) {
        const int n = ctx_len[b];
        if (n < 0 || (long long)n + S > Lmax) {
            skipped[b] = 1;
            continue;
        }
        skipped[b] = 0;
        for (int i = 0; i < S; ++i) {
            const size_t src = ((size_t)b * S + i) * row;
            const size_t dst = ((size_t)b * Lmax + n + i) * row;
            memcpy((char *)k_ctx + dst, (const char *)k_new + src, row);
            memcpy((char *)v_ctx + dst, (const char *)v_new + src, row);
        }
        if (bump)
            ctx_len[b] = n + S;
    }
    return TTREF_OK;
}

/*
 * Mamba-2 layer of the denoiser over one block, started from the seeded state ([SN] "Hvad
 * TwoTower aendrer teknisk": the denoiser's Mamba-2 states are seeded directly from the
 * context tower; [GS] Methodology > Architecture: the context tower produces the KV caches and
 * Mamba states; [GS] ablations: the final design keeps Mamba causal). The scan is the Mamba-2
 * selective state-space recurrence, per sequence b and head h (H heads of width P, state
 * width N, G groups of heads sharing B and C, group of head h = h / (H/G)):
 *
 *   delta_t = softplus(dt[b,t,h] + dt_bias[h]),   A_h = -exp(A_log[h]),   a_t = exp(delta_t A_h)
 *   state_t[p][n] = a_t state_{t-1}[p][n] + delta_t x[b,t,h,p] B[b,t,g,n]
 *   y[b,t,h,p]   = sum_n state_t[p][n] C[b,t,g,n] + D[h] x[b,t,h,p]
 *
 * for t = 0..S-1 in order, from state_{-1} = h0[b,h] (the seeded state). The state after the
 * block goes to h_out when it is given (the context tower's own state update over a committed
 * block is the same recurrence). x, B, C are bf16 bits or fp32 (dtype); dt, dt_bias, A_log,
 * D and the states are fp32; y and h_out are double. softplus(z) = log(1 + e^z).
 * Layouts: x, y [B,S,H,P]; dt [B,S,H]; B, C [B,S,G,N]; h0, h_out [B,H,P,N].
 */
static double ttref_softplus(double z)
{
    return z > 30.0 ? z : log1p(exp(z));
}

int ttref_mamba2_scan(int B, int S, int H, int P, int N, int G, int dtype, const void *x,
                      const float *dt, const float *dt_bias, const float *A_log, const float *Dskip,
                      const void *Bm, const void *Cm, const float *h0, double *y, double *h_out)
{
    if (B < 0 || S < 1 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0)
        return TTREF_EINVAL;
    if (dtype != TTREF_F32 && dtype != TTREF_BF16)
        return TTREF_EINVAL;
    const int hpg = H / G;
    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const int g = h / hpg;
            double *st = (double *)malloc((size_t)P * N * sizeof(double));
            if (!st) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            const size_t soff = ((size_t)b * H + h) * P * N;
            for (size_t k = 0; k < (size_t)P * N; ++k)
                st[k] = (double)h0[soff + k];
            const double A = -exp((double)A_log[h]);
            for (int t = 0; t < S; ++t) {
                const double delta = ttref_softplus((double)dt[((size_t)b * S + t) * H + h] + (double)dt_bias[h]);
                const double a = exp(delta * A);
                const size_t xoff = (((size_t)b * S + t) * H + h) * P;
                const size_t boff = (((size_t)b * S + t) * G + g) * N;
                for (int p = 0; p < P; ++p) {
                    const double xp = ttref_load(x, xoff + p, dtype);
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n) {
                        double *s = st + (size_t)p * N + n;
                        *s = a * *s + delta * xp * ttref_load(Bm, boff + n, dtype);
                        acc += *s * ttref_load(Cm, boff + n, dtype);
                    }
                    y[xoff + p] = acc + (double)Dskip[h] * xp;
                }
            }
            if (h_out)
                for (size_t k = 0; k < (size_t)P * N; ++k)
                    h_out[soff + k] = st[k];
            free(st);
        }
    return failed ? TTREF_ENOMEM : TTREF_OK;
}

/*
 * adaLN-single time modulation of one denoiser layer ([GS] Training and Conditioning > Time
 * Conditioning: the denoiser is conditioned on the diffusion timestep t through adaptive
 * layer normalization; [SN] "Hvad TwoTower aendrer teknisk": every layer is time-modulated by
 * a small adaLN-single block). The single block maps a sequence's timestep to one set of
 * modulation vectors t_mod[b] = (shift, scale, gate), shared by all layers; each layer adds
 * its own learned offsets table = (shift, scale, gate). For a row x[b,i,0:d]:
 *
 *   u = (x - mean(x)) / sqrt(var(x) + eps)         (layer normalization, no affine terms;
 *                                                   var is the mean of squared deviations)
 *   y = u * (1 + scale) + shift                     (adaln_modulate, before the layer's mixer)
 *   out = x + gate * f                              (adaln_gate: the mixer's output f joins
 *                                                    the residual stream)
 *
 * with shift = t_mod[b,0,:] + table[0,:], scale = t_mod[b,1,:] + table[1,:], gate =
 * t_mod[b,2,:] + table[2,:]. x and f are bf16 bits or fp32 (dtype); t_mod [B,3,d] and table
 * [3,d] fp32; y and out double [B,S,d].
 */
int ttref_adaln_modulate(int B, int S, int d, int dtype, const void *x, const float *t_mod,
                         const float *table, double eps, double *y)
{
    if (B < 0 || S < 1 || d < 1 || !(eps >= 0.0))
        return TTREF_EINVAL;
    if (dtype != TTREF_F32 && dtype != TTREF_BF16)
        return TTREF_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < S; ++i) {
            const size_t off = ((size_t)b * S + i) * d;
            double mean = 0.0;
            for (int k = 0; k < d; ++k)
                mean += ttref_load(x, off + k, dtype);
            mean /= d;
            double var = 0.0;
            for (int k = 0; k < d; ++k) {
                const double e = ttref_load(x, off + k, dtype) - mean;
                var += e * e;
            }
            var /= d;
            const double rstd = 1.0 / sqrt(var + eps);
            const float *tm = t_mod + (size_t)b * 3 * d;
            for (int k = 0; k < d; ++k) {
                const double shift = (double)tm[k] + (double)table[k];
                const double scale = (double)tm[d + k] + (double)table[d + k];
                const double u = (ttref_load(x, off + k, dtype) - mean) * rstd;
                y[off + k] = u * (1.0 + scale) + shift;
            }
        }
    return TTREF_OK;
}

int ttref_adaln_gate(int B, int S, int d, int dtype, const void *x, const void *f,
                     const float *t_mod, const float *table, double *out)
{
    if (B < 0 || S < 1 || d < 1)
        return TTREF_EINVAL;
    if (dtype != TTREF_F32 && dtype != TTREF_BF16)
        return TTREF_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < S; ++i) {
            const size_t off = ((size_t)b * S + i) * d;
            const float *tm = t_mod + (size_t)b * 3 * d;
            for (int k = 0; k < d; ++k) {
                const double gate = (double)tm[2 * d + k] + (double)table[2 * d + k];
                out[off + k] = ttref_load(x, off + k, dtype) + gate * ttref_load(f, off + k, dtype);
            }
        }
    return TTREF_OK;
}
