/*
 * libtt -- the hot path of one block-wise diffusion decoding step, for AMD Instinct MI355X
 * (gfx950): the denoiser's block attention over its own block KV plus the frozen context
 * tower's same-layer KV, the confidence-threshold (gamma) commit (on given logits, or fused
 * behind the LM head), the context cache update once a block is committed, and the
 * denoiser's Mamba-2 scan from the seeded state and adaLN-single time modulation.
 *
 * Method source: "Nemotron-TwoTower: Diffusion Language Modeling with Pretrained
 * Autoregressive Context" (gist.science explainer, English), Technical Summary; and the
 * snilld.dk article on TwoTower (sections "Hvad TwoTower aendrer teknisk" and "Blockwise
 * generering i praksis").
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers to caller-owned, contiguous, row-major memory
 *     (last index fastest). The library keeps no pointer after a call returns.
 *   - Calls are asynchronous on the given stream (a hipStream_t; NULL = the default stream).
 *     Host-side validation runs before any launch and never synchronizes. Kernel execution
 *     errors surface at the caller's next synchronization.
 *   - The library allocates no device memory. Scratch space comes from the caller as a
 *     workspace whose minimum size the matching *_workspace() query returns; its contents
 *     on entry are irrelevant, and a workspace must not be shared by calls that may run
 *     concurrently.
 *   - Outputs must not alias inputs or the workspace.
 *   - Element types: TT_F32 is IEEE binary32; TT_BF16 is bfloat16 (the upper 16 bits of a
 *     binary32), passed as 16-bit words.
 */
#ifndef TT_H
#define TT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TT_OK = 0,
    TT_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size, NaN gamma    */
    TT_ERR_UNSUPPORTED = 2, /* a size or dtype outside the supported set listed below    */
    TT_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than the query returned */
    TT_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed                */
} tt_status;

typedef enum { TT_F32 = 0, TT_BF16 = 1 } tt_dtype;

/* Shape of one attention call. B sequences, S block positions, Hq query heads sharing
 * Hkv KV heads (Hq % Hkv == 0; query head h reads KV head h / (Hq/Hkv)), head dim D,
 * and Lmax rows of context KV storage per sequence. */
typedef struct {
    int32_t B, S, Hq, Hkv, D, Lmax;
    int32_t dtype; /* tt_dtype */
} tt_attn_shape;

/* Library version, (major << 16) | minor. */
int32_t tt_version(void);

/* Build identity: the first 16 hex digits of the SHA-256 of the sources this library was
 * compiled from (static string, never NULL). A binding compares it with the sources beside
 * it and refuses a stale library. */
const char *tt_build_id(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *tt_status_str(tt_status s);

/* ---------------------------------------------------------------------------------------
 * tt_block_denoise_attn -- denoiser block attention of one attention layer.
 *
 * Defined by Nemotron-TwoTower (gist.science explainer), Technical Summary > Methodology >
 * Architecture (bidirectional attention inside the noisy block, cross-attention to the
 * same layer of the frozen context tower) and > Generation Process (at each layer the
 * denoiser attends to the context tower's KV cache of past blocks and to its own KV cache
 * of the current block). One softmax spans both key sets:
 *
 *   keys(b, g)   = [ k_ctx[b, 0:ctx_len[b], g, :] ; k_blk[b, 0:S, g, :] ]   (same for values)
 *   o[b,i,h,:]   = softmax_j( q[b,i,h,:] . keys_j / sqrt(D) ) @ values,   g = h / (Hq/Hkv)
 *
 * No mask inside the block, no positional term, no bias. Accumulation is fp32; the output
 * has the input dtype (bf16 rounded to nearest even).
 *
 *   q        [B, S, Hq, D]      dtype                   (device, read)
 *   k_blk    [B, S, Hkv, D]     dtype                   (device, read)
 *   v_blk    [B, S, Hkv, D]     dtype                   (device, read)
 *   k_ctx    [B, Lmax, Hkv, D]  dtype                   (device, read)
 *   v_ctx    [B, Lmax, Hkv, D]  dtype                   (device, read)
 *   ctx_len  [B]                int32, 0 <= ctx_len[b] <= Lmax   (device, read)
 *   o        [B, S, Hq, D]      dtype                   (device, written)
 * Context rows at or beyond ctx_len[b] are never read and may hold anything (NaN included).
 * ctx_len lives on the device, so the host cannot check it; the kernels clamp each value
 * into [0, Lmax] before use (a value outside that range is a caller error, not a fault).
 *
 * Supported: dtype TT_BF16 or TT_F32; 1 <= D <= 256; 1 <= S <= 1024; B*S*Hq*D,
 * B*Lmax*Hkv*D < 2^31; B <= 8191. Anything else returns TT_ERR_UNSUPPORTED. B == 0 is a
 * no-op. k_ctx/v_ctx may be NULL only when Lmax == 0. Tensors need only their element
 * alignment: bf16 with D == 128 takes the MFMA path when q, k_blk, v_blk, k_ctx, v_ctx and
 * o all start on a 16-byte boundary (16-byte copies), and the element-wise path otherwise.
 * ------------------------------------------------------------------------------------- */
size_t tt_block_denoise_attn_workspace(const tt_attn_shape *shape);

tt_status tt_block_denoise_attn(const tt_attn_shape *shape, const void *q, const void *k_blk,
                                const void *v_blk, const void *k_ctx, const void *v_ctx,
                                const int32_t *ctx_len, void *o, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * tt_commit -- confidence unmasking of one denoising step.
 *
 * Defined by Nemotron-TwoTower (gist.science explainer), Technical Summary > Training and
 * Conditioning > Sampling (all masked tokens are predicted at once; those whose confidence
 * is above gamma are committed, the rest stay masked) and the snilld.dk TwoTower article,
 * "Blockwise generering i praksis" (a lower gamma commits more tokens per step).
 *
 * For every masked position (b,i) over its full vocabulary row l[0:V]:
 *   token = lowest v with l_v == max l;  Z = sum_v exp(l_v - max l);  conf = 1/Z;
 *   committed = conf > gamma   (strict).
 * If sequence b has masked positions and none is committed, its masked position with the
 * largest conf (lowest i on ties) is committed. Unmasked positions: token -1, committed 0,
 * conf 0; their logits rows are never read.
 * Decisions are taken as in exact arithmetic evaluated in fp64: positions whose fast fp32
 * estimate lies within a relative 1e-4 band of the threshold or of the fallback's best
 * candidate are recomputed in fp64 on the device.
 *
 *   logits     [B, S, V]   dtype (finite values)   (device, read)
 *   mask       [B, S]      uint8, nonzero = masked (device, read)
 *   gamma      any non-NaN value (gamma <= 0 commits every masked position)
 *   token_id   [B, S]      int32                   (device, written)
 *   committed  [B, S]      uint8                   (device, written)
 *   conf       [B, S]      float, may be NULL      (device, written)
 *
 *   workspace  device memory of tt_commit_workspace(B, S, V, dtype) bytes: 16 bytes per
 *              (position, vocabulary chunk of 16384 bf16 / 8192 fp32 entries); contents on
 *              entry are ignored.
 *
 * Supported: dtype TT_BF16 or TT_F32, 1 <= S <= 1024, 1 <= V, and B*S*ceil(V/chunk) <=
 * 16777215 (one workgroup per position and chunk); anything else returns
 * TT_ERR_UNSUPPORTED. B == 0 is a no-op.
 * ------------------------------------------------------------------------------------- */
size_t tt_commit_workspace(int32_t B, int32_t S, int32_t V, int32_t dtype);

tt_status tt_commit(int32_t B, int32_t S, int32_t V, int32_t dtype, const void *logits,
                    const uint8_t *mask, float gamma, int32_t *token_id, uint8_t *committed,
                    float *conf, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * tt_commit_noalloc -- tt_commit without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, serving loops that must not allocate,
 * harnesses that forbid it). Same operation, arguments, results and kernels as tt_commit;
 * the scratch is the library's own static device array of 4 MiB per GPU (allocated with the
 * library's code object, held until the process ends), so the call allocates nothing.
 *
 * Limit: tt_commit_workspace(B, S, V, dtype) <= 4 MiB (e.g. B*S <= 16384 rows of a
 * 131072-entry bf16 vocabulary); larger shapes return TT_ERR_UNSUPPORTED. Nothing in the
 * array has to start at zero (each call writes every record it reads).
 * Every call on one GPU uses that GPU's single array: calls that may overlap on one GPU
 * (other streams, other threads) race and must be serialized by the caller.
 * ------------------------------------------------------------------------------------- */
tt_status tt_commit_noalloc(int32_t B, int32_t S, int32_t V, int32_t dtype, const void *logits,
                            const uint8_t *mask, float gamma, int32_t *token_id,
                            uint8_t *committed, float *conf, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * tt_lmhead_commit -- the LM head and the confidence commit of one denoising step, fused:
 * the logits are never written to memory.
 *
 * Defined by Nemotron-TwoTower (gist.science explainer), Technical Summary > Training and
 * Conditioning > Sampling (every masked token is predicted at once from the denoiser's
 * output; those whose confidence is above gamma are committed) and the snilld.dk TwoTower
 * article, "Blockwise generering i praksis". The prediction's last step is the LM head: for
 * every masked position (b,i),
 *   l[b,i,v] = sum_k hidden[b,i,k] * weight[v,k]     (bf16 inputs, fp32 accumulation,
 *                                                      summation order unspecified)
 * and then the rule of tt_commit on these fp32 logits: token = lowest v attaining the max,
 * Z = sum_v exp(l_v - max), conf = 1/Z, committed = conf > gamma, and the fallback to the
 * most confident masked position (lowest i on ties) of a sequence that commits nothing.
 * Unlike tt_commit there is no exact recomputation near the threshold (there are no stored
 * logits to recompute from): the decisions are taken on the fp32 logits and an fp64 merge
 * of fp32 partial sums of exp. The logits themselves carry the fp32 accumulation error,
 * at most K * 2^-24 * sum_k |hidden[b,i,k] * weight[v,k]| per logit.
 *
 *   hidden     [B, S, K]   bf16 (device, read: masked rows only)
 *   weight     [V, K]      bf16 (device, read), the head's rows, one per vocabulary entry
 *   mask       [B, S]      uint8, nonzero = masked (device, read)
 *   gamma      any non-NaN value
 *   token_id   [B, S]      int32 (device, written; -1 at unmasked positions)
 *   committed  [B, S]      uint8 (device, written)
 *   conf       [B, S]      float, may be NULL (device, written; 0 at unmasked positions)
 *   workspace  device memory of tt_lmhead_commit_workspace(B, S, K, V) bytes (20 bytes per
 *              position and 256-entry vocabulary chunk, plus 16 per position); contents on
 *              entry are ignored
 *
 * Supported: K a multiple of 64 (at most 2^20); 1 <= S <= 1024; B*S <= 4096;
 * B*S*K < 2^31; any V >= 1; hidden and weight starting on a 16-byte boundary (16-byte
 * loads). Anything else returns TT_ERR_UNSUPPORTED. B == 0 is a no-op.
 * ------------------------------------------------------------------------------------- */
size_t tt_lmhead_commit_workspace(int32_t B, int32_t S, int32_t K, int32_t V);

tt_status tt_lmhead_commit(int32_t B, int32_t S, int32_t K, int32_t V, const void *hidden,
                           const void *weight, const uint8_t *mask, float gamma,
                           int32_t *token_id, uint8_t *committed, float *conf, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * tt_lmhead_commit_exact -- tt_lmhead_commit whose integer outputs are those of exact
 * arithmetic on the bf16 inputs.
 *
 * Same definition and arguments as tt_lmhead_commit, with one more input:
 *   w_bound    float (device, read): an upper bound on max_v ||weight[v,:]||_2, as written by
 *              tt_lmhead_weight_bound for this weight (compute it once per weight)
 * Every fp32 logit lies within eps = 2 K 2^-24 ||hidden[b,i,:]||_2 w_bound of its exact value
 * (bf16 products are exact in fp32; at most K roundings, each within one unit of the sum of
 * the magnitudes). A position whose token (top two logits within 2 eps), threshold test
 * (conf within a factor exp(2 eps + 1e-4) of gamma) or fallback (more than one position
 * whose confidence interval reaches the largest lower bound) the fp32 values cannot settle
 * is recomputed in fp64 on the device (all vocabulary tiles when its decision is open, the
 * tiles whose fp32 max is within 2 eps of the row max when only its token is open) and
 * decided on those values: token_id and committed then equal the exact-arithmetic rule's
 * except where a margin lies below fp64 rounding. conf is the fp64 value for a position
 * recomputed over the whole vocabulary, else the fp32-logit estimate. A recomputed row
 * costs a pass over the head rows in fp64 (about K V fp64 multiply-adds); how many rows are
 * recomputed depends on eps and the logits.
 *
 *   workspace  device memory of tt_lmhead_commit_exact_workspace(B, S, K, V) bytes
 *              (per position and vocabulary chunk 45 bytes, plus about 40 per position)
 *
 * Supported: as tt_lmhead_commit. Errors as tt_lmhead_commit; w_bound NULL is
 * TT_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------------------- */
size_t tt_lmhead_commit_exact_workspace(int32_t B, int32_t S, int32_t K, int32_t V);

tt_status tt_lmhead_commit_exact(int32_t B, int32_t S, int32_t K, int32_t V, const void *hidden,
                                 const void *weight, const uint8_t *mask, float gamma,
                                 const float *w_bound, int32_t *token_id, uint8_t *committed,
                                 float *conf, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * tt_lmhead_weight_bound -- the head-row norm bound of tt_lmhead_commit_exact.
 *
 *   weight  [V, K] bf16 (device, read)
 *   bound   float (device, written): max_v ||weight[v,:]||_2 (fp64 sums of the exact squares),
 *           rounded up to fp32
 * Supported: V >= 0, K >= 1, V*K < 2^40. Errors: TT_ERR_INVALID_ARG for a negative V, K < 1
 * or a NULL pointer (weight may be NULL when V == 0), TT_ERR_UNSUPPORTED past the size limit.
 * ------------------------------------------------------------------------------------- */
tt_status tt_lmhead_weight_bound(const void *weight, int32_t V, int32_t K, float *bound,
                                 hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * tt_ctx_append -- context cache update after a block is committed.
 *
 * Defined by Nemotron-TwoTower (gist.science explainer), Technical Summary > Generation
 * Process (once a block is committed, the context tower updates its states with the new
 * clean tokens) and the snilld.dk TwoTower article, "Blockwise generering i praksis" (the
 * context tower then updates its caches, once per block rather than per token). For one
 * attention layer, the new key and value rows of the committed block (the context tower's
 * output for its clean tokens, computed by the caller) are written after the context:
 *
 *   k_ctx[b, ctx_len[b] + i, :, :] = k_new[b, i, :, :]   for i < S   (likewise v)
 *   and, when bump != 0, ctx_len[b] += S   (call with bump on the last layer of a step)
 *
 *   k_new, v_new  [B, S, Hkv, D]     dtype    (device, read)
 *   k_ctx, v_ctx  [B, Lmax, Hkv, D]  dtype    (device, read and written: rows ctx_len[b] ..
 *                                              ctx_len[b]+S-1 only)
 *   ctx_len       [B] int32                   (device, read; written when bump != 0)
 *   skipped       [B] uint8, may be NULL      (device, written: 1 where the block did not fit)
 * A sequence whose block does not fit (ctx_len[b] < 0 or ctx_len[b] + S > Lmax) is left
 * unchanged, its ctx_len included, and flagged in skipped. Element bits are copied
 * unchanged. The shape's Hq is not used.
 *
 * Supported: dtype TT_BF16 or TT_F32; 1 <= S <= 1024; 1 <= D <= 256; B <= 8191;
 * B*Lmax*Hkv*D, B*S*Hkv*D < 2^31. Anything else returns TT_ERR_UNSUPPORTED. B == 0 is a
 * no-op. k_new/v_new must not overlap k_ctx/v_ctx/ctx_len. No workspace.
 * ------------------------------------------------------------------------------------- */
tt_status tt_ctx_append(const tt_attn_shape *shape, const void *k_new, const void *v_new,
                        void *k_ctx, void *v_ctx, int32_t *ctx_len, int32_t bump,
                        uint8_t *skipped, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * tt_mamba2_seeded_scan -- the denoiser's Mamba-2 layer over one block, from the state the
 * context tower hands over.
 *
 * Defined by the snilld.dk TwoTower article, "Hvad TwoTower aendrer teknisk" (the denoiser's
 * Mamba-2 states are seeded directly from the context tower) and Nemotron-TwoTower
 * (gist.science explainer), Technical Summary > Methodology > Architecture (the context
 * tower produces layer-aligned KV caches and Mamba states) and its ablations (Mamba stays
 * causal). Per sequence b and head h (group g = h / (H/G)), the Mamba-2 selective
 * state-space recurrence over t = 0..S-1 from state_{-1} = h0[b,h]:
 *
 *   delta_t = softplus(dt[b,t,h] + dt_bias[h]),   a_t = exp(-exp(A_log[h]) delta_t)
 *   state_t = a_t state_{t-1} + delta_t x[b,t,h,:] B[b,t,g,:]^T     (P x N)
 *   y[b,t,h,:] = state_t C[b,t,g,:] + Dskip[h] x[b,t,h,:]
 *
 * and, when h_out is given, h_out[b,h] = state_{S-1} (the context tower's own state update
 * over a committed block is the same call). fp32 arithmetic; y in the input dtype (bf16
 * rounded to nearest even).
 *
 *   x        [B, S, H, P]  dtype       (device, read)
 *   dt       [B, S, H]     float       (device, read), before the softplus
 *   dt_bias, A_log, Dskip [H] float    (device, read)
 *   Bm, Cm   [B, S, G, N]  dtype       (device, read)
 *   h0       [B, H, P, N]  float       (device, read; 16-byte aligned)
 *   y        [B, S, H, P]  dtype       (device, written)
 *   h_out    [B, H, P, N]  float, may be NULL (device, written; 16-byte aligned)
 *
 * Supported: dtype TT_BF16 or TT_F32; P a power of 2 in [4, 128]; N <= 128 with N/(256/P)
 * in {4, 8, 16, 32, 64} (e.g. P = 64, N = 128); S <= 1024; element counts < 2^31. Anything
 * else returns TT_ERR_UNSUPPORTED (an h0/h_out off a 16-byte boundary too). B == 0 is a
 * no-op. No workspace. h_out must not overlap h0.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    int32_t B, S, H, P, N, G;
    int32_t dtype; /* tt_dtype of x, Bm, Cm and y */
} tt_mamba_shape;

tt_status tt_mamba2_seeded_scan(const tt_mamba_shape *shape, const void *x, const float *dt,
                                const float *dt_bias, const float *A_log, const float *Dskip,
                                const void *Bm, const void *Cm, const float *h0, void *y,
                                float *h_out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * tt_adaln_modulate / tt_adaln_gate -- adaLN-single time modulation of one denoiser layer.
 *
 * Defined by Nemotron-TwoTower (gist.science explainer), Technical Summary > Training and
 * Conditioning > Time Conditioning (the denoiser is conditioned on the diffusion timestep
 * through adaptive layer normalization) and the snilld.dk TwoTower article, "Hvad TwoTower
 * aendrer teknisk" (every layer is time-modulated by a small adaLN-single block). The single
 * block gives each sequence one set of vectors t_mod[b] = (shift, scale, gate) from its
 * timestep, shared by all layers; each layer adds its own offsets table = (shift, scale,
 * gate). For every row x[b,i,0:d]:
 *
 *   tt_adaln_modulate:  y = (x - mean) / sqrt(var + eps) * (1 + scale) + shift
 *                       (mean and var of the row; no affine terms), before the mixer
 *   tt_adaln_gate:      out = x + gate * f   (the mixer's output f joins the residual)
 *
 * with shift/scale/gate = t_mod[b, 0/1/2, :] + table[0/1/2, :]. fp32 arithmetic; outputs in
 * the input dtype.
 *
 *   x, f, y, out  [B, S, d]  dtype   (device)
 *   t_mod         [B, 3, d]  float   (device, read)
 *   table         [3, d]     float   (device, read)
 *   eps           finite, >= 0
 *
 * Supported: dtype TT_BF16 or TT_F32; d <= 8192; B*S*d < 2^31. Anything else returns
 * TT_ERR_UNSUPPORTED. B == 0 is a no-op. y/out may be x itself (in place); no workspace.
 * ------------------------------------------------------------------------------------- */
tt_status tt_adaln_modulate(int32_t B, int32_t S, int32_t d, int32_t dtype, const void *x,
                            const float *t_mod, const float *table, float eps, void *y,
                            hipStream_t stream);

tt_status tt_adaln_gate(int32_t B, int32_t S, int32_t d, int32_t dtype, const void *x,
                        const void *f, const float *t_mod, const float *table, void *out,
                        hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Kernel timing (measurement support). While enabled, each call records HIP events on its
 * stream around the kernels listed in tt_profile_stats. The events are created once, on
 * the first enable (no device memory); up to 4096 calls per field are recorded, later ones
 * are counted but not timed. tt_profile_read() synchronizes on the recorded events and
 * returns the accumulated times; tt_profile_reset() clears them.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    int64_t attn_calls;       /* tt_block_denoise_attn calls timed                        */
    double attn_total_ms;     /* sum over those calls, first launch to last              */
    double attn_main_ms;      /* sum over those calls, the main attention kernel alone   */
    int64_t commit_calls;     /* tt_commit calls timed                                   */
    double commit_total_ms;   /* sum over those calls, first launch to last              */
    double commit_reduce_ms;  /* sum over those calls, the vocabulary reduction kernel   */
    int64_t lm_calls;         /* tt_lmhead_commit calls timed                            */
    double lm_total_ms;       /* sum over those calls, first launch to last              */
    double lm_reduce_ms;      /* sum over those calls, the fused head + reduction kernel */
} tt_profile_stats;

tt_status tt_profile_enable(int32_t enable);
tt_status tt_profile_reset(void);
tt_status tt_profile_read(tt_profile_stats *out);

#ifdef __cplusplus
}
#endif

#endif /* TT_H */
