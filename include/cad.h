/*
 * cad.h — C ABI of the MI355X (gfx950) span-commit / verify library, libcad.so.
 *
 * One data-parallel hot path, in three calls:
 *   cad_ngram_lookup  — prompt-lookup draft search over int32 token histories
 *                       (PLD page, "The n-gram match, precisely"; SwitchSD's kappa-gram gate
 *                       and recency-ranked candidate retrieval);
 *   cad_span_forward  — one parallel forward of a decoder layer + LM head over Nq new tokens
 *                       per sequence, appending their K/V to the cache (Copy-as-Decode §2.4,
 *                       copy-span splicing via parallel prefill; the same forward is the
 *                       speculative verifier), with a causal-span or a block-triangular
 *                       multi-candidate mask (SwitchSD, block-triangular verification);
 *   cad_accept_scan   — greedy left-to-right acceptance of drafts against the forward's argmax
 *                       (PLD page, "Verification in a single parallel pass"; SwitchSD's
 *                       longest validated continuation), with KV-length update.
 *
 * Conventions for every call
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library never
 *     allocates, frees or synchronizes; all work is enqueued on `stream` in order.
 *   - Return value: CAD_OK (0) or a negative CAD_E* code.  Argument errors are detected on
 *     the host and returned before anything is enqueued.  No exception crosses the ABI.
 *   - Conditions only the device can see (a sequence whose cache or history would overflow)
 *     are reported per sequence in `err[b]` (when given) and make that sequence's work a
 *     no-op: nothing is written for it and its lengths stay unchanged.
 *   - Layouts are dense row-major with the shapes given; no strides except where named.
 *   - The first call on a device compiles nothing and allocates nothing; calls on one
 *     stream are ordered, calls on different streams that share buffers race.
 */
#ifndef CAD_H
#define CAD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define CAD_OK            0
#define CAD_EINVAL       -1   /* null pointer, non-positive size, inconsistent arguments      */
#define CAD_EUNSUPPORTED -2   /* shape outside what the kernels handle (see each call)        */
#define CAD_ECAPACITY    -3   /* device-side: len + Nq > cap, or history overflow            */
#define CAD_EHIP         -4   /* a HIP launch failed                                          */
#define CAD_EWORKSPACE   -5   /* workspace missing or smaller than cad_span_forward_workspace */

/* storage format of weights, cache and activations */
#define CAD_DTYPE_BF16    0   /* bf16 storage, fp32 accumulation                              */
#define CAD_DTYPE_F32     1   /* fp32 storage and accumulation                                */

/* attention mask of a span forward */
#define CAD_MASK_CAUSAL_SPAN 0  /* row i at slot/position len+i sees slots [0, len+i]           */
#define CAD_MASK_BLOCK_TRI   1  /* Nq = W*D; row (w,j) at slot len+w*D+j, position len+j, sees
                                   [0,len) and slots len+w*D+j' for j' <= j                    */

/* span-forward flags */
#define CAD_COMMIT_ALL   1    /* len += Nq at the end of the forward (a copy span: acceptance 1) */
#define CAD_KV_ONLY      2    /* stop after appending K/V (prefill of a cache); no outputs     */
#define CAD_LOGITS_LAST  4    /* copy-commit mode: final norm, LM head and argmax only for each
                                 sequence's last row (inside a copy span only the prediction after
                                 the span is used); causal-span mask only                     */

/*
 * A pre-norm decoder layer with grouped-query attention and a SwiGLU MLP, followed by a
 * final RMSNorm and an untied LM head.  RMSNorm gains are 1, there are no biases, RoPE is the
 * half-split form (element i pairs with i + head_dim/2) at absolute positions with angles
 * p * rope_base^(-2i/head_dim).  Query head h reads KV head h / (n_q_heads / n_kv_heads).
 * All matrices are row-major [out, in] in `dtype`:
 *   embed     [vocab, hidden]
 *   w_qkv     [(n_q_heads + 2*n_kv_heads) * head_dim, hidden]   rows: Q heads, K heads, V heads
 *   w_o       [hidden, n_q_heads * head_dim]
 *   w_gate_up [2 * ffn, hidden]                                rows: gate, then up
 *   w_down    [hidden, ffn]
 *   w_lm      [vocab, hidden]
 * Supported: hidden, head_dim*n_q_heads and ffn multiples of 8, hidden <= 8192; head_dim in {32, 64, 128};
 * n_q_heads a multiple of n_kv_heads.
 */
typedef struct {
    int hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int dtype;                 /* CAD_DTYPE_BF16 or CAD_DTYPE_F32 */
    float rms_eps;             /* added to mean(x^2) before the inverse square root */
    double rope_base;
    const void *embed, *w_qkv, *w_o, *w_gate_up, *w_down, *w_lm;
} cad_layer_desc;

/*
 * KV cache of B sequences, in `dtype`:
 *   k: [B, n_kv_heads, cap, head_dim]  slot-major: k[b][g][s][i]
 *   v: [B, n_kv_heads, head_dim, cap]  dim-major:  v[b][g][i][s]
 * Slot s of sequence b holds the key/value of the token at position s (after acceptance); slots
 * at or past len + Nq may hold anything, NaN included (the attention reads whole 64-slot tiles
 * but no such value reaches a result).  The
 * value cache is stored transposed so that attention reads, for one dimension, a contiguous run
 * of slots (the operand layout of the value product).  cap must be a multiple of 4.
 * len: [B] int32, device-resident current lengths.  err: [B] int32, nullable; set to
 * CAD_ECAPACITY for a sequence whose operation would overflow, and by a forward to CAD_EINVAL for
 * a sequence whose tokens hold an id outside [0, vocab) (never cleared by the library).
 * n_kv_heads, head_dim and dtype must match the layer the cache is used with.
 */
typedef struct {
    void *k, *v;
    int32_t *len;
    int32_t *err;
    int B, cap;
    int n_kv_heads, head_dim, dtype;
} cad_kv_desc;

/*
 * cad_ngram_lookup — most-recent-first suffix match (PLD page, "The n-gram match,
 * precisely"; SwitchSD, candidate retrieval ranked by recency).
 *
 *   ctx        [B, ctx_stride] int32 histories; sequence b uses ctx[b*ctx_stride + 0 .. len-1]
 *   ctx_len    [B] int32 device lengths (len)
 *   n, W, D    suffix length (>= 1), candidates kept (1..8), draft length (1..64)
 *   with_current 0 or 1.  Row layout of `draft` for sequence b is
 *                [with_current ? ctx[len-1] : nothing, cand_0[0..D-1], ..., cand_{W-1}[0..D-1]]
 *                so with_current=1 gives directly the token rows [g, d_1..d_D] of a causal
 *                verify forward, and with_current=0 the W*D rows of a block verify.
 *   draft      [B, with_current + W*D] int32 out; entries past a candidate's length are 0
 *   draft_len  [B, W] int32 out; min(D, len - (j + n)) for a hit at start j, else 0
 *   match_pos  [B, W] int32 out, nullable; the start j of each hit, -1 where none
 *
 * The suffix is ctx[len-n .. len-1]; candidate starts are j = len-n-1 down to 0 (at least one
 * continuation token, the suffix never matching itself, overlap allowed), the first W hits
 * are kept in that order.  len < n+1 gives no hit.  Lengths outside [0, ctx_stride] are
 * clamped for the scan.  Errors: CAD_EINVAL, CAD_EUNSUPPORTED (W > 8, D > 64, n > 64).
 */
int cad_ngram_lookup(const int32_t *ctx, int64_t ctx_stride, const int32_t *ctx_len, int B,
                     int n, int W, int D, int with_current,
                     int32_t *draft, int32_t *draft_len, int32_t *match_pos,
                     hipStream_t stream);

/*
 * cad_ngram_lookup_longest — the longest-match policy of the same search (PLD page, "The n-gram
 * match, precisely": with several matches a policy may prefer the longest; n is often 1-3).
 * Suffix lengths n = n_max, n_max-1, ..., n_min are tried in turn; the hits of the first length
 * with any hit are kept exactly as cad_ngram_lookup keeps them for that n.
 *
 *   n_max, n_min  1 <= n_min <= n_max <= 64
 *   match_n    [B] int32 out, nullable: the suffix length used, 0 when no length matched
 *   other arguments, outputs and layouts as for cad_ngram_lookup.
 * Errors: CAD_EINVAL, CAD_EUNSUPPORTED (W > 8, D > 64, n_max > 64).
 */
int cad_ngram_lookup_longest(const int32_t *ctx, int64_t ctx_stride, const int32_t *ctx_len, int B,
                             int n_max, int n_min, int W, int D, int with_current,
                             int32_t *draft, int32_t *draft_len, int32_t *match_pos,
                             int32_t *match_n, hipStream_t stream);

/*
 * cad_span_forward — one parallel forward of Nq new tokens per sequence (Copy-as-Decode §2.4
 * and Appendix K; SwitchSD block-triangular verification).
 *
 *   tokens      [B, Nq] int32 token ids; a sequence holding an id outside [0, vocab) is flagged
 *               CAD_EINVAL in kv->err and its forward is a no-op (nothing written, length kept)
 *   mask_mode   CAD_MASK_CAUSAL_SPAN, or CAD_MASK_BLOCK_TRI with Nq == W*D
 *   flags       CAD_COMMIT_ALL, CAD_KV_ONLY, CAD_LOGITS_LAST (or-ed)
 *   argmax_out  [B, Nq] int32 out: LM-head argmax per row, ties to the lowest id (nullable
 *               only with CAD_KV_ONLY); [B] (the last row's) with CAD_LOGITS_LAST
 *   hidden_out  [B*Nq, hidden] dtype out, nullable: the layer output (residual stream)
 *   logits_out  [B*Nq, vocab] fp32 out, nullable (debug; costs a full logits write);
 *               [B, vocab] with CAD_LOGITS_LAST
 *   top2_gap    [B*Nq] fp32 out, nullable ([B] with CAD_LOGITS_LAST): largest minus second-largest
 *               logit of each row (0 for a tie), the margin by which the argmax is decided
 *   workspace   device scratch of at least cad_span_forward_workspace(...) bytes, 256-aligned
 *
 * Every row first appends its K/V at slot len+i (RoPE at the row's position), then attends
 * to the cached prefix and the span rows its mask allows (append-then-attend: a row reads
 * its own key as stored).  Rounding points (bf16 round-to-nearest-even for a bf16 layer):
 * normed input, rotated q, stored k and v, attention output, second normed input, SwiGLU
 * product, hidden_out, final normed input; the residual stream and logits are fp32.
 * Copy-as-Decode's copy-span commit (§2.4) needs only the prediction after the span:
 * CAD_LOGITS_LAST runs the final norm, LM head and argmax for row Nq-1 of each sequence; the
 * cache rows and hidden_out are those of a full forward.
 * Errors: CAD_EINVAL (also: CAD_LOGITS_LAST with the block mask), CAD_EUNSUPPORTED (also: cap
 * not a multiple of 4, or one head's bf16 K cache, cap * head_dim * 2 bytes, of 2 GiB or more),
 * CAD_EWORKSPACE, CAD_EHIP; per sequence CAD_ECAPACITY in kv->err when len + Nq > cap.
 */
int cad_span_forward(const cad_layer_desc *layer, const cad_kv_desc *kv,
                     const int32_t *tokens, int B, int Nq,
                     int mask_mode, int W, int D, int flags,
                     int32_t *argmax_out, void *hidden_out, float *logits_out, float *top2_gap,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * cad_span_forward_noalloc — cad_span_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The same
 * forward with the same arguments, except that its workspace is a static device array of
 * CAD_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library: every device the library runs on holds
 * one from the library's load until the process ends.  The call allocates nothing.
 *   Limit: forwards whose cad_span_forward_workspace(...) exceeds CAD_NOALLOC_SCRATCH_BYTES return
 *   CAD_EWORKSPACE (at the 1.5B shape up to 64 rows fit, at the 7B shape up to 32).
 *   Sharing: every call on one device uses that device's one array, which keeps the last call's
 *   contents (nothing in it needs to start at zero).  Calls on one stream are ordered; calls that
 *   overlap on one device (several streams, or host threads) race on the array.
 * Errors: as cad_span_forward; CAD_EWORKSPACE (too large, see above); CAD_EHIP when the array's
 * device address cannot be obtained.
 */
#define CAD_NOALLOC_SCRATCH_BYTES (32 << 20)
int cad_span_forward_noalloc(const cad_layer_desc *layer, const cad_kv_desc *kv,
                             const int32_t *tokens, int B, int Nq,
                             int mask_mode, int W, int D, int flags,
                             int32_t *argmax_out, void *hidden_out, float *logits_out, float *top2_gap,
                             hipStream_t stream);

/*
 * cad_span_forward_allowed — a causal span forward whose argmax is restricted to a per-row set
 * of allowed token ids (Copy-as-Decode §2.3: at the grammar's decision points the FSM intersects
 * the model's logits with the ids its state allows, e.g. {<, </} at an op boundary).  Only the
 * allowed rows of the LM head are read (A of them per row instead of the vocabulary).
 *
 *   flags       CAD_COMMIT_ALL and/or CAD_LOGITS_LAST (the decision after each sequence's last row
 *               only, as at the end of a forced-template prefill or a copy splice); R = B*Nq rows,
 *               or R = B with CAD_LOGITS_LAST
 *   allowed     [R, A] int32 ids; entries outside [0, vocab) are padding
 *   A           1 .. CAD_MAX_ALLOWED
 *   argmax_out  [R] int32 out: the allowed id with the largest logit, ties to the lowest id;
 *               -1 for a row whose set holds no valid id
 *   logits_out  [R, A] fp32 out, nullable: the logit at each allowed slot, -inf for padding
 *   hidden_out, workspace (cad_span_forward_workspace with the same B, Nq), stream: as for
 *               cad_span_forward; the cache rows are those of a full forward.
 * Errors: CAD_EINVAL, CAD_EUNSUPPORTED (A out of range, and as cad_span_forward), CAD_EWORKSPACE,
 * CAD_EHIP; per sequence CAD_ECAPACITY in kv->err when len + Nq > cap.
 */
#define CAD_MAX_ALLOWED 16
int cad_span_forward_allowed(const cad_layer_desc *layer, const cad_kv_desc *kv,
                             const int32_t *tokens, int B, int Nq, int flags,
                             const int32_t *allowed, int A,
                             int32_t *argmax_out, float *logits_out, void *hidden_out,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * cad_span_forward_sampled — a causal span forward whose LM head draws tokens instead of
 * taking the argmax, for stochastic verification of a retrieved draft (PLD page, speculative
 * decoding: with the rejection-sampling correction the output keeps the target's sampling
 * distribution).  The draft is deterministic, so the correction reads: keep the draft token d
 * with probability p(d), otherwise draw from p without d; after the last draft draw the bonus
 * token from p.  p = softmax(logits / temperature).
 *
 *   tokens      [B, Nq] the forward's input [g, d_1 .. d_k, padding]; row i < draft_len[b]
 *               (clamped to Nq - 1) holds the draft d = tokens[b, i + 1]
 *   draft_len   [B] device int32, nullable (then no row holds a draft)
 *   flags       CAD_COMMIT_ALL and/or CAD_LOGITS_LAST (each sequence's last row only, no drafts)
 *   pred_out    [R] int32 out (R = B*Nq, or B with CAD_LOGITS_LAST): a drafted row gives d if
 *               kept, else its replacement draw; a row without a draft gives a plain draw.  Fed
 *               to cad_accept_scan as pred (causal mode, with_current = 1) it yields exactly the
 *               stochastic acceptance: the scan runs while drafts were kept and emits the first
 *               replacement, or the bonus draw.
 *   logits_out  [R, vocab] fp32 out, nullable
 * Randomness: Philox4x32-10 (Salmon et al., SC'11) with key (seed low word, seed high word).
 * The Gumbel noise of vocabulary id x in the row of sequence b at absolute position pos uses
 * counter (x / 4, pos, b, 0), output word x % 4; the acceptance uniform of that row uses counter
 * (0, pos, b, 1), word 0.  A word w becomes the uniform (2 * (w >> 9) + 1) / 2^24.  Draws of one
 * (seed, sequence, position) are therefore the same in every launch shape.
 * Errors: CAD_EINVAL (temperature not a positive finite number, flags, as cad_span_forward),
 * CAD_EUNSUPPORTED (fp32 layers), CAD_EWORKSPACE (cad_span_forward_workspace with the same B,
 * Nq, flags), CAD_EHIP; per sequence CAD_ECAPACITY in kv->err.
 */
int cad_span_forward_sampled(const cad_layer_desc *layer, const cad_kv_desc *kv, const int32_t *tokens,
                             int B, int Nq, int flags, float temperature, uint64_t seed,
                             const int32_t *draft_len, int32_t *pred_out, float *logits_out,
                             void *hidden_out, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * cad_stack_span_forward — the span forward through a whole stack of n_layers decoder layers
 * (Copy-as-Decode §2.4 splices a copy span through the full model; its Table 11 times whole
 * models).  Same arguments and outputs as cad_span_forward, with:
 *   layers   [n_layers] descriptors of identical shape, dtype, eps and rope base; the embedding
 *            of layers[0] and the LM head of layers[n_layers-1] are used (those fields of the
 *            other layers are ignored and may be NULL)
 *   kvs      [n_layers] caches, one per layer, of identical B and cap; the lengths and error
 *            flags are those of kvs[0] (every layer's rows are written at kvs[0].len and only
 *            kvs[0].len is advanced); kvs[l].len / .err are ignored for l > 0
 * Layer l+1 takes layer l's residual output as its input and that output's RMSNorm (gain 1) as
 * its normed input.  With CAD_KV_ONLY every layer but the last runs in full (their outputs feed
 * the next layer's K/V) and the last writes its K/V rows only.
 * Errors: as cad_span_forward; CAD_EINVAL also for n_layers outside 1..CAD_MAX_LAYERS or layers
 * that disagree in shape.
 */
#define CAD_MAX_LAYERS 256
int cad_stack_span_forward(const cad_layer_desc *layers, int n_layers, const cad_kv_desc *kvs,
                           const int32_t *tokens, int B, int Nq, int mode, int W, int D, int flags,
                           int32_t *argmax_out, void *hidden_out, float *logits_out, float *top2_gap,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);
/* The masked-decision forward (as cad_span_forward_allowed) through a stack of layers, with the
 * layers, caches and lengths of cad_stack_span_forward: a grammar decision point of a program run
 * on the whole model. */
int cad_stack_span_forward_allowed(const cad_layer_desc *layers, int n_layers, const cad_kv_desc *kvs,
                                   const int32_t *tokens, int B, int Nq, int flags,
                                   const int32_t *allowed, int A, int32_t *argmax_out, float *logits_out,
                                   void *hidden_out, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);
/* The sampled forward (as cad_span_forward_sampled: stochastic verification of the drafts in
 * tokens[:, 1:], or plain draws) through a stack of layers, with the layers, caches and lengths
 * of cad_stack_span_forward; the draws are keyed by (seed, sequence, position) as there. */
int cad_stack_span_forward_sampled(const cad_layer_desc *layers, int n_layers, const cad_kv_desc *kvs,
                                   const int32_t *tokens, int B, int Nq, int flags, float temperature,
                                   uint64_t seed, const int32_t *draft_len, int32_t *pred_out,
                                   float *logits_out, void *hidden_out, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);
/* Workspace of cad_stack_span_forward (0 for an invalid shape); the buffers are reused by every
 * layer, so this is the one-layer size (the full one when n_layers > 1, even with CAD_KV_ONLY). */
size_t cad_stack_span_forward_workspace(const cad_layer_desc *layers, int n_layers, int B, int Nq, int mode,
                                        int W, int D, int cap, int flags);

/* Bytes of workspace cad_span_forward needs for these arguments and flags (0 on invalid
 * arguments).  A CAD_KV_ONLY forward needs far less than a full one. */
size_t cad_span_forward_workspace(const cad_layer_desc *layer, int B, int Nq, int mask_mode,
                                  int W, int D, int cap, int flags);

/*
 * cad_accept_scan — greedy acceptance and commit (PLD page, "Verification in a single
 * parallel pass"; SwitchSD, longest validated continuation).
 *
 *   draft, with_current, draft_len : as written by cad_ngram_lookup (same W, D)
 *   pred        causal: [B, 1+D] argmax of the verify forward over [g, d_1..d_D];
 *               block:  [B, W*D] argmax of the block forward over the W candidates
 *   first_pred  block: [B] the target's prediction at the cached anchor; NULL in causal mode
 *   mask_mode   CAD_MASK_CAUSAL_SPAN (W must be 1, with_current 1) or CAD_MASK_BLOCK_TRI
 *               (with_current 0)
 *   accepted    [B] out: a (causal) or a* (block)
 *   best_w      [B] out, nullable: winning candidate (0 in causal mode)
 *   emitted     [B, D+1] out: the a accepted draft tokens then the bonus token; rest 0
 *   n_emitted   [B] out: a + 1
 *   ctx, ctx_stride, ctx_len, ctx_cap : nullable history; when given the emitted tokens are
 *               appended at ctx_len[b] and ctx_len[b] grows by a+1 (if ctx_len+a+1 > ctx_cap the
 *               sequence is flagged CAD_ECAPACITY in kv->err and nothing is appended)
 *   kv          nullable; when given, causal: len += a+1 (g and the accepted drafts are now
 *               cached); block: the winner's first a* slots move from slot len+w*D+j to len+j
 *               (keys and values) and len += a*.
 * Causal: a = number of leading i < draft_len with d_{i+1} == pred[i]; bonus = pred[a].
 * Block: a_w = leading run of candidate w checked against first_pred, then against
 * pred[w*D + j - 1]; the largest a_w wins, ties to the lowest w; bonus = first_pred when a* = 0,
 * else pred[w*D + a* - 1].  Draft lengths are clamped to [0, D].
 * A skipped sequence (kv->err already set, or its history or cache would overflow; an overflow
 * is flagged CAD_ECAPACITY in kv->err when kv is given) gets accepted = 0, best_w = 0,
 * n_emitted = 0 and a zero emitted row, and no length changes: n_emitted[b] == 0 identifies it,
 * since a sequence that ran always emits at least one token.
 * Errors: CAD_EINVAL, CAD_EUNSUPPORTED (W > 8, D > 64).
 */
int cad_accept_scan(const int32_t *draft, int with_current, const int32_t *draft_len,
                    const int32_t *pred, const int32_t *first_pred,
                    int B, int W, int D, int mask_mode,
                    int32_t *accepted, int32_t *best_w, int32_t *emitted, int32_t *n_emitted,
                    int32_t *ctx, int64_t ctx_stride, int32_t *ctx_len, int ctx_cap,
                    const cad_kv_desc *kv, hipStream_t stream);

/*
 * cad_stack_accept_scan — cad_accept_scan for a verify forward run through a stack of layers
 * (cad_stack_span_forward; SwitchSD's block verify on the whole model).  Arguments as
 * cad_accept_scan, with the caches of cad_stack_span_forward:
 *   kvs        [n_layers] caches (required), lengths and error flags those of kvs[0]
 *   best_w     required in block mode with n_layers > 1
 * Causal mode: kvs[0].len += a+1 (every layer's rows are already in place).  Block mode: the
 * winner's first a* K/V slots move from len + w*D + j to len + j in EVERY layer's cache, then
 * kvs[0].len += a*.
 * Errors: as cad_accept_scan; CAD_EINVAL also for n_layers outside 1..CAD_MAX_LAYERS, a missing
 * best_w, or caches that disagree in B, cap, heads, head_dim or dtype.
 */
int cad_stack_accept_scan(const int32_t *draft, int with_current, const int32_t *draft_len,
                          const int32_t *pred, const int32_t *first_pred,
                          int B, int W, int D, int mask_mode,
                          int32_t *accepted, int32_t *best_w, int32_t *emitted, int32_t *n_emitted,
                          int32_t *ctx, int64_t ctx_stride, int32_t *ctx_len, int ctx_cap,
                          const cad_kv_desc *kvs, int n_layers, hipStream_t stream);

/*
 * Diagnostics: per-stage GPU time of cad_span_forward.  While enabled, every forward records a
 * HIP event on its stream before and after each kernel stage (the events come from a pool the
 * library creates on first use; no device memory is allocated).  cad_profile_read waits for the
 * recorded events, adds each stage's elapsed milliseconds into ms_sum[stage] and its launch count
 * into count[stage] (arrays of max_stages, zero them first), clears the record and returns the
 * number of stages.  cad_profile_stage_name names a stage.  Single-threaded use only; not for
 * use under graph capture.
 */
int cad_profile_enable(int on);
int cad_profile_read(int max_stages, double *ms_sum, int *count);
const char *cad_profile_stage_name(int stage);

/* Static description of a status code. */
const char *cad_status_string(int status);

/* Library version: major*10000 + minor*100 + patch. */
int cad_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CAD_H */
