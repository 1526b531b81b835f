/*
 * decode_attn.h -- C ABI of the MI355X (gfx950) decode-attention library.
 *
 * The library computes the attention core of one autoregressive decode step
 * over a bf16 KV cache, for s query tokens per sequence (s = 1 plain decode,
 * s > 1 speculative / multi-token-prediction drafts), in two forms:
 *
 *  - mla_decode: multi-head latent attention in absorbed form. The absorbed
 *    query q_lat = Q.Wk^T scores directly against the cached latent Z, the
 *    decoupled rope part q_rope scores against the cached rope keys, and the
 *    output stays in latent space, softmax(.).Z ("Mla Analysis" skill page,
 *    sections "Absorption Trick (FlashMLA)" and "Tensor Shapes"). Decompressing
 *    the output through Wv is the caller's separate step.
 *  - gqa_decode: grouped-query attention, covering MHA (hkv = hq), GQA and MQA
 *    (hkv = 1); query heads form contiguous groups of hq/hkv that share one K/V
 *    head ("Why MLA and MTP Fight Each Other", introduction table of attention
 *    variants; "MQA, GQA & MLA" lesson, Concept section).
 *
 * Semantics shared by both entry points
 *  - Softmax attention per query row: lse = ln(sum_j exp(scale * q.k_j)) over
 *    the visible cache rows j, out = sum_j exp(scale * q.k_j - lse) * v_j.
 *  - Draft mask: with L = seqlens[b] clamped to [0, t_max], query token i
 *    (0 <= i < s) of sequence b sees cache rows 0 .. L - s + i (L counts the
 *    drafts' own rows). A row that sees no cache row gets out = 0, lse = -inf.
 *  - lse is in natural-log units, fp32. out is bf16, rounded to nearest even.
 *  - Arithmetic: bf16 products with fp32 accumulation (MFMA / dot2), fp32
 *    online softmax. A sequence split over several workers passes through
 *    per-segment partial outputs normalized by their own softmax sums and
 *    stored as bf16 (one extra rounding, as the final output's), with fp32
 *    log-sum-exps, before its combine. Results are not bitwise identical
 *    across split choices.
 *
 * Pointers and ownership
 *  - Every tensor pointer is a DEVICE pointer to contiguous row-major memory;
 *    bf16 tensors are passed as uint16_t bit patterns. The caller allocates and
 *    owns every buffer, including the workspace; the library allocates nothing
 *    per call and keeps only a cached device-property query (thread-safe).
 *  - `stream` is a hipStream_t (NULL = the default stream). All work is queued
 *    asynchronously on it; no call synchronizes the host and no call reads
 *    seqlens on the host. Buffers must stay alive until the stream's work ends.
 *  - Inputs must not alias outputs or the workspace.
 *
 * Workspace: device memory the caller passes for the split-KV plan and the
 * per-segment partial results (size from the matching *_workspace_size,
 * 256-byte aligned, contents on entry irrelevant). A NULL workspace (with
 * workspace_bytes ignored) is allowed for the three attention calls and
 * forces one split: every sequence is one worker's, whose blocks write its
 * rows directly (no partials, no combine launch; num_workers is ignored).
 * That path is slower when b times the blocks per sequence is small against
 * the device's compute units.
 *
 * Errors: a problem the host can see returns a status and queues nothing.
 *  DA_ERR_INVALID_ARG  null tensor pointer, a dimension <= 0, hq % hkv != 0,
 *                      s > t_max, num_workers < 0, a non-finite scale, a
 *                      misaligned pointer.
 *  DA_ERR_UNSUPPORTED  a dimension outside the compiled set (see each call).
 *  DA_ERR_WORKSPACE    workspace_bytes below the matching *_workspace_size.
 *  DA_ERR_HIP          a HIP launch error (the HIP error is cleared).
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DA_OK = 0,
    DA_ERR_INVALID_ARG = 1,
    DA_ERR_UNSUPPORTED = 2,
    DA_ERR_WORKSPACE = 3,
    DA_ERR_HIP = 4
} da_status;

/* Library ABI version (major * 100 + minor). */
int da_version(void);

/* Human-readable name of a status code (static storage, never NULL). */
const char *da_status_string(da_status status);

/*
 * Work partition ("split-KV"): the cache rows of all sequences are cut into
 * tiles and the flat list of tiles is divided evenly among `num_workers`
 * workers; a sequence touched by several workers is merged afterwards by a
 * log-sum-exp combine. num_workers = 0 lets the library choose from the
 * device's compute-unit count and the shapes. Any value >= 1 is valid and
 * gives the same result up to rounding (of the bf16 partials when split).
 */

/*
 * Bytes of workspace mla_decode needs for these shapes and num_workers (same
 * meaning as in mla_decode). Returns 0 for arguments mla_decode would reject.
 */
size_t mla_decode_workspace_size(int b, int s, int h, int k, int p, int t_max, int num_workers);

/*
 * Absorbed-latent MLA decode.
 *   q_lat   [b, s, h, k]     bf16   absorbed queries, row (b, i, head)
 *   q_rope  [b, s, h, p]     bf16   rope part of the queries
 *   cache   [b, t_max, k+p]  bf16   per token: k latent columns, then p rope columns
 *   seqlens [b]              int32  valid cache rows per sequence, drafts included
 *   scale                    fp32   multiplies the full latent+rope dot product
 *   out_lat [b, s, h, k]     bf16   softmax-weighted latent rows (value = latent part)
 *   lse     [b, s, h]        fp32   natural-log log-sum-exp of the scaled scores
 *   workspace                device memory of at least
 *                            mla_decode_workspace_size(b, s, h, k, p, t_max, num_workers)
 *                            bytes, 256-byte aligned; its contents on entry do not matter;
 *                            or NULL (one split per sequence, see above).
 * Compiled set: (k, p) in {(512, 64), (256, 64), (128, 64), (64, 16)}, h >= 1,
 * s * h <= 65536, t_max * (k + p) * 2 < 2^31.
 */
da_status mla_decode(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *cache,
                     const int32_t *seqlens, int b, int s, int h, int k, int p, int t_max,
                     float scale, uint16_t *out_lat, float *lse, void *workspace,
                     size_t workspace_bytes, int num_workers, void *stream);

/*
 * mla_decode without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * semantics and errors as mla_decode, minus the workspace: the plan and the
 * split-KV partials live in a device array inside the library of
 * DA_NO_ALLOC_SCRATCH_BYTES bytes per device, held until the process ends.
 * Returns DA_ERR_WORKSPACE when the call needs more than that (the
 * mla_decode_workspace_size of the same arguments is the need; about 21 MB at
 * b=32, s=1, h=128, k=512, t=4096 and 34 MB at s=4), DA_ERR_HIP if the
 * array's device address cannot be obtained. Every call on one device shares
 * that device's array: calls that overlap on one device (different streams
 * or host threads without ordering) race and must not be issued.
 */
#define DA_NO_ALLOC_SCRATCH_BYTES (64u << 20)
da_status mla_decode_no_alloc(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *cache,
                              const int32_t *seqlens, int b, int s, int h, int k, int p, int t_max,
                              float scale, uint16_t *out_lat, float *lse, int num_workers, void *stream);

/* Bytes of workspace gqa_decode needs for these shapes, num_workers and path
 * (0 for arguments gqa_decode would reject). */
size_t gqa_decode_workspace_size(int b, int s, int hq, int hkv, int d, int t_max, int num_workers, int path);

/*
 * Grouped-query decode (MHA when hkv == hq, MQA when hkv == 1).
 *   q       [b, s, hq, d]      bf16
 *   k_cache [b, t_max, hkv, d] bf16
 *   v_cache [b, t_max, hkv, d] bf16
 *   seqlens [b]                int32
 *   out     [b, s, hq, d]      bf16
 *   lse     [b, s, hq]         fp32 (natural log)
 * Query head hh reads K/V head hh / (hq / hkv).
 * Compiled set: d in {64, 128, 256}; R = (hq / hkv) * s query rows per K/V
 * head with R <= 256 (R <= 128 for d = 256); t_max * hkv * d * 2 < 2^31.
 * `path` selects the kernel: 1 = VALU dot kernel (R <= 16), 2 = MFMA kernel
 * (rows padded to blocks of 16, spread over up to four waves per K/V head
 * that share its cache reads), 0 = automatic (currently the MFMA kernel for
 * every R). Both give the same result up to rounding. Workspace as for
 * mla_decode (NULL allowed). With the MFMA kernel, d = 64 or 128 (R <= 64)
 * or d = 256 (R <= 32), and either a NULL workspace or num_workers == 0 with
 * b * hkv at least the device's compute-unit count, no sequence is split:
 * one block per (sequence, K/V head) splits the tokens over its waves and
 * writes the rows itself, and the workspace is not touched (at d = 64 with
 * hkv a multiple of 8 the automatic choice keeps the split form instead).
 * The automatic choice assumes sequences near t_max; pass num_workers > 0 to
 * balance a batch of very unequal lengths over split-KV workers instead.
 */
da_status gqa_decode(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                     const int32_t *seqlens, int b, int s, int hq, int hkv, int d, int t_max,
                     float scale, uint16_t *out, float *lse, void *workspace,
                     size_t workspace_bytes, int num_workers, int path, void *stream);

/* Bytes of workspace mla_decode_unabsorbed needs (0 for arguments it would
 * reject). */
size_t mla_decode_unabsorbed_workspace_size(int b, int s, int h, int dqk, int dv, int t_max, int num_workers);

/*
 * Un-absorbed (FlashAttention-style) MLA decode: the same attention as
 * mla_decode, computed on per-head decompressed keys and values instead of the
 * shared latent ("MLA Cost Analysis & Regime Guide": "Cost Models",
 * FlashAttention, whose byte count charges per head and token a d + p key row
 * and a d value row; "Regime Selection" sets it against FlashMLA as s grows).
 * Every query head has its own K/V head (hkv = h).
 *   q       [b, s, h, dqk]      bf16   per head [q_nope | q_rope]
 *   k_cache [b, t_max, h, dqk]  bf16   per token and head [k_nope | k_rope]
 *   v_cache [b, t_max, h, dv]   bf16
 *   seqlens [b]                 int32  valid cache rows, drafts included
 *   scale                       fp32   multiplies q . k
 *   out     [b, s, h, dv]       bf16
 *   lse     [b, s, h]           fp32   natural log
 * Draft mask, ownership, errors and workspace (NULL allowed) as for mla_decode.
 * Compiled set: (dqk, dv) = (192, 128) (DeepSeek's 128 + 64 rope / 128);
 * s <= 64; t_max * h * dqk * 2 < 2^31.
 */
da_status mla_decode_unabsorbed(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                                const int32_t *seqlens, int b, int s, int h, int dqk, int dv, int t_max,
                                float scale, uint16_t *out, float *lse, void *workspace,
                                size_t workspace_bytes, int num_workers, void *stream);

/*
 * Per-head projections either side of absorbed MLA decode ("MLA Cost Analysis
 * & Regime Guide", "Absorption Trick (FlashMLA)": the queries enter latent
 * space through Wk^T before the attention; a separate kernel decompresses the
 * latent output with Wv after it). For every head hd:
 *   mla_absorb_queries:    q_lat[b,s,hd,:] = w_k[hd] . q_nope[b,s,hd,:]
 *       q_nope [b,s,h,d], w_k [h,k,d] (Wk of the head: latent row c holds a d-vector), q_lat [b,s,h,k]
 *   mla_decompress_output: out[b,s,hd,:] = w_v_t[hd] . o_lat[b,s,hd,:]
 *       o_lat [b,s,h,k], w_v_t [h,d,k] (Wv of the head transposed: row j holds a k-vector), out [b,s,h,d]
 * bf16 in and out (round to nearest even), fp32 accumulation. The contracted
 * width (d for the queries, k for the output) must be a multiple of 32 and all
 * three tensors 16-byte aligned. No workspace; queued asynchronously on `stream`.
 * Errors: DA_ERR_INVALID_ARG (null pointer, dimension <= 0, misaligned input),
 * DA_ERR_UNSUPPORTED (contracted width not a multiple of 32, or 64 * h * width
 * * 2 bytes, the span of a 64-row tile's inputs, not below 2^31).
 */
da_status mla_absorb_queries(const uint16_t *q_nope, const uint16_t *w_k, uint16_t *q_lat, int b, int s, int h,
                             int d, int k, void *stream);
da_status mla_decompress_output(const uint16_t *o_lat, const uint16_t *w_v_t, uint16_t *out, int b, int s, int h,
                                int k, int d, void *stream);

/* Bytes of workspace mla_decode_split_cache needs (0 for arguments it would reject). */
size_t mla_decode_split_cache_workspace_size(int b, int s, int h, int o_max, int n_max, int num_workers);

/*
 * MLA decode over a split cache ("MLA Cost Analysis & Regime Guide", "MLAvar6+
 * Design"): the o older tokens of a sequence stay as latent rows, the n newest
 * (the s drafts among them) are kept decompressed per head. Attention over all
 * o + n tokens, computed as absorbed attention on the old part (queries taken
 * into latent space with w_k, output decompressed with w_v_t), un-absorbed
 * attention on the new part, and a log-sum-exp merge of the two.
 *   q_nope  [b,s,h,128], q_rope [b,s,h,64]   bf16
 *   w_k     [h,512,128], w_v_t [h,128,512]    bf16 (as for the projections above)
 *   latent  [b,o_max,576]  bf16, seqlens_old [b] int32 (o per sequence, clamped)
 *   k_new   [b,n_max,h,192], v_new [b,n_max,h,128]  bf16, seqlens_new [b] int32
 *   out     [b,s,h,128] bf16, lse [b,s,h] fp32 (natural log)
 * Draft i sees every old row and the first n - s + i + 1 new rows (the drafts'
 * own rows are the last s of the new part, so n >= s; with n < s the drafts'
 * order across the split is not the un-split one). Compiled set: latent 512,
 * rope 64, head 128; s <= n_max, s <= 64. Ownership and errors as for
 * mla_decode; the workspace is required (it also holds the intermediates).
 */
da_status mla_decode_split_cache(const uint16_t *q_nope, const uint16_t *q_rope, const uint16_t *w_k,
                                 const uint16_t *w_v_t, const uint16_t *latent, const int32_t *seqlens_old,
                                 const uint16_t *k_new, const uint16_t *v_new, const int32_t *seqlens_new, int b,
                                 int s, int h, int o_max, int n_max, float scale, uint16_t *out, float *lse,
                                 void *workspace, size_t workspace_bytes, int num_workers, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
