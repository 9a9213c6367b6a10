/*
 * orthrus.h -- C ABI of the MI355X (gfx950) hot path of one Orthrus
 * dual-view decode step: block attention over a shared paged KV cache,
 * greedy consensus (argmax + longest-prefix accept), its sampling form at
 * temperature T > 0, the LM head with a fused argmax, KV append and the
 * prompt prefill that fills the cache.
 *
 * Semantics follow the Orthrus explainer page for "Orthrus: Memory-Efficient
 * Parallel Token Generation via Dual-View Diffusion" (gist.science, arXiv
 * 2605.12825), technical summary §2.1-§2.3.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer (hipMalloc / torch CUDA
 *     memory) owned by the caller.  The library never allocates, frees or
 *     retains caller memory; its only mutable global state is the fixed
 *     scratch array of orthrus_block_attn_noalloc.
 *   - Work is only enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream); no call synchronises.  Results are ready when the stream is.
 *   - Errors are synchronous and host-detectable only: a non-OK status means
 *     nothing was enqueued.  ORTHRUS_ERR_LAUNCH means a launch was attempted
 *     and the HIP runtime reported an error right after it.
 *   - Device-resident values (ctx_lens, page ids, accept_len) are checked by
 *     the kernels: an out-of-range context length or page id never faults; it
 *     makes the affected rows' results unspecified (cache rows are not
 *     written through an invalid page id).
 *   - Alignment: q, out, k_cache, v_cache, k_blk, v_blk, k, v (prefill),
 *     hidden and the LM-head weights must be 16-byte aligned, arrays of
 *     device addresses 8-byte aligned and int32 arrays 4-byte aligned;
 *     otherwise the call returns ORTHRUS_ERR_SHAPE and enqueues nothing.
 *   - For a fixed descriptor every output is bit-identical from run to run.
 *   - Calls are reentrant; calls that share a workspace must be ordered on
 *     one stream.
 *
 * Layouts (row-major, innermost last)
 *   q, out          [B, K, Hq, D]            storage dtype
 *   k_blk, v_blk    [B, K, Hkv, D]           storage dtype
 *   k_cache, v_cache[num_pages, Hkv, P, D]   storage dtype (one (page, head)
 *                                            is P*D contiguous elements)
 *   page_table      [B, max_pages_per_seq]   int32 physical page ids
 *   ctx_lens        [B]                      int32 cached tokens per sequence
 *   ar_logits, draft_logits [B, K, V]        fp32
 *   draft_tokens    [B, K]                   int32
 *   u_accept [B, K], u_resample [B]          fp32
 *   hidden [rows, H], weight [V, H]          bf16 (LM head; the calls take the
 *                                            weight packed once)
 *   accept_len, next_token, new_ctx_lens [B] int32
 *   ar_tokens, slots[B, K]                   int32
 * Logical position p of sequence b lives in page page_table[b][p / P], slot
 * p % P.  Query head h reads KV head h * Hkv / Hq (grouped-query attention).
 */
#ifndef ORTHRUS_H
#define ORTHRUS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORTHRUS_ABI_VERSION 1

/* Which view's mask the block rows use inside the block (explainer §2.2,
 * §2.3).  Both views see the whole cached context. */
typedef enum {
  ORTHRUS_DIFF_BIDIR = 0, /* diffusion view, M_diff: block rows attend to each other both ways */
  ORTHRUS_AR_CAUSAL = 1   /* frozen AR head's verify pass: block row i sees block rows j <= i   */
} orthrus_mode;

typedef enum { ORTHRUS_BF16 = 0, ORTHRUS_F32 = 1 } orthrus_dtype;

/* split_tokens value that asks for the balanced split of a ragged batch.
 * With bf16 storage, Hq / Hkv <= 4, 2 <= batch <= 64, batch * Hkv < 256 and
 * max_ctx_len < 2^24, the kernels read every ctx_lens[b] and take the
 * smallest split (a multiple of 64 in [320, 8192]) that gives at most
 * Q = ceil(256 / Hkv) work-groups per KV head, so that one round of about 256
 * work-groups covers the batch as evenly as 64-position tiles allow.  When
 * that round would be poorly balanced (the average work-group below 85 % of
 * the longest), they take the smallest split with at most 2 Q work-groups
 * per KV head instead (two rounds of shorter work-groups); a batch of equal
 * lengths always stays at one round.  The launch and the workspace are sized
 * for the worst case that max_ctx_len allows.  Outside those bounds it means
 * 0 (automatic). */
#define ORTHRUS_SPLIT_BALANCED (-1)

typedef enum {
  ORTHRUS_OK = 0,
  ORTHRUS_ERR_NULL = 1,        /* a required pointer is NULL                          */
  ORTHRUS_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent    */
  ORTHRUS_ERR_UNSUPPORTED = 3, /* dtype / head_dim / group / page size not supported  */
  ORTHRUS_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required          */
  ORTHRUS_ERR_LAUNCH = 5       /* the HIP runtime reported an error after a launch    */
} orthrus_status;

/* Shape of one block-attention / append call.
 *   batch               B >= 1
 *   block_k             K, 1 <= K <= 32 (the pages use K = 32: anchor + 31 masks)
 *   n_q_heads, n_kv_heads  Hq, Hkv; Hq % Hkv == 0, Hq / Hkv in {1, 2, 4, 8}
 *   head_dim            D in {64, 128}
 *   page_size           P, must be 16
 *   max_pages_per_seq   row length of page_table
 *   num_pages           physical pages in k_cache / v_cache
 *   max_ctx_len         upper bound on every ctx_lens[b] (sizes the launch);
 *                       max_ctx_len + K <= max_pages_per_seq * P
 *   dtype               storage type of q, out, caches and block K/V
 *   softmax_scale       <= 0 selects 1 / sqrt(D)
 *   split_tokens        context positions per work-group: a multiple of 64
 *                       in [64, 8192]; 0 = automatic (the shortest split,
 *                       at least 320, that keeps a batch of max_ctx_len
 *                       contexts within one round of ceil(256 / Hkv)
 *                       work-groups per KV head; for one sequence whose
 *                       context then needs at most 8 stages of 64 positions
 *                       per work-group, the shortest split of at least 192
 *                       that fills about 80 % of a round instead; the best
 *                       measured choices when the lengths are equal);
 *                       ORTHRUS_SPLIT_BALANCED = chosen on the device from
 *                       ctx_lens (ragged batches, below) */
typedef struct {
  int32_t batch;
  int32_t block_k;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t max_ctx_len;
  int32_t dtype;
  float softmax_scale;
  int32_t split_tokens;
} orthrus_attn_desc;

int32_t orthrus_abi_version(void);
/* Text of a status code (any int; unknown codes give "unknown status").
 * Codes and modes cross the ABI as int32_t: a caller may pass any value, and
 * the library checks it before treating it as one of the enumerations. */
const char* orthrus_status_str(int32_t status);

/* Bytes of caller-provided scratch orthrus_block_attn needs for `desc`
 * (split-context partial results: bf16 for bf16 storage with Hq/Hkv <= 4,
 * fp32 otherwise, plus fp32 row statistics; under the balanced split also one
 * (splits, first slot) pair per sequence).  0 for an invalid descriptor or
 * when no sequence can be split.  The workspace needs no initialisation. */
size_t orthrus_block_attn_workspace_bytes(const orthrus_attn_desc* desc);

/* Context positions per work-group that orthrus_block_attn will use for
 * `desc` (the split length), or 0 for an invalid descriptor.  Under the
 * balanced split it is the split of a batch whose lengths all equal
 * max_ctx_len; the kernels choose the actual one from ctx_lens. */
int32_t orthrus_block_attn_split_tokens(const orthrus_attn_desc* desc);

/* Block attention of one decode step (explainer §2.1-§2.3).
 *
 * mode is an orthrus_mode value (anything else: ORTHRUS_ERR_SHAPE).
 * For every sequence b (L = ctx_lens[b]), query head h and block row i < K:
 *   keys/values = the L cached rows of KV head h*Hkv/Hq followed by the K
 *   block rows k_blk/v_blk[b, :, h*Hkv/Hq]; row i sees all L cached keys and
 *   block key j when mode == DIFF_BIDIR (any j) or AR_CAUSAL (j <= i);
 *   out[b, i, h] = softmax(scale * q . k) . v over the visible keys.
 * Accumulation is fp32; bf16 outputs are rounded to nearest even once.
 * k_cache/v_cache are read only (the cache holds the AR keys/values that both
 * views share).  `out` must not alias any input.  workspace may be NULL only
 * when orthrus_block_attn_workspace_bytes(desc) == 0. */
orthrus_status orthrus_block_attn(const void* q, const void* k_cache, const void* v_cache,
                                  const void* k_blk, const void* v_blk, const int32_t* page_table,
                                  const int32_t* ctx_lens, int32_t mode, void* out,
                                  const orthrus_attn_desc* desc, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Largest workspace orthrus_block_attn_noalloc can serve (32 MiB: every
 * decode shape up to 32 query heads x 32 rows x 64 partial slots per
 * sequence and KV-head group, e.g. Qwen3-8B heads at batch 16 x 8192 or
 * batch 4 x 32768 cached tokens, or the balanced split of 16 ragged
 * sequences of up to 16384 tokens, whose two rounds take 64 slots). */
#define ORTHRUS_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/* orthrus_block_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics and results as orthrus_block_attn,
 * without the workspace: the split partials go to a fixed device array of
 * ORTHRUS_STATIC_SCRATCH_BYTES that the library owns, one copy per GPU, held
 * until the process ends.  The call allocates nothing (its first call on a
 * GPU looks up that GPU's copy once).
 *   ORTHRUS_ERR_WORKSPACE  when orthrus_block_attn_workspace_bytes(desc)
 *                          exceeds ORTHRUS_STATIC_SCRATCH_BYTES;
 *   ORTHRUS_ERR_LAUNCH     when the stream's device cannot be determined.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (on different streams or
 * from different threads) race and give unspecified results.  Calls ordered
 * on one stream are safe. */
orthrus_status orthrus_block_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const void* k_blk, const void* v_blk, const int32_t* page_table,
                                          const int32_t* ctx_lens, int32_t mode, void* out,
                                          const orthrus_attn_desc* desc, void* stream);

/* Bytes of the workspace orthrus_greedy_accept needs (one 8-byte key per
 * (row, logit chunk); chunks of 4096 logits when batch * block_k <= 64,
 * else 8192).  The workspace needs no initialisation. */
size_t orthrus_greedy_accept_workspace_bytes(int32_t batch, int32_t block_k, int32_t vocab);

/* Greedy consensus of one step (explainer §2.3).
 *   g[b, i]       = lowest index of the maximum of ar_logits[b, i, :]
 *                   (fp32 compare; -0.0 ties with +0.0; logits must not be NaN)
 *   accept_len[b] = number of leading i with draft_tokens[b, i] == g[b, i], in [0, K]
 *   next_token[b] = g[b, min(accept_len[b], K-1)]  (the AR correction token, or
 *                   the last accepted token when all K drafts agree)
 *   ar_tokens     = g when non-NULL.
 * The step commits min(accept_len + 1, K) tokens: g[b, 0 .. n-1].
 * 1 <= K <= 32, 1 <= V < 2^31. */
orthrus_status orthrus_greedy_accept(const float* ar_logits, const int32_t* draft_tokens,
                                     int32_t* accept_len, int32_t* next_token, int32_t* ar_tokens,
                                     int32_t batch, int32_t block_k, int32_t vocab, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Bytes of the workspace orthrus_sample_accept needs (per row and
 * logit chunk one 16-byte pair of (max, sum) for each head, plus per
 * sequence the decision and one residual sum per chunk; chunks of 4096
 * logits when batch * block_k <= 64, else 8192).  0 for an invalid shape.
 * The workspace needs no initialisation. */
size_t orthrus_sample_accept_workspace_bytes(int32_t batch, int32_t block_k, int32_t vocab);

/* Lossless consensus at temperature T > 0: the stochastic form of the
 * accept step (explainer §2.3; §4 names the sampling temperatures), the
 * standard rejection rule under which the committed tokens follow the AR
 * head's distribution.  For row i of sequence b, p = softmax(ar_logits/T),
 * q = softmax(draft_logits/T) (fp32, each row's max subtracted) and
 * x = draft_tokens[b, i]:
 *   x is accepted when u_accept[b, i] * q[x] < p[x];
 *   accept_len[b] = the first rejected i, or K when none is rejected;
 *   next_token[b] = at a rejection, the smallest v whose running sum of
 *                   r = max(p - q, 0) exceeds u_resample[b] * sum(r) (from p
 *                   itself when r is zero everywhere); with no rejection,
 *                   draft_tokens[b, K-1].
 * The step commits min(accept_len + 1, K) tokens: the accepted drafts, then
 * next_token.  The caller draws the uniforms (u_accept [B, K] and
 * u_resample [B], fp32 in [0, 1)); draft_logits has ar_logits' layout
 * [B, K, V] fp32.  A draft outside [0, V) is rejected.  Every row needs a
 * finite logit; logits must not be NaN or +inf.  T must be finite with
 * log2(e) / T finite.  1 <= K <= 32, 1 <= V < 2^31. */
orthrus_status orthrus_sample_accept(const float* ar_logits, const float* draft_logits,
                                     const int32_t* draft_tokens, const float* u_accept,
                                     const float* u_resample, float temperature, int32_t* accept_len,
                                     int32_t* next_token, int32_t batch, int32_t block_k, int32_t vocab,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the packed LM-head weight: ceil(V / 32) * 32 * H * 2.  0 for an
 * invalid shape (H a multiple of 256 in [256, 65536], V >= 1). */
size_t orthrus_lm_head_packed_bytes(int32_t hidden_size, int32_t vocab);

/* Repack an LM-head weight [V, H] bf16 (row-major) into the layout the
 * LM-head calls stream, once per weight.  For vocabulary tile t (rows
 * 32t .. 32t+31), k-step s (hidden elements 16s .. 16s+15) and lane l in
 * [0, 64), the 16 bytes at byte offset ((t * H/16 + s) * 64 + l) * 16 hold
 * weight[32t + l % 32][16s + 8 (l / 32) .. 16s + 8 (l / 32) + 7], zero for
 * rows >= V.  Each wave of the LM-head kernel then reads its 32-row tile as
 * one sequential stream.  weight and packed are 16-byte aligned device
 * buffers that must not overlap. */
orthrus_status orthrus_lm_head_pack_weight(const void* weight, void* packed, int32_t hidden_size, int32_t vocab,
                                           void* stream);

/* Bytes of the workspace the LM-head calls need for `rows` hidden rows: one
 * 8-byte key per (row, 128-entry vocabulary tile).  0 for an invalid shape.
 * The workspace needs no initialisation. */
size_t orthrus_lm_head_workspace_bytes(int32_t rows, int32_t hidden_size, int32_t vocab);

/* Greedy tokens straight from final hidden states: the vocabulary projection
 * of each view (explainer §2.3: the drafts and the AR targets are the two
 * heads' predictions over the vocabulary) with its argmax fused, so the
 * logits are never stored.
 *   logits[m, v] = sum_k hidden[m, k] * weight[v, k]  (bf16 operands, fp32
 *                  accumulation; no bias or scaling)
 *   tokens[m]    = lowest v attaining the maximum (-0.0 ties with +0.0;
 *                  inputs must not produce NaN)
 *   max_logits[m]= that maximum (optional, may be NULL)
 * hidden [rows, H] bf16 (row-major); packed_weight is the weight [V, H] in
 * the layout of orthrus_lm_head_pack_weight; both 16-byte aligned.
 * H a multiple of 256 in [256, 65536]; 1 <= rows <= 2^24; V >= 1. */
orthrus_status orthrus_lm_head_argmax(const void* hidden, const void* packed_weight, int32_t* tokens,
                                      float* max_logits, int32_t rows, int32_t hidden_size, int32_t vocab,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Greedy consensus straight from the AR view's final hidden states [B, K, H]:
 * the tokens g of orthrus_lm_head_argmax over its B*K rows, then
 * accept_len / next_token / ar_tokens exactly as orthrus_greedy_accept
 * defines them from g.  The workspace is that of
 * orthrus_lm_head_workspace_bytes(B * K, H, V).  1 <= K <= 32. */
orthrus_status orthrus_lm_head_greedy_accept(const void* hidden, const void* packed_weight,
                                             const int32_t* draft_tokens, int32_t* accept_len,
                                             int32_t* next_token, int32_t* ar_tokens, int32_t batch,
                                             int32_t block_k, int32_t hidden_size, int32_t vocab,
                                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the workspace orthrus_lm_head_denoise_step needs for `rows`
 * hidden rows: per (row, 128-entry vocabulary tile) one 8-byte argmax key
 * and one (max, sum) pair of floats.  0 for an invalid shape.  The
 * workspace needs no initialisation. */
size_t orthrus_lm_head_denoise_workspace_bytes(int32_t rows, int32_t hidden_size, int32_t vocab);

/* One step of multi-step denoising for the diffusion view (the agentlenshq
 * Orthrus-Qwen3 blog, training and implementation details, and the warokai
 * guide, advanced settings, name the iterated variant; its re-mask rule is
 * not given, so this is low-confidence remasking), fused into the LM head:
 * from the final
 * hidden states [B, K, H] of the block and the packed weight,
 *   tokens[b, i]     = greedy token of row i (as orthrus_lm_head_argmax)
 *   confidence[b, i] = its softmax probability 1 / sum_v exp(logit_v - max)
 *                      (optional, may be NULL)
 *   new_masked[b, i] = masked[b, i] unless row i is among the n_unmask[b]
 *                      most confident rows with masked != 0 (ties to the
 *                      lower row), which become 0.
 * The logits are never stored.  masked / new_masked are uint8 [B, K]
 * (nonzero = still masked) and may alias; n_unmask is int32 [B].
 * 1 <= K <= 32; shapes as for orthrus_lm_head_argmax. */
orthrus_status orthrus_lm_head_denoise_step(const void* hidden, const void* packed_weight, const uint8_t* masked,
                                            const int32_t* n_unmask, int32_t* tokens, float* confidence,
                                            uint8_t* new_masked, int32_t batch, int32_t block_k,
                                            int32_t hidden_size, int32_t vocab, void* workspace,
                                            size_t workspace_bytes, void* stream);

/* Commit the accepted block rows to the shared cache (explainer §2.3: the
 * cache keeps only the committed positions).
 *   n_b = min(max(accept_len[b], 0) + 1, K); for r < n_b and every KV head,
 *   k_blk/v_blk[b, r] is copied bit-exactly to logical position
 *   L_b + r = ctx_lens[b] + r of k_cache/v_cache.  Nothing else is written.
 *   new_ctx_lens[b] = L_b + n_b            (optional, may be NULL)
 *   slots[b, r] = page * P + slot written, -1 for r >= n_b (optional)
 * A sequence with ctx_lens[b] outside [0, max_ctx_len] violates the
 * descriptor: nothing of it is written, new_ctx_lens[b] = -1 and its slots
 * are all -1 (the other sequences are unaffected).  A row whose page id is
 * outside [0, num_pages) is not written and its slot is -1.
 * ctx_lens is read only: in a multi-layer step pass new_ctx_lens only on
 * the last layer so every layer appends at the same positions.  Neither
 * output may alias ctx_lens, accept_len or page_table. */
orthrus_status orthrus_kv_append(void* k_cache, void* v_cache, const void* k_blk, const void* v_blk,
                                 const int32_t* page_table, const int32_t* ctx_lens,
                                 const int32_t* accept_len, int32_t* new_ctx_lens, int32_t* slots,
                                 const orthrus_attn_desc* desc, void* stream);

/* orthrus_kv_append for n_layers layers in one launch.  The four arguments
 * *_ptrs are DEVICE arrays of n_layers device addresses (layer l's k_cache,
 * v_cache, k_blk, v_blk); every layer shares page_table, ctx_lens and
 * accept_len (one step commits the same positions in every layer).
 * new_ctx_lens and slots are written once.  1 <= n_layers <= 4096. */
orthrus_status orthrus_kv_append_layers(const uint64_t* k_cache_ptrs, const uint64_t* v_cache_ptrs,
                                        const uint64_t* k_blk_ptrs, const uint64_t* v_blk_ptrs, int32_t n_layers,
                                        const int32_t* page_table, const int32_t* ctx_lens,
                                        const int32_t* accept_len, int32_t* new_ctx_lens, int32_t* slots,
                                        const orthrus_attn_desc* desc, void* stream);

/* Bytes of the workspace orthrus_prefill needs: the virtual page-table rows
 * and context lengths of the prompt's 32-row chunks plus the block-attention
 * workspace of that virtual batch.  0 for an invalid shape.  The workspace
 * needs no initialisation; it must be 256-byte aligned. */
size_t orthrus_prefill_workspace_bytes(const orthrus_attn_desc* desc, int32_t max_prompt);

/* How many of the prompt's 32-row chunks one attention work-group of
 * orthrus_prefill serves for this shape: 2 when the work-groups of chunk
 * pairs still fill two rounds of the GPU (bf16 with at most 4 query heads per
 * KV head; each work-group then streams its keys once for both chunks), else
 * 1.  0 for an invalid shape.  Informational: the results do not depend on
 * it beyond rounding order. */
int32_t orthrus_prefill_chunks_per_workgroup(const orthrus_attn_desc* desc, int32_t max_prompt);

/* Prompt prefill by the frozen AR head (explainer §2.1: the prompt's keys
 * and values fill the shared cache that both views read).  For sequence b
 * with L = ctx_lens[b] tokens already cached and n = prompt_lens[b] prompt
 * rows (0 <= n <= max_prompt):
 *   - rows r < n of k/v are written bit-exactly to logical positions L + r of
 *     k_cache/v_cache (through page_table; nothing else is written);
 *   - out[b, i, h] for i < n = softmax(scale * q . k) . v over cached
 *     positions 0 .. L-1 and prompt rows 0 .. i (causal), KV head
 *     h * Hkv / Hq, fp32 accumulation; rows i >= n are unspecified;
 *   - new_ctx_lens[b] = L + n (optional, may be NULL; must not alias
 *     ctx_lens).
 * q, out [B, S, Hq, D] and k, v [B, S, Hkv, D] in the storage dtype, with
 * S = max_prompt rounded up to a multiple of 32 (rows past n are padding
 * the caller allocates).  desc is as for orthrus_block_attn with
 * max_ctx_len bounding every L and block_k ignored (split_tokens 0 selects
 * 8192, the fewest splits); max_ctx_len + S <= max_pages_per_seq * P.  The prompt's 32-row chunks run
 * as AR_CAUSAL blocks of orthrus_block_attn over B * S / 32 virtual
 * sequences, after the cache write, on `stream`. */
orthrus_status orthrus_prefill(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                               const int32_t* page_table, const int32_t* ctx_lens, const int32_t* prompt_lens,
                               int32_t max_prompt, void* out, int32_t* new_ctx_lens,
                               const orthrus_attn_desc* desc, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Measurement helper: streams `bytes` (a multiple of 16) from src to dst with
 * plain 16-byte loads and stores.  Used to calibrate hardware counters and to
 * measure the achievable HBM rate; not part of the decode step. */
orthrus_status orthrus_copy_probe(void* dst, const void* src, size_t bytes, void* stream);

/* Measurement helper: reads `bytes` (a multiple of 16) of src once with
 * 16-byte loads, 16 in flight per thread, and stores one XOR fold per thread
 * into sink (sink_bytes >= 4 MiB; its contents are meaningless).  Measures the
 * achievable HBM read rate; not part of the decode step. */
orthrus_status orthrus_read_probe(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ORTHRUS_H */
