/*
 * pagedkv.h -- C ABI of the paged KV-cache attention library (libpagedkv.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The library implements the attention hot path of a serving engine whose KV
 * cache is paged through block tables and whose batches mix three kinds of
 * request, reordered [decode : extend : prefill]:
 *
 *   kv_write         slot-mapped store of the step's new K/V into the cache
 *   paged_decode     one query token per request against its whole cache
 *   extend_attn      new prompt tokens against cached context (chunked, LSE
 *                    merged) plus the new tokens themselves (causal)
 *   prefill_attn     causal attention over fresh prompts (varlen batch)
 *   kv_pack_layer    gather one layer's KV blocks into a contiguous buffer
 *   kv_unpack_layer  scatter such a buffer into (other) blocks of a cache
 *   mla_decode       absorbed multi-head latent attention decode over a paged
 *                    576-dim latent cache
 *
 * Sources (web pages; cited by title and section):
 *  [ROCm]  "Beyond just running: native inference optimisation in vLLM on AMD
 *          ROCm", vLLM blog 2026-02-27 (ROCm attention backends).
 *  [PD]    "Advanced inference: why your single-node vLLM setup needs
 *          prefill/decode disaggregation", vLLM blog 2026-04-07 (MORI-IO KV
 *          connector).
 *  [Guide] "vLLM disaggregated serving guide", agentlenshq.com.
 *  [Perf]  "From LLM performance optimisation to DeepSeek deployment",
 *          aif.amtbbs.org 2025-02-20.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless stated otherwise.  `stream` is a
 *   hipStream_t passed as void* (NULL = the null stream).  Every call only
 *   enqueues work on `stream`: no host synchronisation, no allocation.
 * - The caller owns every buffer (inputs, outputs and workspace).  Workspace
 *   sizes come from the matching *_workspace_bytes query.
 * - bf16 = bfloat16, fp8 = OCP FP8 E4M3 ("e4m3fn", max 448, no infinities).
 * - Grouped-query attention: query head h reads KV head h / (H_q / H_kv).
 * - lse outputs are natural-log log-sum-exp of the scaled scores:
 *   lse = ln sum_j exp(scale * <q, k_j>).  Any lse pointer may be NULL.
 * - Outputs are rounded to bf16 round-half-to-even from fp32 accumulation.
 * - Return value: KV_OK (0) or a negative kv_status.  Arguments are validated
 *   on the host before any HIP call; on error nothing is enqueued and
 *   kv_last_error() describes the problem.  KV_EHIP reports a failed launch.
 * - Device-resident indices (block ids, slots, lengths) are trusted not to
 *   exceed the bounds the caller passes; kernels clamp block ids to
 *   [0, num_blocks) and lengths to the table width so a bad index cannot
 *   reach outside the cache, but the result is then unspecified.
 * - Calls on different streams may run concurrently; the library keeps no
 *   state besides the thread-local error message.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAGEDKV_ABI_VERSION 1

typedef enum {
  KV_OK = 0,
  KV_EINVAL = -22,    /* bad argument (null pointer, bad size, inconsistent shape) */
  KV_ENOSPC = -28,    /* workspace or destination buffer too small */
  KV_ENOTSUP = -95,   /* valid but unsupported combination (e.g. head_dim != 128) */
  KV_EHIP = -1000     /* a HIP launch failed */
} kv_status;

typedef enum { KV_DTYPE_BF16 = 0, KV_DTYPE_FP8_E4M3 = 1 } kv_dtype;

/* [Perf] section 3 "Paged Attention": fixed-size blocks, stored anywhere,
 * reached through a per-request block table (logical block i of a request ->
 * physical block table[i]).  Two layouts of one layer's cache:
 *  KV_LAYOUT_NHD          k, v: [num_blocks][block_size][num_kv_heads][head_dim]
 *                         (the standard layout: the paged form of [ROCm]
 *                         section "Processing details of the three paths",
 *                         [num_tokens, num_heads, head_dim]).
 *  KV_LAYOUT_PRESHUFFLED  [ROCm] section "ROCM_AITER_FA", hardware-oriented
 *                         KV cache layout:
 *                         k: [num_blocks][num_kv_heads][head_dim/x][block_size][x]
 *                         v: [num_blocks][num_kv_heads][block_size/x][head_dim][x]
 *                         with x = 16 bytes / element size (16 for fp8,
 *                         8 for bf16). */
typedef enum { KV_LAYOUT_NHD = 0, KV_LAYOUT_PRESHUFFLED = 1 } kv_layout;

/* Host struct describing ONE layer's cache.  k_cache / v_cache are device
 * pointers aligned to 16 bytes.  For fp8 the stored code c means c * scale
 * (per-tensor k_scale / v_scale, > 0); for bf16 the scales must be 1. */
typedef struct {
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  int32_t block_size;     /* power of two in [1, 256]; preshuffled: multiple of x */
  int32_t num_kv_heads;
  int32_t head_dim;       /* 128 */
  int32_t dtype;          /* kv_dtype */
  int32_t layout;         /* kv_layout */
  int32_t x;              /* preshuffled only: 16 / element size; ignored for NHD */
  float k_scale;
  float v_scale;
} kv_cache_t;

/* ---------------------------------------------------------------------------
 * kv_write -- [ROCm] section "Unified attention backends": every forward first
 * writes the new key/value into the KV cache, then runs attention; section
 * "Processing details of the three paths", decode: the store keeps the cache
 * in the layout the decode kernel reads.
 *   k, v          [num_tokens][num_kv_heads][head_dim] bf16, contiguous.
 *   slot_mapping  [num_tokens] int64: slot = block * block_size + offset;
 *                 a negative slot skips the token.  Slots must be distinct.
 * bf16 caches receive the bits unchanged.  fp8 caches receive
 * round-half-even(fl32(x) * fl32(1/scale)) saturated to +-448.
 * num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------- */
int kv_write(const kv_cache_t* cache, const void* k, const void* v,
             const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * paged_decode -- [ROCm] section "Every batch handles a mixed workload":
 * decode produces one token per request and must load the request's whole KV
 * cache, so it is bound by memory bandwidth.
 *   q             [batch][num_q_heads][head_dim] bf16
 *   block_tables  [batch][max_blocks_per_seq] int32 physical block ids
 *   seq_lens      [batch] int32, 0 <= seq_lens[b] <= max_seq_len (device)
 *   max_seq_len   host-side upper bound of seq_lens (sizes the split grid)
 *   out           [batch][num_q_heads][head_dim] bf16
 *   lse           [batch][num_q_heads] fp32 or NULL
 *   scale         softmax scale, finite and > 0 (else KV_EINVAL)
 *   workspace     >= paged_decode_workspace_bytes(...) bytes, 16-byte aligned;
 *                 holds the plan and the fp32 partials of split requests
 *                 (about (pieces + batch) * num_q_heads * 516 bytes; a few
 *                 MB to tens of MB at serving shapes), contents need not be
 *                 initialised and are overwritten by every call
 * Balanced split-K: the requests' token streams are concatenated and cut into
 * equal pieces (a small on-device planning pass reads seq_lens), so every
 * workgroup reads the same amount of KV; requests spanning several pieces are
 * combined by log-sum-exp weights ([ROCm] section "Processing details of the
 * three paths", LSE merge).  Lengths above max_seq_len or the table capacity
 * are clamped; a request of length 0 sees no key and gets out = 0 and
 * lse = -inf; batch * max_seq_len must stay below 2^31.  The workspace query
 * sizes for the current device; a call whose stream belongs to a device with
 * more compute units may need more (KV_ENOSPC says so).
 * Layouts/dtypes: NHD bf16, NHD fp8, PRESHUFFLED bf16, PRESHUFFLED fp8.
 * num_q_heads must be a multiple of num_kv_heads.
 * ------------------------------------------------------------------------- */
size_t paged_decode_workspace_bytes(const kv_cache_t* cache, int32_t batch,
                                    int32_t num_q_heads, int32_t max_seq_len);
int paged_decode(const kv_cache_t* cache, const void* q, int32_t batch,
                 int32_t num_q_heads, const int32_t* block_tables,
                 int32_t max_blocks_per_seq, const int32_t* seq_lens,
                 int32_t max_seq_len, float scale, void* out, float* lse,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Same call with an explicit piece length (split_tokens: a multiple of 32 up
 * to 16384, clamped to what the LDS block-table slice holds; 0 = automatic),
 * for tuning and for split-invariance tests. */
size_t paged_decode_workspace_bytes_ex(const kv_cache_t* cache, int32_t batch,
                                       int32_t num_q_heads, int32_t max_seq_len,
                                       int32_t split_tokens);
int paged_decode_ex(const kv_cache_t* cache, const void* q, int32_t batch,
                    int32_t num_q_heads, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* seq_lens,
                    int32_t max_seq_len, float scale, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, int32_t split_tokens,
                    void* stream);

/* ---------------------------------------------------------------------------
 * paged_decode_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): paged_decode with the automatic piece length and no workspace
 * argument.  The plan and the split partials live in a static scratch array
 * of the library, 64 MiB per device (held by every device the library runs
 * on until the process ends), whose address is looked up once per device on
 * the first call there.  Nothing is allocated by the call.  A batch that
 * needs more than 64 MiB of scratch (paged_decode_workspace_bytes) returns
 * KV_ENOSPC.  All calls on one device share that array: calls that may
 * overlap on one device (different streams, or other host threads) race and
 * must be serialised by the caller.  The scratch needs no initialisation
 * (every call rewrites what it reads).  Arguments as for paged_decode.
 * ------------------------------------------------------------------------- */
int paged_decode_noalloc(const kv_cache_t* cache, const void* q, int32_t batch,
                         int32_t num_q_heads, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                         int32_t max_seq_len, float scale, void* out, float* lse,
                         void* stream);

/* ---------------------------------------------------------------------------
 * prefill_attn -- [ROCm] section "Processing details of the three paths",
 * prefill path: Q, K, V in the standard [num_tokens, num_heads, head_dim]
 * layout; section "ROCM_AITER_FA": new sequences go to a variable-length
 * flash-attention kernel on the matrix cores (compute bound).
 *   q             [total_tokens][num_q_heads][head_dim] bf16
 *   k, v          [total_tokens][num_kv_heads][head_dim] bf16
 *   cu_seqlens    [num_seqs+1] int32, cu_seqlens[0] = 0, non-decreasing;
 *                 sequence n owns rows cu_seqlens[n] .. cu_seqlens[n+1]-1
 *   max_seqlen    host-side upper bound of the sequence lengths
 *   causal        1: row i of a sequence sees rows 0..i; 0: all rows
 *   scale         softmax scale, finite and > 0 (else KV_EINVAL)
 *   out           [total_tokens][num_q_heads][head_dim] bf16
 *   lse           [total_tokens][num_q_heads] fp32 or NULL
 * ------------------------------------------------------------------------- */
int prefill_attn(const void* q, const void* k, const void* v,
                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                 float scale, int32_t causal, void* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * extend_attn -- [ROCm] section "Processing details of the three paths",
 * extend path: (1) attention of the new tokens among themselves, (2) for each
 * chunk of the cached context, attention of all new tokens to the chunk,
 * (3) log-sum-exp merge of the partial results; section "ROCM_AITER_FA":
 * chunks follow a per-iteration context budget of about 32K tokens shared by
 * the extend requests.
 *   q             [total_new][num_q_heads][head_dim] bf16
 *   k_new, v_new  [total_new][num_kv_heads][head_dim] bf16 (this step's tokens)
 *   cu_q_lens     [num_seqs+1] int32 prefix sums of new-token counts
 *   ctx_lens      [num_seqs] int32 cached tokens before this step (>= 0)
 *   block_tables  [num_seqs][max_blocks_per_seq] int32 (cached context)
 *   max_q_len / max_ctx_len   host-side bounds
 *   chunk_budget_tokens       context tokens per iteration across all
 *                 requests; each request's chunk = budget / num_seqs rounded
 *                 down to a multiple of max(block_size, 64), the key tile
 *                 (at least one such unit).  The result does not depend on
 *                 the chunk size beyond fp32 rounding.
 *   out           [total_new][num_q_heads][head_dim] bf16
 *   lse           [total_new][num_q_heads] fp32 or NULL
 *   scale         softmax scale, finite and > 0 (else KV_EINVAL)
 *   workspace     >= extend_attn_workspace_bytes(...) bytes (0 in fused mode;
 *                 in automatic mode a smaller one forgoes the work list)
 * New token i of a request with C cached tokens sits at position C + i and
 * sees cached tokens 0..C-1 and new tokens 0..i.  Caches: NHD (any block
 * size) or preshuffled (block size 16), bf16 or fp8; the context is read in
 * place through the block table (fp8 codes decoded and scaled on the way, no
 * gather copy); the new tokens come from k_new / v_new (bf16).
 * Table capacity (max_blocks_per_seq * block_size) at most 2^30 tokens.
 *
 * Two executions of the same algorithm (they differ only in fp32 rounding):
 *  split  every (request, part) is its own work item: part 0 = the new tokens
 *         among themselves, part c >= 1 = all new tokens against context
 *         chunk c-1 (chunk = the request's share of the budget); each writes
 *         an fp32 (o, lse) partial to the workspace and a final pass merges
 *         them by log-sum-exp weights -- the pages' stages (1)-(3) literally,
 *         with the chunks run in parallel.
 *  fused  one workgroup walks the context chunks (the same key tiles in the
 *         same order) and then the new tokens with one running softmax
 *         state: the merge happens in registers and no workspace is used.
 * extend_attn picks fused when the new tokens alone fill the GPU (or there is
 * no context), else split; extend_attn_ex lets the caller choose.  A fused
 * pick whose longest context spans two or more chunks (at most 1024
 * requests) runs from a work list built on the GPU: every query item of the
 * batch, requests heaviest first, with the requests whose fused walk would
 * hold workgroups beyond half the batch's mean load per CU run split (their
 * chunks in parallel; at most 16 such requests and 64 MiB of fp32 partials)
 * and merged as above.  extend_attn_workspace_bytes then counts the plan, the
 * list and those partials; a smaller workspace runs plain fused.
 * ------------------------------------------------------------------------- */
size_t extend_attn_workspace_bytes(const kv_cache_t* cache, int32_t num_seqs,
                                   int32_t total_new_tokens, int32_t num_q_heads,
                                   int32_t max_ctx_len, int32_t chunk_budget_tokens);

typedef enum { KV_EXTEND_AUTO = 0, KV_EXTEND_SPLIT = 1, KV_EXTEND_FUSED = 2 } kv_extend_mode;
int extend_attn(const kv_cache_t* cache, const void* q, const void* k_new,
                const void* v_new, const int32_t* cu_q_lens, const int32_t* ctx_lens,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                int32_t num_seqs, int32_t total_new_tokens, int32_t max_q_len,
                int32_t max_ctx_len, int32_t num_q_heads, int32_t chunk_budget_tokens,
                float scale, void* out, float* lse, void* workspace,
                size_t workspace_bytes, void* stream);

/* Same call with the execution chosen by the caller (mode: kv_extend_mode);
 * the workspace query takes the same mode. */
size_t extend_attn_workspace_bytes_ex(const kv_cache_t* cache, int32_t num_seqs,
                                      int32_t total_new_tokens, int32_t num_q_heads,
                                      int32_t max_ctx_len, int32_t chunk_budget_tokens,
                                      int32_t mode);
int extend_attn_ex(const kv_cache_t* cache, const void* q, const void* k_new,
                   const void* v_new, const int32_t* cu_q_lens, const int32_t* ctx_lens,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   int32_t num_seqs, int32_t total_new_tokens, int32_t max_q_len,
                   int32_t max_ctx_len, int32_t num_q_heads, int32_t chunk_budget_tokens,
                   float scale, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, int32_t mode, void* stream);

/* ---------------------------------------------------------------------------
 * mla_decode -- [ROCm] section "AITER MLA backend: optimised for DeepSeek":
 * multi-head latent attention keeps one 576-dim latent row per token (about
 * 14x less than standard MHA) shared by every query head, and decodes
 * "absorbed", directly in that latent space; decode stays bound by memory
 * bandwidth.  The benchmark there runs with block size 16.
 *   kv_cache      [num_blocks][block_size][576] bf16: row = [c (512) | k_rope (64)]
 *   kv_dim, v_dim 576 and 512 (the only supported values): the score of
 *                 head h against token j is scale * <q_h, row_j> over all 576
 *                 dims, the value is the row's first 512 dims (the compressed
 *                 KV; the split is a reading of DeepSeek's published MLA)
 *   q             [batch][num_heads][576] bf16 (absorbed queries)
 *   block_tables  [batch][max_blocks_per_seq] int32
 *   seq_lens      [batch] int32 in [0, max_seq_len]; 0 gives out = 0, lse = -inf
 *   block_size    power of two in [16, 256]
 *   scale         finite and > 0
 *   out           [batch][num_heads][512] bf16 (the latent output; its
 *                 up-projection is part of the model, not of attention)
 *   lse           [batch][num_heads] fp32 or NULL
 *   workspace     >= mla_decode_workspace_bytes(...) bytes (plan + partials)
 * Balanced split-K over the concatenated token stream, as paged_decode.
 * ------------------------------------------------------------------------- */
size_t mla_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t max_seq_len);
int mla_decode(const void* kv_cache, int32_t num_blocks, int32_t block_size, int32_t kv_dim,
               int32_t v_dim, const void* q, int32_t batch, int32_t num_heads,
               const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* seq_lens, int32_t max_seq_len, float scale, void* out,
               float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Layer pack / unpack -- [PD] section "Architecture", write mode: after each
 * layer is computed the prefill side pushes that layer's KV blocks into
 * blocks preallocated on the decode side; the handshake exchanges the cache
 * base address, block size and per-layer stride.  [Guide] section
 * "Disaggregated architecture technical details": 320 KiB per token for a
 * 70B bf16 model.  These two calls are the on-GPU half of that push.
 *   block_ids  [n] int32 physical block ids (distinct for unpack)
 *   packed buffer: [K of ids[0]] ... [K of ids[n-1]] [V of ids[0]] ... [V of
 *   ids[n-1]], each block's bytes verbatim (one block of one layer is
 *   contiguous in both layouts), 16-byte aligned,
 *   kv_layer_packed_bytes(cache, n) = 2 * n * block_bytes.
 * ------------------------------------------------------------------------- */
size_t kv_layer_packed_bytes(const kv_cache_t* cache, int32_t num_block_ids);
int kv_pack_layer(const kv_cache_t* cache, const int32_t* block_ids, int32_t n,
                  void* dst, size_t dst_bytes, void* stream);
int kv_unpack_layer(const kv_cache_t* cache, const int32_t* block_ids, int32_t n,
                    const void* src, size_t src_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kv_reorder_batch -- HOST pointers.  [ROCm] section "ROCM_AITER_FA", batch
 * reorder: requests are reordered [decode : extend : prefill] before routing,
 * with reorder_batch_threshold = 1.  Request i is a decode if
 * query_lens[i] <= threshold, else an extend if ctx_lens[i] > 0, else a
 * prefill.  perm[j] = original index of the request placed at j (stable
 * within each class); counts[0..2] = (#decode, #extend, #prefill).
 * ------------------------------------------------------------------------- */
int kv_reorder_batch(const int32_t* query_lens, const int32_t* ctx_lens, int32_t n,
                     int32_t threshold, int32_t* perm, int32_t* counts);

/* Thread-local description of the last non-OK return (never NULL). */
const char* kv_last_error(void);
int kv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
