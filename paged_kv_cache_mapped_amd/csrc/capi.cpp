// C ABI of libpagedkv: host-side argument validation, workspace sizing and
// dispatch to the gfx950 launchers.  Nothing here allocates device memory or
// synchronises; every check happens before the first HIP call.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "internal.h"

namespace {

thread_local char g_err[512] = "no error";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KV_OK;
  return fail(KV_EHIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool pow2(int32_t v) { return v > 0 && (v & (v - 1)) == 0; }

int64_t elem_bytes(const kv_cache_t* c) { return c->dtype == KV_DTYPE_BF16 ? 2 : 1; }

// Shape / layout checks shared by every call that takes a cache.
int check_cache(const kv_cache_t* c, const char* fn) {
  if (!c) return fail(KV_EINVAL, "%s: cache descriptor is NULL", fn);
  if (!c->k_cache || !c->v_cache) return fail(KV_EINVAL, "%s: k_cache/v_cache is NULL", fn);
  if (!aligned16(c->k_cache) || !aligned16(c->v_cache))
    return fail(KV_EINVAL, "%s: cache pointers must be 16-byte aligned", fn);
  if (c->num_blocks <= 0) return fail(KV_EINVAL, "%s: num_blocks must be > 0", fn);
  if (c->num_kv_heads <= 0) return fail(KV_EINVAL, "%s: num_kv_heads must be > 0", fn);
  if (c->dtype != KV_DTYPE_BF16 && c->dtype != KV_DTYPE_FP8_E4M3)
    return fail(KV_EINVAL, "%s: unknown dtype %d", fn, c->dtype);
  if (c->layout != KV_LAYOUT_NHD && c->layout != KV_LAYOUT_PRESHUFFLED)
    return fail(KV_EINVAL, "%s: unknown layout %d", fn, c->layout);
  if (c->head_dim <= 0) return fail(KV_EINVAL, "%s: head_dim must be > 0", fn);
  if (c->head_dim != 128) return fail(KV_ENOTSUP, "%s: head_dim %d unsupported (128 only)", fn, c->head_dim);
  if (!pow2(c->block_size) || c->block_size > 256)
    return fail(KV_EINVAL, "%s: block_size %d must be a power of two in [1, 256]", fn, c->block_size);
  if (c->layout == KV_LAYOUT_PRESHUFFLED) {
    const int32_t want_x = (int32_t)(16 / elem_bytes(c));
    if (c->x != want_x)
      return fail(KV_EINVAL, "%s: preshuffled x must be 16 / element size = %d (got %d)", fn, want_x, c->x);
    if (c->block_size % c->x != 0)
      return fail(KV_EINVAL, "%s: preshuffled block_size %d must be a multiple of x = %d", fn,
                  c->block_size, c->x);
  }
  if (!(c->k_scale > 0.f) || !(c->v_scale > 0.f))
    return fail(KV_EINVAL, "%s: k_scale/v_scale must be > 0", fn);
  if (c->dtype == KV_DTYPE_BF16 && (c->k_scale != 1.f || c->v_scale != 1.f))
    return fail(KV_EINVAL, "%s: bf16 caches take k_scale = v_scale = 1", fn);
  const int64_t slots = (int64_t)c->num_blocks * c->block_size;
  if (slots * c->num_kv_heads * c->head_dim * elem_bytes(c) > ((int64_t)1 << 46))
    return fail(KV_EINVAL, "%s: cache larger than 64 TiB", fn);
  return KV_OK;
}

// Softmax scale of the attention calls: a finite positive number.  (The
// kernels take the running maximum of the raw scores and scale afterwards,
// which is the maximum of the scaled scores only for a positive scale.)
int check_scale(float scale, const char* fn) {
  if (!(scale > 0.f) || !(scale <= 3.4e38f))
    return fail(KV_EINVAL, "%s: scale must be finite and > 0 (got %g)", fn, (double)scale);
  return KV_OK;
}

int check_heads(const kv_cache_t* c, int32_t num_q_heads, const char* fn) {
  if (num_q_heads <= 0) return fail(KV_EINVAL, "%s: num_q_heads must be > 0", fn);
  if (num_q_heads % c->num_kv_heads != 0)
    return fail(KV_EINVAL, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", fn,
                num_q_heads, c->num_kv_heads);
  return KV_OK;
}

}  // namespace

extern "C" {

int kv_abi_version(void) { return PAGEDKV_ABI_VERSION; }

const char* kv_last_error(void) { return g_err; }

int kv_write(const kv_cache_t* cache, const void* k, const void* v,
             const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  int st = check_cache(cache, "kv_write");
  if (st) return st;
  if (num_tokens < 0) return fail(KV_EINVAL, "kv_write: num_tokens < 0");
  if (num_tokens == 0) return KV_OK;
  if (!k || !v || !slot_mapping) return fail(KV_EINVAL, "kv_write: k, v and slot_mapping must be non-NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(KV_EINVAL, "kv_write: k and v must be 16-byte aligned");
  return hip_status(pkv::launch_kv_write(*cache, k, v, slot_mapping, num_tokens, (hipStream_t)stream),
                    "kv_write");
}

static int decode_checks(const kv_cache_t* cache, int32_t batch, int32_t num_q_heads,
                         int32_t max_seq_len, int32_t split_tokens, const char* fn) {
  int st = check_cache(cache, fn);
  if (st) return st;
  st = check_heads(cache, num_q_heads, fn);
  if (st) return st;
  if (batch <= 0 || batch > 65535) return fail(KV_EINVAL, "%s: batch must be in [1, 65535]", fn);
  if (max_seq_len <= 0) return fail(KV_EINVAL, "%s: max_seq_len must be > 0", fn);
  if (split_tokens < 0 || split_tokens % 32 != 0 || split_tokens > 16384)
    return fail(KV_EINVAL, "%s: split_tokens must be 0 or a multiple of 32 up to 16384", fn);
  if ((num_q_heads / cache->num_kv_heads + 15) / 16 * cache->num_kv_heads > 65535)
    return fail(KV_EINVAL, "%s: too many heads", fn);
  if ((int64_t)batch * (((int64_t)max_seq_len + 31) & ~(int64_t)31) >= ((int64_t)1 << 31))
    return fail(KV_EINVAL, "%s: batch * max_seq_len must stay below 2^31", fn);
  return KV_OK;
}

size_t paged_decode_workspace_bytes_ex(const kv_cache_t* cache, int32_t batch,
                                       int32_t num_q_heads, int32_t max_seq_len,
                                       int32_t split_tokens) {
  if (decode_checks(cache, batch, num_q_heads, max_seq_len, split_tokens, "paged_decode_workspace_bytes"))
    return 0;
  const pkv::DecodePlan p =
      pkv::plan_decode(*cache, batch, num_q_heads, max_seq_len, split_tokens, nullptr);
  return pkv::decode_workspace_bytes(p, batch, num_q_heads, cache->head_dim);
}

size_t paged_decode_workspace_bytes(const kv_cache_t* cache, int32_t batch, int32_t num_q_heads,
                                    int32_t max_seq_len) {
  return paged_decode_workspace_bytes_ex(cache, batch, num_q_heads, max_seq_len, 0);
}

// Every check of a decode call that does not involve the workspace.
static int decode_call_checks(const kv_cache_t* cache, const void* q, int32_t batch,
                              int32_t num_q_heads, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              int32_t max_seq_len, float scale, const void* out,
                              int32_t split_tokens, const char* fn) {
  int st = decode_checks(cache, batch, num_q_heads, max_seq_len, split_tokens, fn);
  if (st) return st;
  if (!q || !block_tables || !seq_lens || !out)
    return fail(KV_EINVAL, "%s: q, block_tables, seq_lens and out must be non-NULL", fn);
  if (!aligned16(q) || !aligned16(out)) return fail(KV_EINVAL, "%s: q and out must be 16-byte aligned", fn);
  if (max_blocks_per_seq <= 0) return fail(KV_EINVAL, "%s: max_blocks_per_seq must be > 0", fn);
  if ((int64_t)max_blocks_per_seq * cache->block_size < max_seq_len)
    return fail(KV_EINVAL, "%s: max_seq_len %d exceeds the table capacity %lld", fn, max_seq_len,
                (long long)max_blocks_per_seq * cache->block_size);
  if ((int64_t)max_blocks_per_seq * cache->block_size > (int64_t)1 << 30)
    return fail(KV_EINVAL, "%s: table capacity above 2^30 tokens", fn);
  return check_scale(scale, fn);
}

static int decode_launch(const kv_cache_t* cache, const pkv::DecodePlan& p, const void* q,
                         int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                         float scale, void* out, float* lse, void* workspace, void* stream,
                         const char* fn) {
  return hip_status(pkv::launch_decode(*cache, p, q, batch, num_q_heads, block_tables,
                                       max_blocks_per_seq, seq_lens, max_seq_len, scale, out, lse,
                                       workspace, (hipStream_t)stream),
                    fn);
}

int paged_decode_ex(const kv_cache_t* cache, const void* q, int32_t batch, int32_t num_q_heads,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t max_seq_len, float scale, void* out,
                    float* lse, void* workspace, size_t workspace_bytes, int32_t split_tokens,
                    void* stream) {
  const char* fn = "paged_decode";
  int st = decode_call_checks(cache, q, batch, num_q_heads, block_tables, max_blocks_per_seq,
                              seq_lens, max_seq_len, scale, out, split_tokens, fn);
  if (st) return st;
  const pkv::DecodePlan p = pkv::plan_decode(*cache, batch, num_q_heads, max_seq_len, split_tokens,
                                             (hipStream_t)stream);
  const size_t need = pkv::decode_workspace_bytes(p, batch, num_q_heads, cache->head_dim);
  if (!workspace) return fail(KV_EINVAL, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (workspace_bytes < need)
    return fail(KV_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  if (!aligned16(workspace)) return fail(KV_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  return decode_launch(cache, p, q, batch, num_q_heads, block_tables, max_blocks_per_seq, seq_lens,
                       max_seq_len, scale, out, lse, workspace, stream, fn);
}

int paged_decode(const kv_cache_t* cache, const void* q, int32_t batch, int32_t num_q_heads,
                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                 int32_t max_seq_len, float scale, void* out, float* lse, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return paged_decode_ex(cache, q, batch, num_q_heads, block_tables, max_blocks_per_seq, seq_lens,
                         max_seq_len, scale, out, lse, workspace, workspace_bytes, 0, stream);
}

int paged_decode_noalloc(const kv_cache_t* cache, const void* q, int32_t batch,
                         int32_t num_q_heads, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                         float scale, void* out, float* lse, void* stream) {
  const char* fn = "paged_decode_noalloc";
  int st = decode_call_checks(cache, q, batch, num_q_heads, block_tables, max_blocks_per_seq,
                              seq_lens, max_seq_len, scale, out, 0, fn);
  if (st) return st;
  const pkv::DecodePlan p =
      pkv::plan_decode(*cache, batch, num_q_heads, max_seq_len, 0, (hipStream_t)stream);
  const size_t need = pkv::decode_workspace_bytes(p, batch, num_q_heads, cache->head_dim);
  if (need > pkv::kDecodeScratchBytes)
    return fail(KV_ENOSPC,
                "%s: this batch needs %zu bytes of decode scratch, more than the library's "
                "%zu; use paged_decode with a caller workspace",
                fn, need, pkv::kDecodeScratchBytes);
  hipError_t e;
  void* ws = pkv::decode_scratch((hipStream_t)stream, &e);
  if (!ws) return hip_status(e == hipSuccess ? hipErrorUnknown : e, fn);
  return decode_launch(cache, p, q, batch, num_q_heads, block_tables, max_blocks_per_seq, seq_lens,
                       max_seq_len, scale, out, lse, ws, stream, fn);
}

int prefill_attn(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                 int32_t num_seqs, int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                 int32_t head_dim, float scale, int32_t causal, void* out, float* lse,
                 void* stream) {
  const char* fn = "prefill_attn";
  if (num_seqs < 0) return fail(KV_EINVAL, "%s: num_seqs < 0", fn);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(KV_EINVAL, "%s: num_q_heads must be a positive multiple of num_kv_heads", fn);
  if (head_dim != 128) return fail(KV_ENOTSUP, "%s: head_dim %d unsupported (128 only)", fn, head_dim);
  if (causal != 0 && causal != 1) return fail(KV_EINVAL, "%s: causal must be 0 or 1", fn);
  if (max_seqlen < 0) return fail(KV_EINVAL, "%s: max_seqlen < 0", fn);
  int st = check_scale(scale, fn);
  if (st) return st;
  if (num_seqs == 0 || max_seqlen == 0) return KV_OK;
  if (!q || !k || !v || !cu_seqlens || !out)
    return fail(KV_EINVAL, "%s: q, k, v, cu_seqlens and out must be non-NULL", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(KV_EINVAL, "%s: q, k, v and out must be 16-byte aligned", fn);
  if (num_q_heads > 65535 || num_seqs > 65535) return fail(KV_EINVAL, "%s: grid too large", fn);
  return hip_status(pkv::launch_prefill(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_q_heads,
                                        num_kv_heads, scale, causal, out, lse, (hipStream_t)stream),
                    fn);
}

static int extend_checks(const kv_cache_t* cache, int32_t num_seqs, int32_t total_new,
                         int32_t num_q_heads, int32_t max_ctx_len, int32_t budget, int32_t mode,
                         const char* fn) {
  int st = check_cache(cache, fn);
  if (st) return st;
  st = check_heads(cache, num_q_heads, fn);
  if (st) return st;
  if (cache->layout == KV_LAYOUT_PRESHUFFLED && cache->block_size != 16)
    return fail(KV_ENOTSUP, "%s: the extend path reads preshuffled caches of block size 16", fn);
  if (num_seqs < 0 || total_new < 0 || max_ctx_len < 0)
    return fail(KV_EINVAL, "%s: negative size", fn);
  if (budget <= 0) return fail(KV_EINVAL, "%s: chunk_budget_tokens must be > 0", fn);
  if (mode < KV_EXTEND_AUTO || mode > KV_EXTEND_FUSED)
    return fail(KV_EINVAL, "%s: unknown mode %d", fn, mode);
  return KV_OK;
}

size_t extend_attn_workspace_bytes_ex(const kv_cache_t* cache, int32_t num_seqs, int32_t total_new,
                                      int32_t num_q_heads, int32_t max_ctx_len, int32_t budget,
                                      int32_t mode) {
  if (extend_checks(cache, num_seqs, total_new, num_q_heads, max_ctx_len, budget, mode,
                    "extend_attn_workspace_bytes"))
    return 0;
  const pkv::ExtendPlan p =
      pkv::plan_extend(*cache, num_seqs, total_new, num_q_heads, max_ctx_len, budget, mode, nullptr);
  return pkv::extend_workspace_bytes(p, num_seqs, total_new, num_q_heads, cache->head_dim);
}

size_t extend_attn_workspace_bytes(const kv_cache_t* cache, int32_t num_seqs, int32_t total_new,
                                   int32_t num_q_heads, int32_t max_ctx_len, int32_t budget) {
  return extend_attn_workspace_bytes_ex(cache, num_seqs, total_new, num_q_heads, max_ctx_len,
                                        budget, KV_EXTEND_AUTO);
}

int extend_attn_ex(const kv_cache_t* cache, const void* q, const void* k_new, const void* v_new,
                   const int32_t* cu_q_lens, const int32_t* ctx_lens, const int32_t* block_tables,
                   int32_t max_blocks_per_seq, int32_t num_seqs, int32_t total_new,
                   int32_t max_q_len, int32_t max_ctx_len, int32_t num_q_heads, int32_t budget,
                   float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                   int32_t mode, void* stream) {
  const char* fn = "extend_attn";
  int st = extend_checks(cache, num_seqs, total_new, num_q_heads, max_ctx_len, budget, mode, fn);
  if (st) return st;
  if (max_q_len < 0) return fail(KV_EINVAL, "%s: max_q_len < 0", fn);
  st = check_scale(scale, fn);
  if (st) return st;
  if (num_seqs == 0 || total_new == 0 || max_q_len == 0) return KV_OK;
  if (!q || !k_new || !v_new || !cu_q_lens || !ctx_lens || !out)
    return fail(KV_EINVAL, "%s: q, k_new, v_new, cu_q_lens, ctx_lens and out must be non-NULL", fn);
  if (max_ctx_len > 0 && (!block_tables || max_blocks_per_seq <= 0))
    return fail(KV_EINVAL, "%s: block_tables needed when max_ctx_len > 0", fn);
  if (max_ctx_len > 0 && (int64_t)max_blocks_per_seq * cache->block_size < max_ctx_len)
    return fail(KV_EINVAL, "%s: max_ctx_len %d exceeds the table capacity", fn, max_ctx_len);
  if ((int64_t)max_blocks_per_seq * cache->block_size > (int64_t)1 << 30)
    return fail(KV_EINVAL, "%s: table capacity above 2^30 tokens", fn);
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return fail(KV_EINVAL, "%s: q, k_new, v_new and out must be 16-byte aligned", fn);
  if (num_q_heads > 65535 || num_seqs > 65535) return fail(KV_EINVAL, "%s: grid too large", fn);
  pkv::ExtendPlan p = pkv::plan_extend(*cache, num_seqs, total_new, num_q_heads, max_ctx_len,
                                       budget, mode, (hipStream_t)stream);
  size_t need = pkv::extend_workspace_bytes(p, num_seqs, total_new, num_q_heads, cache->head_dim);
  if (p.hybrid && (!workspace || workspace_bytes < need || !aligned16(workspace))) {
    p.hybrid = 0;                 // no room for the hybrid plan: plain fused
    need = 0;
  }
  if (need > 0) {
    if (!workspace) return fail(KV_EINVAL, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (workspace_bytes < need)
      return fail(KV_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
    if (!aligned16(workspace)) return fail(KV_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  }
  return hip_status(pkv::launch_extend(*cache, p, q, k_new, v_new, cu_q_lens, ctx_lens,
                                       block_tables, max_blocks_per_seq, num_seqs, total_new,
                                       max_q_len, num_q_heads, scale, out, lse, workspace,
                                       (hipStream_t)stream),
                    fn);
}

int extend_attn(const kv_cache_t* cache, const void* q, const void* k_new, const void* v_new,
                const int32_t* cu_q_lens, const int32_t* ctx_lens, const int32_t* block_tables,
                int32_t max_blocks_per_seq, int32_t num_seqs, int32_t total_new, int32_t max_q_len,
                int32_t max_ctx_len, int32_t num_q_heads, int32_t budget, float scale, void* out,
                float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return extend_attn_ex(cache, q, k_new, v_new, cu_q_lens, ctx_lens, block_tables,
                        max_blocks_per_seq, num_seqs, total_new, max_q_len, max_ctx_len,
                        num_q_heads, budget, scale, out, lse, workspace, workspace_bytes,
                        KV_EXTEND_AUTO, stream);
}

static int mla_checks(int32_t num_blocks, int32_t block_size, int32_t kv_dim, int32_t v_dim,
                      int32_t batch, int32_t num_heads, int32_t max_seq_len, const char* fn) {
  if (kv_dim != 576 || v_dim != 512)
    return fail(KV_ENOTSUP, "%s: latent rows of 576 dims with a 512-dim value part only (got %d, %d)",
                fn, kv_dim, v_dim);
  if (num_blocks <= 0) return fail(KV_EINVAL, "%s: num_blocks must be > 0", fn);
  if (!pow2(block_size) || block_size > 256)
    return fail(KV_EINVAL, "%s: block_size %d must be a power of two in [1, 256]", fn, block_size);
  if (block_size < 16)
    return fail(KV_ENOTSUP, "%s: block_size %d below the 16-token tile", fn, block_size);
  if (batch <= 0 || batch > 65535) return fail(KV_EINVAL, "%s: batch must be in [1, 65535]", fn);
  if (num_heads <= 0 || num_heads > 4096) return fail(KV_EINVAL, "%s: num_heads must be in [1, 4096]", fn);
  if (max_seq_len <= 0) return fail(KV_EINVAL, "%s: max_seq_len must be > 0", fn);
  if ((int64_t)batch * (((int64_t)max_seq_len + 15) & ~(int64_t)15) >= ((int64_t)1 << 31))
    return fail(KV_EINVAL, "%s: batch * max_seq_len must stay below 2^31", fn);
  if ((int64_t)num_blocks * block_size * 1152 > ((int64_t)1 << 46))
    return fail(KV_EINVAL, "%s: cache larger than 64 TiB", fn);
  return KV_OK;
}

size_t mla_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t max_seq_len) {
  if (mla_checks(1, 16, 576, 512, batch, num_heads, max_seq_len, "mla_decode_workspace_bytes"))
    return 0;
  const pkv::MlaPlan p = pkv::plan_mla(batch, num_heads, max_seq_len, nullptr);
  return pkv::mla_workspace_bytes(p, batch, num_heads);
}

int mla_decode(const void* kv_cache, int32_t num_blocks, int32_t block_size, int32_t kv_dim,
               int32_t v_dim, const void* q, int32_t batch, int32_t num_heads,
               const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
               int32_t max_seq_len, float scale, void* out, float* lse, void* workspace,
               size_t workspace_bytes, void* stream) {
  const char* fn = "mla_decode";
  int st = mla_checks(num_blocks, block_size, kv_dim, v_dim, batch, num_heads, max_seq_len, fn);
  if (st) return st;
  if (!kv_cache || !q || !block_tables || !seq_lens || !out)
    return fail(KV_EINVAL, "%s: kv_cache, q, block_tables, seq_lens and out must be non-NULL", fn);
  if (!aligned16(kv_cache) || !aligned16(q) || !aligned16(out))
    return fail(KV_EINVAL, "%s: kv_cache, q and out must be 16-byte aligned", fn);
  if (max_blocks_per_seq <= 0) return fail(KV_EINVAL, "%s: max_blocks_per_seq must be > 0", fn);
  if ((int64_t)max_blocks_per_seq * block_size < max_seq_len)
    return fail(KV_EINVAL, "%s: max_seq_len %d exceeds the table capacity %lld", fn, max_seq_len,
                (long long)max_blocks_per_seq * block_size);
  if ((int64_t)max_blocks_per_seq * block_size > (int64_t)1 << 30)
    return fail(KV_EINVAL, "%s: table capacity above 2^30 tokens", fn);
  st = check_scale(scale, fn);
  if (st) return st;
  const pkv::MlaPlan p = pkv::plan_mla(batch, num_heads, max_seq_len, (hipStream_t)stream);
  const size_t need = pkv::mla_workspace_bytes(p, batch, num_heads);
  if (!workspace) return fail(KV_EINVAL, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (workspace_bytes < need)
    return fail(KV_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  if (!aligned16(workspace)) return fail(KV_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  return hip_status(pkv::launch_mla_decode(p, kv_cache, num_blocks, block_size, q, batch,
                                           num_heads, block_tables, max_blocks_per_seq, seq_lens,
                                           max_seq_len, scale, out, lse, workspace,
                                           (hipStream_t)stream),
                    fn);
}

size_t kv_layer_packed_bytes(const kv_cache_t* cache, int32_t n) {
  if (check_cache(cache, "kv_layer_packed_bytes") || n < 0) return 0;
  return (size_t)2 * n * cache->block_size * cache->num_kv_heads * cache->head_dim * elem_bytes(cache);
}

static int pack_common(const kv_cache_t* cache, const int32_t* ids, int32_t n, const void* buf,
                       size_t bytes, bool unpack, void* stream) {
  const char* fn = unpack ? "kv_unpack_layer" : "kv_pack_layer";
  int st = check_cache(cache, fn);
  if (st) return st;
  if (n < 0) return fail(KV_EINVAL, "%s: n < 0", fn);
  if (n == 0) return KV_OK;
  if (n > 2147483647 / 2) return fail(KV_EINVAL, "%s: n too large", fn);
  if (!ids || !buf) return fail(KV_EINVAL, "%s: block_ids and the buffer must be non-NULL", fn);
  if (!aligned16(buf)) return fail(KV_EINVAL, "%s: buffer must be 16-byte aligned", fn);
  const size_t need = kv_layer_packed_bytes(cache, n);
  if (bytes < need) return fail(KV_ENOSPC, "%s: buffer %zu bytes < %zu needed", fn, bytes, need);
  return hip_status(pkv::launch_pack(*cache, ids, n, (void*)buf, unpack, (hipStream_t)stream), fn);
}

int kv_pack_layer(const kv_cache_t* cache, const int32_t* block_ids, int32_t n, void* dst,
                  size_t dst_bytes, void* stream) {
  return pack_common(cache, block_ids, n, dst, dst_bytes, false, stream);
}

int kv_unpack_layer(const kv_cache_t* cache, const int32_t* block_ids, int32_t n, const void* src,
                    size_t src_bytes, void* stream) {
  return pack_common(cache, block_ids, n, src, src_bytes, true, stream);
}

int kv_reorder_batch(const int32_t* query_lens, const int32_t* ctx_lens, int32_t n,
                     int32_t threshold, int32_t* perm, int32_t* counts) {
  const char* fn = "kv_reorder_batch";
  if (n < 0) return fail(KV_EINVAL, "%s: n < 0", fn);
  if (!counts) return fail(KV_EINVAL, "%s: counts is NULL", fn);
  if (n > 0 && (!query_lens || !ctx_lens || !perm))
    return fail(KV_EINVAL, "%s: query_lens, ctx_lens and perm must be non-NULL", fn);
  // three stable passes: decode, extend, prefill
  int32_t pos = 0;
  for (int cls = 0; cls < 3; ++cls) {
    int32_t cnt = 0;
    for (int32_t i = 0; i < n; ++i) {
      if (query_lens[i] < 0 || ctx_lens[i] < 0) return fail(KV_EINVAL, "%s: negative length at %d", fn, i);
      const int c = query_lens[i] <= threshold ? 0 : (ctx_lens[i] > 0 ? 1 : 2);
      if (c == cls) {
        perm[pos++] = i;
        ++cnt;
      }
    }
    counts[cls] = cnt;
  }
  return KV_OK;
}

}  // extern "C"
