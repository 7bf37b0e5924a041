// Host-side launchers of the gfx950 kernels (called by capi.cpp after the
// arguments have been validated).  Each returns hipSuccess or the launch error.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pagedkv.h"

namespace pkv {

// Compute units of the device that `stream` belongs to (the current device for
// the null stream; 256 on MI355X).  Host queries only, no synchronisation; the
// answer is cached per device.
inline int32_t device_cu_count(hipStream_t stream) {
  static int32_t cached[64] = {};
  int dev = 0;
  if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
    if (hipGetDevice(&dev) != hipSuccess) return 256;
  }
  if (dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cached[dev] = n;
  return n;
}

// ----------------------------------------------------------------- kv_write
hipError_t launch_kv_write(const kv_cache_t& c, const void* k, const void* v,
                           const int64_t* slots, int32_t num_tokens, hipStream_t s);

// ----------------------------------------------------------------- pack
hipError_t launch_pack(const kv_cache_t& c, const int32_t* ids, int32_t n, void* dst,
                       bool unpack, hipStream_t s);

// ----------------------------------------------------------------- decode
struct DecodePlan {
  int32_t split_tokens;      // fixed piece length requested by the caller (0 = automatic)
  int32_t n_gchunks;         // ceil(G / 16) groups of query heads per KV head
  int32_t fixed_len;         // piece length if fixed, else 0
  int32_t len_min, len_max;  // bounds of the automatic piece length
  int32_t pieces_per_group;  // grid x: workgroups along the token stream
  int32_t gpw;               // head groups per workgroup (1, 2, 4 or 8)
  int32_t target_pieces;     // pieces the automatic length aims at
  int32_t max_pieces;        // upper bound of the number of pieces
  int32_t part_rows;         // partial (o, lse) rows per query head: max_pieces + batch
};
DecodePlan plan_decode(const kv_cache_t& c, int32_t batch, int32_t num_q_heads,
                       int32_t max_seq_len, int32_t split_tokens, hipStream_t stream);
size_t decode_workspace_bytes(const DecodePlan& p, int32_t batch, int32_t num_q_heads,
                              int32_t head_dim);
// Size of the library's static decode scratch (paged_decode_noalloc).
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
void* decode_scratch(hipStream_t stream, hipError_t* err);
hipError_t launch_decode(const kv_cache_t& c, const DecodePlan& p, const void* q,
                         int32_t batch, int32_t num_q_heads, const int32_t* tables,
                         int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                         float scale, void* out, float* lse, void* workspace, hipStream_t s);

// ----------------------------------------------------------------- MLA decode
struct MlaPlan {
  int32_t n_gchunks;         // groups of up to 16 query heads
  int32_t waves;             // workers (4 per compute unit)
  int32_t target_pieces;     // pieces the automatic length aims at
  int32_t len_min, len_max;  // bounds of the piece length (tokens, multiple of 16)
  int32_t max_pieces;        // upper bound of the number of pieces
  int32_t part_rows;         // partial rows per head: max_pieces + batch
};
MlaPlan plan_mla(int32_t batch, int32_t num_heads, int32_t max_seq_len, hipStream_t stream);
size_t mla_workspace_bytes(const MlaPlan& p, int32_t batch, int32_t num_heads);
hipError_t launch_mla_decode(const MlaPlan& p, const void* cache, int32_t num_blocks,
                             int32_t block_size, const void* q, int32_t batch, int32_t num_heads,
                             const int32_t* tables, int32_t max_blocks, const int32_t* seq_lens,
                             int32_t max_seq_len, float scale, void* out, float* lse,
                             void* workspace, hipStream_t s);

// ----------------------------------------------------------------- prefill / extend
hipError_t launch_prefill(const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                          int32_t num_q_heads, int32_t num_kv_heads, float scale,
                          int32_t causal, void* out, float* lse, hipStream_t s);

struct ExtendPlan {
  int32_t chunk_tokens;   // cached tokens per chunk (multiple of block_size)
  int32_t n_chunks;       // context chunks of the longest context
  int32_t n_parts;        // n_chunks + 1 (the new-token part)
  int32_t fused;          // 1: one workgroup runs every part of its rows (no partials)
  // hybrid (automatic mode, fused plan, context over two or more chunks): a
  // device-side plan runs the requests whose walk would outlast the rest
  // split, in compact partial rows; 0 when the workspace is too small for it
  int32_t hybrid;
  int32_t max_split;      // requests that may run split
  int32_t cap_rows;       // compact partial rows
  int32_t list_cap;       // work-list entries
};
ExtendPlan plan_extend(const kv_cache_t& c, int32_t num_seqs, int32_t total_new,
                       int32_t num_q_heads, int32_t max_ctx_len, int32_t chunk_budget_tokens,
                       int32_t mode, hipStream_t stream);
size_t extend_workspace_bytes(const ExtendPlan& p, int32_t num_seqs, int32_t total_new,
                              int32_t num_q_heads, int32_t head_dim);
hipError_t launch_extend(const kv_cache_t& c, const ExtendPlan& p, const void* q,
                         const void* k_new, const void* v_new, const int32_t* cu_q_lens,
                         const int32_t* ctx_lens, const int32_t* tables, int32_t max_blocks,
                         int32_t num_seqs, int32_t total_new, int32_t max_q_len,
                         int32_t num_q_heads, float scale, void* out, float* lse,
                         void* workspace, hipStream_t s);

}  // namespace pkv
