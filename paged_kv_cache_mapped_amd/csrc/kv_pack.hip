// Layer-wise KV block pack / unpack for gfx950.
//
// "Advanced inference: why your single-node vLLM setup needs prefill/decode
// disaggregation", section "Architecture" (write mode): once a layer is
// computed, the prefill side pushes that layer's KV blocks straight into blocks
// preallocated on the decode side; the handshake shares the cache base address,
// block size and per-layer stride.  These kernels are the on-GPU part of that
// push: gather one layer's listed blocks into one contiguous buffer (what goes
// on the wire) and scatter such a buffer into (possibly different) blocks.
//
// Buffer: [K block ids[0]] .. [K block ids[n-1]] [V block ids[0]] .. [V block
// ids[n-1]], each block's bytes verbatim.  One block of one layer is a
// contiguous byte range in both cache layouts, so the copy is layout-agnostic.
//
// Pure HBM streaming: one workgroup per (block, K|V), 256 threads, each thread
// keeps eight 16-byte loads in flight before storing them.
#include "common.h"
#include "internal.h"

namespace pkv {

template <bool UNPACK>
__global__ __launch_bounds__(256) void pack_kernel(u32x4_t* __restrict__ kc, u32x4_t* __restrict__ vc,
                                                   const int32_t* __restrict__ ids, int32_t n,
                                                   int32_t num_blocks, int32_t cpb,
                                                   u32x4_t* __restrict__ buf) {
  const int32_t i = blockIdx.x;            // position in the id list
  const int32_t kv = blockIdx.y;           // 0: K, 1: V
  const int32_t id = ids[i];
  if (id < 0 || id >= num_blocks) return;  // out-of-range ids are skipped
  u32x4_t* cache = (kv == 0 ? kc : vc) + (int64_t)id * cpb;
  u32x4_t* packed = buf + ((int64_t)kv * n + i) * cpb;
  const u32x4_t* src = UNPACK ? packed : cache;
  u32x4_t* dst = UNPACK ? cache : packed;
  constexpr int U = 8;
  for (int32_t base = threadIdx.x; base < cpb; base += 256 * U) {
    u32x4_t r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t c = base + u * 256;
      if (c < cpb) r[u] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t c = base + u * 256;
      if (c < cpb) __builtin_nontemporal_store(r[u], dst + c);
    }
  }
}

hipError_t launch_pack(const kv_cache_t& c, const int32_t* ids, int32_t n, void* buf,
                       bool unpack, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t elem = c.dtype == KV_DTYPE_BF16 ? 2 : 1;
  const int64_t block_bytes = (int64_t)c.block_size * c.num_kv_heads * c.head_dim * elem;
  const int32_t cpb = (int32_t)(block_bytes / 16);
  dim3 grid((unsigned)n, 2);
  if (unpack)
    hipLaunchKernelGGL(pack_kernel<true>, grid, dim3(256), 0, s, (u32x4_t*)c.k_cache,
                       (u32x4_t*)c.v_cache, ids, n, c.num_blocks, cpb, (u32x4_t*)buf);
  else
    hipLaunchKernelGGL(pack_kernel<false>, grid, dim3(256), 0, s, (u32x4_t*)c.k_cache,
                       (u32x4_t*)c.v_cache, ids, n, c.num_blocks, cpb, (u32x4_t*)buf);
  return hipGetLastError();
}

}  // namespace pkv
