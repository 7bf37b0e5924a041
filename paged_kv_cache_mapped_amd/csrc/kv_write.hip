// Slot-mapped KV cache write for gfx950.
//
// "Beyond just running: native inference optimisation in vLLM on AMD ROCm",
// section "Unified attention backends": stage 1 of every forward writes the
// step's new key/value into the KV cache; section "Processing details of the
// three paths" (decode path): the store keeps the cache in the layout the
// decode kernel reads, so attention needs no conversion.  Token i goes to slot
// s = slot_mapping[i] = block * block_size + offset (s < 0: padding, skipped).
//
// One thread moves 8 consecutive (head, dim) elements of one token (one 16-byte
// bf16 load per tensor), so a token row of H_kv*D elements is read fully
// coalesced; where the destination layout keeps those 8 elements together
// (NHD, and K of the preshuffled layout) the store is one 16- or 8-byte store.
#include "common.h"
#include "internal.h"

namespace pkv {

// fp32 -> OCP E4M3 code ("e4m3fn": sign, 4 exponent bits biased by 7, 3
// mantissa bits, subnormals m/8 * 2^-6, no infinities, 0x7f = NaN), rounding
// half to even and saturating magnitudes >= 448 (including inf) to 448.
__device__ __forceinline__ uint32_t e4m3fn_rne_sat(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;      // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;     // >= 448: saturate
  if (a >= 0x3c800000u) {                         // >= 2^-6: normal
    const uint32_t e = (a >> 23) - 120u;         // 127-bias -> 7-bias
    const uint32_t keep = (a >> 20) & 7u;
    const uint32_t rem = a & 0xfffffu;           // 20 dropped mantissa bits
    uint32_t code = (e << 3) | keep;
    code += (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
    return sign | code;                           // a carry moves to the next binade
  }
  // subnormal range: value = k * 2^-9 with k = round-half-even(|y| * 2^9) <= 8
  const float t = __uint_as_float(a) * 512.0f;   // exact scaling
  return sign | (uint32_t)__builtin_rintf(t);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 8 bf16 (as 4 dwords) -> 8 fp8 codes (as 2 dwords) of fl32(x) * fl32(inv)
__device__ __forceinline__ u32x2_t quant8(u32x4_t x, float inv) {
  u32x2_t r = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = x[j >> 1];
    const uint32_t h = (j & 1) ? (w >> 16) : (w & 0xffffu);
    const float y = bf16_bits_to_f32(h) * inv;
    r[j >> 2] |= e4m3fn_rne_sat(y) << (8 * (j & 3));
  }
  return r;
}

template <int LAYOUT, int DT>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const u32x4_t* __restrict__ k, const u32x4_t* __restrict__ v,
    const int64_t* __restrict__ slots, int32_t num_tokens, int32_t H, int32_t D,
    int32_t bs, int64_t num_slots, float k_inv, float v_inv,
    void* __restrict__ kc, void* __restrict__ vc) {
  const int32_t per_tok = (H * D) >> 3;                 // 8-element groups per token
  const int64_t total = (int64_t)num_tokens * per_tok;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int32_t t = (int32_t)(idx / per_tok);
    const int32_t grp = (int32_t)(idx - (int64_t)t * per_tok);
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) continue;
    const u32x4_t kx = k[idx];
    const u32x4_t vx = v[idx];
    if constexpr (LAYOUT == KV_LAYOUT_NHD) {
      if constexpr (DT == KV_DTYPE_BF16) {
        ((u32x4_t*)kc)[s * per_tok + grp] = kx;
        ((u32x4_t*)vc)[s * per_tok + grp] = vx;
      } else {
        ((u32x2_t*)kc)[s * per_tok + grp] = quant8(kx, k_inv);
        ((u32x2_t*)vc)[s * per_tok + grp] = quant8(vx, v_inv);
      }
    } else {
      const int32_t e0 = grp << 3;                       // first of 8 elements
      const int32_t h = e0 / D, d0 = e0 - h * D;
      const int64_t blk = s / bs;
      const int32_t off = (int32_t)(s - blk * bs);
      const int64_t bh = blk * H + h;
      if constexpr (DT == KV_DTYPE_BF16) {
        constexpr int X = 8;
        // k[blk][h][d/X][off][d%X]: the 8 elements form one x-group
        uint16_t* kp = (uint16_t*)kc + ((bh * (D / X) + d0 / X) * bs + off) * X;
        *(u32x4_t*)kp = kx;
        // v[blk][h][off/X][d][off%X]: one element per d
        uint16_t* vp = (uint16_t*)vc + (bh * (bs / X) + off / X) * (int64_t)D * X + off % X;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w = vx[j >> 1];
          vp[(int64_t)(d0 + j) * X] = (uint16_t)((j & 1) ? (w >> 16) : (w & 0xffffu));
        }
      } else {
        constexpr int X = 16;
        uint8_t* kp = (uint8_t*)kc + ((bh * (D / X) + d0 / X) * bs + off) * X + (d0 % X);
        *(u32x2_t*)kp = quant8(kx, k_inv);
        const u32x2_t vq = quant8(vx, v_inv);
        uint8_t* vp = (uint8_t*)vc + (bh * (bs / X) + off / X) * (int64_t)D * X + off % X;
#pragma unroll
        for (int j = 0; j < 8; ++j) vp[(int64_t)(d0 + j) * X] = (uint8_t)(vq[j >> 2] >> (8 * (j & 3)));
      }
    }
  }
}

hipError_t launch_kv_write(const kv_cache_t& c, const void* k, const void* v,
                           const int64_t* slots, int32_t num_tokens, hipStream_t s) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t total = (int64_t)num_tokens * ((c.num_kv_heads * c.head_dim) >> 3);
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  const float k_inv = 1.0f / c.k_scale, v_inv = 1.0f / c.v_scale;
  const int64_t num_slots = (int64_t)c.num_blocks * c.block_size;
#define PKV_LAUNCH(L, T)                                                                    \
  hipLaunchKernelGGL((kv_write_kernel<L, T>), dim3((unsigned)blocks), dim3(threads), 0, s, \
                     (const u32x4_t*)k, (const u32x4_t*)v, slots, num_tokens,              \
                     c.num_kv_heads, c.head_dim, c.block_size, num_slots, k_inv, v_inv,    \
                     c.k_cache, c.v_cache)
  if (c.layout == KV_LAYOUT_NHD) {
    if (c.dtype == KV_DTYPE_BF16) PKV_LAUNCH(KV_LAYOUT_NHD, KV_DTYPE_BF16);
    else PKV_LAUNCH(KV_LAYOUT_NHD, KV_DTYPE_FP8_E4M3);
  } else {
    if (c.dtype == KV_DTYPE_BF16) PKV_LAUNCH(KV_LAYOUT_PRESHUFFLED, KV_DTYPE_BF16);
    else PKV_LAUNCH(KV_LAYOUT_PRESHUFFLED, KV_DTYPE_FP8_E4M3);
  }
#undef PKV_LAUNCH
  return hipGetLastError();
}

}  // namespace pkv
