// Paged decode attention for gfx950: split-K over the block table, then a
// log-sum-exp combine of the splits.
//
// "Beyond just running: native inference optimisation in vLLM on AMD ROCm",
// section "Every batch handles a mixed workload": a decode request produces one
// token and has to stream its whole KV cache, so this path is bound by HBM
// bandwidth and wants contiguous accesses and few cache reads.  Section
// "Processing details of the three paths": partial results carry an LSE (the
// log of the softmax denominator) so they merge exactly and stably.
// "From LLM performance optimisation to DeepSeek deployment", section 3 "Paged
// Attention": logical block i of a request lives in physical block table[i].
//
// Work split.  One workgroup (4 waves) owns (request b, KV head, group of up to
// 16 query heads sharing it, token range of split_tokens).  Its waves take
// interleaved 32-token tiles of the range.  Per tile a wave:
//   * loads K rows straight into MFMA A-operand registers (16-byte loads),
//   * computes S^T = K Q^T for its query-head group with v_mfma_f32_16x16x32_bf16
//     (query heads are the 16 MFMA columns; grouped-query decode is a dense
//     contraction with G rows),
//   * runs the online softmax in registers (per query head: max / sum over the
//     4 lanes holding its 32 scores via cross-lane shuffles),
//   * accumulates O^T = V^T P^T with V^T as the A operand.  In the NHD layout V
//     rows are staged in LDS with 16-byte coalesced stores and read back
//     transposed with ds_read_b64_tr_b16; in the preshuffled layout V is
//     already stored token-minor ([block][head][bs/x][D][x]) and is loaded
//     straight into registers.
// The 4 waves merge their (m, l, O) in LDS; the workgroup writes either the
// final output (single-split request) or an fp32 partial (o, lse) that a
// second kernel merges with LSE weights.
//
// fp8 (OCP e4m3fn) caches are decoded to bf16 in registers (exact) and the
// per-tensor scales are applied to the scores (k_scale) and to the output
// (v_scale): <q, c*ks> = ks <q, c>, sum p (c*vs) = vs sum p c.
#include "common.h"
#include "internal.h"

namespace pkv {
namespace {

constexpr int kD = 128;
constexpr int kTile = 32;
constexpr int kWaves = 4;
constexpr int kVRowBytes = 288;                  // 128 bf16 + 32 B pad (bank spread)
constexpr int kVTileBytes = kTile * kVRowBytes;  // per wave; also holds 16x128 fp32 at the end
constexpr float kNegInf = -__builtin_huge_valf();

struct DecodeArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const __bf16* q;
  const int32_t* tables;
  const int32_t* seq_lens;
  __bf16* out;
  float* lse;
  float* part_o;
  float* part_lse;
  int32_t max_blocks, num_blocks, bs, bs_log2, Hkv, Hq, G, n_gchunks;
  int32_t split_tokens, n_splits, batch;
  float qk_mult;   // scale * k_scale * log2(e): scores in the exp2 domain
  float v_scale;
};

__device__ __forceinline__ int32_t clamp_block(int32_t blk, int32_t nb) {
  return blk < 0 ? 0 : (blk >= nb ? nb - 1 : blk);
}

// Query dims held by lane quarter q4 for MFMA k-step kk.  bf16 caches use the
// natural order; fp8 caches hand each lane 16 consecutive dims per load, i.e.
// k-steps 2p and 2p+1 read one 16-dim chunk 4p + q4.
template <int DT>
__device__ __forceinline__ int dmap(int kk, int q4) {
  if constexpr (DT == KV_DTYPE_BF16) return 32 * kk + 8 * q4;
  else return 64 * (kk >> 1) + 16 * q4 + 8 * (kk & 1);
}

template <int LAYOUT, int DT>
__device__ __forceinline__ void load_k(const DecodeArgs& a, const int32_t* trow, int hkv,
                                       int32_t tok, int q4, bf16x8_t (&ka)[4]) {
  const int32_t blk = clamp_block(trow[tok >> a.bs_log2], a.num_blocks);
  const int32_t off = tok & (a.bs - 1);
  if constexpr (LAYOUT == KV_LAYOUT_NHD) {
    const int64_t row = ((int64_t)blk * a.bs + off) * a.Hkv + hkv;
    if constexpr (DT == KV_DTYPE_BF16) {
      const uint8_t* p = a.kc + row * (kD * 2);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ka[kk] = *(const bf16x8_t*)(p + dmap<DT>(kk, q4) * 2);
    } else {
      const uint8_t* p = a.kc + row * kD;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const u32x4_t w = *(const u32x4_t*)(p + 16 * (4 * pp + q4));
        ka[2 * pp] = fp8x8_to_bf16(u32x2_t{w[0], w[1]});
        ka[2 * pp + 1] = fp8x8_to_bf16(u32x2_t{w[2], w[3]});
      }
    }
  } else {
    const int64_t bh = (int64_t)blk * a.Hkv + hkv;
    if constexpr (DT == KV_DTYPE_BF16) {   // [blk][h][D/8][bs][8]
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int64_t e = ((bh * (kD / 8) + (4 * kk + q4)) * a.bs + off) * 8;
        ka[kk] = *(const bf16x8_t*)(a.kc + e * 2);
      }
    } else {                                // [blk][h][D/16][bs][16]
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int64_t e = ((bh * (kD / 16) + (4 * pp + q4)) * a.bs + off) * 16;
        const u32x4_t w = *(const u32x4_t*)(a.kc + e);
        ka[2 * pp] = fp8x8_to_bf16(u32x2_t{w[0], w[1]});
        ka[2 * pp + 1] = fp8x8_to_bf16(u32x2_t{w[2], w[3]});
      }
    }
  }
}

template <int LAYOUT, int DT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(3)))
void decode_split_kernel(DecodeArgs a) {
  const int32_t split = blockIdx.x;
  const int32_t b = blockIdx.z;
  const int32_t hkv = blockIdx.y / a.n_gchunks;
  const int32_t gc = blockIdx.y - hkv * a.n_gchunks;
  int32_t L = a.seq_lens[b];
  const int32_t cap = a.max_blocks << a.bs_log2;
  L = L > cap ? cap : L;
  const int32_t t_begin = split * a.split_tokens;
  if (t_begin >= L) return;                 // uniform over the workgroup
  const int32_t t_end = min(L, t_begin + a.split_tokens);
  const int32_t n_b = (L + a.split_tokens - 1) / a.split_tokens;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q4 = lane >> 4, r = lane & 15;
  const int g0 = gc * 16;
  const int gcnt = min(16, a.G - g0);
  const int32_t h_base = hkv * a.G + g0;

  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves * kVTileBytes];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  uint8_t* vt = smem + wave * kVTileBytes;

  // Q^T as the B operand: lane (q4, r) holds q[h_base + r][dmap(kk, q4) .. +8]
  bf16x8_t qb[4];
  {
    const bf16x8_t zero = {};
    const __bf16* qrow = a.q + ((int64_t)b * a.Hq + h_base + r) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qb[kk] = (r < gcnt) ? *(const bf16x8_t*)(qrow + dmap<DT>(kk, q4)) : zero;
  }

  const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
  f32x4_t o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const int32_t n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  for (int32_t it = wave; it < n_tiles; it += kWaves) {
    const int32_t t0 = t_begin + it * kTile;
    const bool partial = t0 + kTile > t_end;

    // ---- K: A operand rows = tokens t0 + 8*(r/4) + 4*s + r%4 (subtile s)
    bf16x8_t ka[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int32_t tok = min(t0 + 8 * (r >> 2) + 4 * s + (r & 3), t_end - 1);
      load_k<LAYOUT, DT>(a, trow, hkv, tok, q4, ka[s]);
    }

    // ---- V: NHD rows go through LDS; preshuffled V is loaded as V^T directly
    bf16x8_t va[8];
    if constexpr (LAYOUT == KV_LAYOUT_NHD) {
      const int a4 = lane >> 4, c16 = lane & 15;
#pragma unroll
      for (int j4 = 0; j4 < 8; ++j4) {
        const int j = 4 * j4 + a4;
        const int32_t tok = min(t0 + j, t_end - 1);
        const int32_t blk = clamp_block(trow[tok >> a.bs_log2], a.num_blocks);
        const int64_t row = ((int64_t)blk * a.bs + (tok & (a.bs - 1))) * a.Hkv + hkv;
        u32x4_t w;
        if constexpr (DT == KV_DTYPE_BF16) {
          w = *(const u32x4_t*)(a.vc + row * (kD * 2) + c16 * 16);
        } else {
          const u32x2_t c = *(const u32x2_t*)(a.vc + row * kD + c16 * 8);
          w = __builtin_bit_cast(u32x4_t, fp8x8_to_bf16(c));
        }
        *(u32x4_t*)(vt + j * kVRowBytes + c16 * 16) = w;
      }
    } else {
      constexpr int X = (DT == KV_DTYPE_BF16) ? 8 : 16;
      const int32_t tv = t0 + 8 * q4;                        // 8 tokens, aligned to 8
      const int32_t tb = min(tv, (t_end - 1) & ~7);
      const int32_t blk = clamp_block(trow[tb >> a.bs_log2], a.num_blocks);
      const int32_t off = tb & (a.bs - 1);
      const int64_t base = (((int64_t)blk * a.Hkv + hkv) * (a.bs / X) + off / X) * kD;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int64_t e = (base + 16 * n + r) * X + (off % X);
        if constexpr (DT == KV_DTYPE_BF16) va[n] = *(const bf16x8_t*)(a.vc + e * 2);
        else va[n] = fp8x8_to_bf16(*(const u32x2_t*)(a.vc + e));
      }
      if (partial) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (tv + jj >= t_end) {
#pragma unroll
            for (int n = 0; n < 8; ++n) va[n][jj] = (__bf16)0.f;
          }
      }
    }

    // ---- S^T = K Q^T: element i of acc[s] is token t0 + 8*q4 + 4*s + i, head r
    f32x4_t acc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc[s] = mfma16(ka[s][kk], qb[kk], acc[s]);
    }
    float sc[8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t tok = t0 + 8 * q4 + 4 * s + i;
        sc[4 * s + i] = (partial && tok >= t_end) ? kNegInf : acc[s][i] * a.qk_mult;
      }

    // ---- online softmax for query head r (exp2 domain)
    float mt = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sc[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);    // finite: every tile has a valid token
    const float alpha = fast_exp2(m_run - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = fast_exp2(sc[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;            // lane-partial; reduced at the end
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] *= alpha;
    const bf16x8_t pb = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                         (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};

    // ---- O^T += V^T P^T: element i of o[n] is dim 16n + 4*q4 + i, head r
    if constexpr (LAYOUT == KV_LAYOUT_NHD) {
      order_lds();
      const int row0 = 8 * q4 + (r >> 2);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int colb = (16 * n + 4 * (r & 3)) * 2;
        const s16x4_t lo = lds_read_tr16(vt + row0 * kVRowBytes + colb);
        const s16x4_t hi = lds_read_tr16(vt + (row0 + 4) * kVRowBytes + colb);
        o[n] = mfma16(cat_tr(lo, hi), pb, o[n]);
      }
      order_lds();
    } else {
#pragma unroll
      for (int n = 0; n < 8; ++n) o[n] = mfma16(va[n], pb, o[n]);
    }
  }

  // ---- merge the 4 waves
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (q4 == 0) {
    sm_m[wave][r] = m_run;
    sm_l[wave][r] = l_run;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
  float Lt = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = sm_m[w][r];
    Lt += (mw == kNegInf) ? 0.f : sm_l[w][r] * fast_exp2(mw - M);
  }
  const float f = (m_run == kNegInf || !(Lt > 0.f)) ? 0.f : fast_exp2(m_run - M) / Lt;
  float* ob = (float*)vt;                    // [16 heads][128 dims] fp32
#pragma unroll
  for (int n = 0; n < 8; ++n) *(f32x4_t*)(ob + r * kD + 16 * n + 4 * q4) = o[n] * f;
  __syncthreads();

  const bool final_out = (n_b == 1);
  for (int idx = threadIdx.x; idx < gcnt * (kD / 4); idx += 256) {
    const int g = idx / (kD / 4), d4 = idx - g * (kD / 4);
    f32x4_t s4 = *(const f32x4_t*)((const float*)smem + g * kD + 4 * d4);
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
      s4 += *(const f32x4_t*)((const float*)(smem + w * kVTileBytes) + g * kD + 4 * d4);
    s4 *= a.v_scale;
    const int64_t bh = (int64_t)b * a.Hq + h_base + g;
    if (final_out) {
      const bf16x4_t v4 = {(__bf16)s4[0], (__bf16)s4[1], (__bf16)s4[2], (__bf16)s4[3]};
      *(bf16x4_t*)(a.out + bh * kD + 4 * d4) = v4;
    } else {
      *(f32x4_t*)(a.part_o + (bh * a.n_splits + split) * kD + 4 * d4) = s4;
    }
  }
  if (threadIdx.x < gcnt) {
    const int g = threadIdx.x;
    float Mg = kNegInf;
    for (int w = 0; w < kWaves; ++w) Mg = fmaxf(Mg, sm_m[w][g]);
    float Lg = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][g];
      Lg += (mw == kNegInf) ? 0.f : sm_l[w][g] * fast_exp2(mw - Mg);
    }
    const float lse_v = (Mg + __log2f(Lg)) * kLn2;
    const int64_t bh = (int64_t)b * a.Hq + h_base + g;
    if (final_out) {
      if (a.lse) a.lse[bh] = lse_v;
    } else {
      a.part_lse[bh * a.n_splits + split] = lse_v;
    }
  }
}

// Second pass: o = sum_i w_i o_i / sum_i w_i with w_i = exp(lse_i - max lse),
// lse = max + ln sum_i w_i.  One wave per (request, query head).
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + wave;
  if (bh >= (int64_t)a.batch * a.Hq) return;
  const int32_t b = (int32_t)(bh / a.Hq);
  int32_t L = a.seq_lens[b];
  const int32_t cap = a.max_blocks << a.bs_log2;
  L = L > cap ? cap : L;
  const int32_t n_b = (L + a.split_tokens - 1) / a.split_tokens;
  if (n_b <= 1) return;                      // written by the first pass
  const float* pl = a.part_lse + bh * a.n_splits;
  float M = kNegInf;
  for (int i = 0; i < n_b; ++i) M = fmaxf(M, pl[i]);
  f32x2_t acc = {0.f, 0.f};
  float wsum = 0.f;
  const f32x2_t* po = (const f32x2_t*)(a.part_o + bh * a.n_splits * kD) + lane;
  for (int i = 0; i < n_b; ++i) {
    const float w = fast_exp2((pl[i] - M) * kLog2e);
    wsum += w;
    acc += w * po[i * (kD / 2)];
  }
  const float inv = 1.f / wsum;
  const __bf16 o0 = (__bf16)(acc[0] * inv), o1 = (__bf16)(acc[1] * inv);
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  *(bf16x2_t*)(a.out + bh * kD + 2 * lane) = bf16x2_t{o0, o1};
  if (lane == 0 && a.lse) a.lse[bh] = M + __log2f(wsum) * kLn2;
}

}  // namespace

DecodePlan plan_decode(const kv_cache_t& c, int32_t batch, int32_t num_q_heads,
                       int32_t max_seq_len, int32_t split_tokens) {
  DecodePlan p;
  const int32_t G = num_q_heads / c.num_kv_heads;
  p.n_gchunks = (G + 15) / 16;
  if (split_tokens <= 0) {
    // Largest split (<= 1024 tokens) that still gives ~32 workgroups per CU
    // for the longest request; short batches fall back to 128-token splits.
    const int64_t units = (int64_t)batch * c.num_kv_heads * p.n_gchunks;
    split_tokens = 1024;
    while (split_tokens > 128 &&
           units * ((max_seq_len + split_tokens - 1) / split_tokens) < 8192)
      split_tokens >>= 1;
  }
  p.split_tokens = split_tokens;
  p.n_splits = (max_seq_len + split_tokens - 1) / split_tokens;
  if (p.n_splits < 1) p.n_splits = 1;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(const DecodePlan& p, int32_t batch, int32_t num_q_heads,
                              int32_t head_dim) {
  const size_t rows = (size_t)batch * num_q_heads * p.n_splits;
  return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float));
}

hipError_t launch_decode(const kv_cache_t& c, const DecodePlan& p, const void* q,
                         int32_t batch, int32_t num_q_heads, const int32_t* tables,
                         int32_t max_blocks, const int32_t* seq_lens, float scale,
                         void* out, float* lse, void* workspace, hipStream_t s) {
  DecodeArgs a;
  a.kc = (const uint8_t*)c.k_cache;
  a.vc = (const uint8_t*)c.v_cache;
  a.q = (const __bf16*)q;
  a.tables = tables;
  a.seq_lens = seq_lens;
  a.out = (__bf16*)out;
  a.lse = lse;
  const size_t rows = (size_t)batch * num_q_heads * p.n_splits;
  a.part_o = (float*)workspace;
  a.part_lse = (float*)((uint8_t*)workspace + align256(rows * c.head_dim * sizeof(float)));
  a.max_blocks = max_blocks;
  a.num_blocks = c.num_blocks;
  a.bs = c.block_size;
  a.bs_log2 = 0;
  while ((1 << a.bs_log2) < c.block_size) ++a.bs_log2;
  a.Hkv = c.num_kv_heads;
  a.Hq = num_q_heads;
  a.G = num_q_heads / c.num_kv_heads;
  a.n_gchunks = p.n_gchunks;
  a.split_tokens = p.split_tokens;
  a.n_splits = p.n_splits;
  a.batch = batch;
  a.qk_mult = scale * c.k_scale * kLog2e;
  a.v_scale = c.v_scale;
  dim3 grid((unsigned)p.n_splits, (unsigned)(c.num_kv_heads * p.n_gchunks), (unsigned)batch);
#define PKV_LAUNCH(L, T) \
  hipLaunchKernelGGL((decode_split_kernel<L, T>), grid, dim3(256), 0, s, a)
  if (c.layout == KV_LAYOUT_NHD) {
    if (c.dtype == KV_DTYPE_BF16) PKV_LAUNCH(KV_LAYOUT_NHD, KV_DTYPE_BF16);
    else PKV_LAUNCH(KV_LAYOUT_NHD, KV_DTYPE_FP8_E4M3);
  } else {
    if (c.dtype == KV_DTYPE_BF16) PKV_LAUNCH(KV_LAYOUT_PRESHUFFLED, KV_DTYPE_BF16);
    else PKV_LAUNCH(KV_LAYOUT_PRESHUFFLED, KV_DTYPE_FP8_E4M3);
  }
#undef PKV_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.n_splits > 1) {
    const int64_t bh = (int64_t)batch * num_q_heads;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((bh + 3) / 4)), dim3(256), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pkv
