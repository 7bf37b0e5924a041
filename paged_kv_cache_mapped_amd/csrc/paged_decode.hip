// Paged decode attention for gfx950: balanced split-K over the block table,
// then a log-sum-exp combine of the pieces of each request.
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
// Work split.  The requests' lengths, rounded up to the 32-token tile, are
// concatenated into one token stream that is cut into equal pieces.  Every
// wave is an independent worker that owns (piece, KV head, group of up to 16
// query heads sharing it) and runs one segment per request its piece
// overlaps, streaming the segment's 32-token tiles.  Per tile the wave:
//   * loads K with non-temporal 16-byte loads, every instruction reading
//     whole 128-byte lines: NHD K as whole token rows (like V), turned into
//     MFMA A-operand fragments through the wave's LDS slice; preshuffled K
//     straight into A-operand registers, each subtile taking one whole
//     16-token block (bf16) or 8 consecutive tokens from each 16-token half
//     of the tile (fp8),
//   * computes S^T = K Q^T for its query-head group with v_mfma_f32_16x16x32_bf16
//     (query heads are the 16 MFMA columns; grouped-query decode is a dense
//     contraction with G rows),
//   * runs the online softmax in registers (per query head: max / sum over the
//     4 lanes holding its 32 scores via cross-lane shuffles),
//   * accumulates O^T = V^T P^T with V^T as the A operand.  In the NHD layout V
//     rows are staged in the wave's LDS rows with 16-byte coalesced stores and
//     read back transposed with ds_read_b64_tr_b16; in the preshuffled layout V
//     is already stored token-minor ([block][head][bs/x][D][x]) and is loaded
//     straight into registers, lane rows trading words so that each lane
//     holds the tokens of its P^T fragment.
// At the end of a segment the wave writes either the final output (a request
// inside one piece) or an fp32 partial (o, lse) that a second kernel merges
// with LSE weights.  The partial of piece p of request b goes to row p + b:
// a request's pieces are consecutive and the next request starts at or after
// the last piece of the previous one, so rows never collide and at most
// (number of pieces + batch) rows exist, whatever the lengths.  (Merging in the last piece to finish would need
// device-scope fences, which on this multi-XCD part write back and invalidate
// whole L2 caches: far slower than a second launch.)
//
// fp8 (OCP e4m3fn) caches are decoded to bf16 in registers (exact) and the
// per-tensor scales are applied to the scores (k_scale) and to the output
// (v_scale): <q, c*ks> = ks <q, c>, sum p (c*vs) = vs sum p c.
#include <mutex>

#include "common.h"
#include "internal.h"

namespace pkv {

// Scratch memory of paged_decode_noalloc: the decode workspace (plan and fp32
// partials) for callers that cannot allocate.  Every device that runs the
// library holds one copy until the process ends.  In host code `scratch` is
// only a stand-in for the symbol: its device address, per device, comes from
// hipGetSymbolAddress and is the only handle used for it.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {

constexpr int kD = 128;
constexpr int kTile = 32;
constexpr int kWaves = 8;                        // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kVRowBytes = 288;                  // 128 bf16 + 32 B pad (bank spread)
constexpr int kVTileBytes = kTile * kVRowBytes;  // per wave
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kTabCap = 256;                     // block ids of one wave's segment staged in LDS
constexpr int kPlanLdsMax = 2048;                // batches up to this size plan in LDS

struct DecodeArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const __bf16* q;
  const int32_t* tables;
  const int32_t* seq_lens;
  __bf16* out;
  float* lse;
  float* part_o;              // [part_rows][Hq][D]: row p + b for piece p of request b
  float* part_lse;            // [part_rows][Hq]
  int32_t* hdr;               // [0] padded total T, [1] piece length, [2] pieces
  int32_t* cum;               // [B+1] exclusive prefix sums of lengths rounded up to 32
  int32_t* first_seq;         // [max_pieces] first request touched by each piece
  int32_t max_blocks, num_blocks, bs, bs_log2, Hkv, Hq, G, n_gchunks;
  int32_t batch, fixed_len, len_min, len_max, target_pieces;
  int32_t max_len;            // lengths are clamped to min(table capacity, max_seq_len)
  int32_t lds_plan;           // 1: every workgroup plans in LDS (batch <= kPlanLdsMax)
  int32_t gpw;                // head groups per workgroup (1, 2 or 4); 4 / gpw waves share a group
  float qk_mult;   // scale * k_scale * log2(e): scores in the exp2 domain
  float v_scale;
};

__device__ __forceinline__ int32_t clamp_block(int32_t blk, int32_t nb) {
  return blk < 0 ? 0 : (blk >= nb ? nb - 1 : blk);
}

// Query dims held by lane quarter q4 for MFMA k-step kk.  Natural order where
// the K fragments come as bf16 (bf16 caches, and NHD fp8 whose K is decoded
// into LDS rows); the preshuffled fp8 cache hands each lane 16 consecutive
// dims per load, i.e. k-steps 2p and 2p+1 read one 16-dim chunk 4p + q4.
template <int LAYOUT, int DT>
__device__ __forceinline__ int dmap(int kk, int q4) {
  if constexpr (LAYOUT == KV_LAYOUT_PRESHUFFLED && DT == KV_DTYPE_FP8_E4M3)
    return 64 * (kk >> 1) + 16 * q4 + 8 * (kk & 1);
  else return 32 * kk + 8 * q4;
}

// Token (relative to the tile start) of row rr of K subtile s, and of element
// i of a lane's score accumulator s in lane quarter q4 (its accumulator rows
// are 4 q4 .. 4 q4 + 3); the score of that token is probability k-slot
// 4 s + i of the lane's P^T fragment.  Default: k-slots 8 q4 .. 8 q4 + 7 are
// tokens 8 q4 .. 8 q4 + 7 of the tile.  The preshuffled K cache stores the
// tokens of a block consecutively for each 16-byte dim chunk.  With bf16
// (8-token V x-groups) each subtile takes one whole 16-token block -- every
// K load instruction reads 256-byte runs -- and lane quarter q4 gets tokens
// 4 q4 .. + 3 of both blocks.  With fp8 (16-token V x-groups) each subtile
// takes 8 consecutive tokens from each 16-token half of the tile (128-byte
// runs), so that lane quarter q4 ends up with tokens of half q4 / 2 only; in
// both cases one swap between lane rows q4 and q4 ^ 1 builds the V^T
// fragments (see consume_tile).
template <int LAYOUT, int DT>
__device__ __forceinline__ int k_row_token(int s, int rr) {
  if constexpr (LAYOUT == KV_LAYOUT_PRESHUFFLED && DT == KV_DTYPE_BF16) return 16 * s + rr;
  else if constexpr (LAYOUT == KV_LAYOUT_PRESHUFFLED) return 16 * (rr >> 3) + 8 * s + (rr & 7);
  else return 8 * (rr >> 2) + 4 * s + (rr & 3);
}
template <int LAYOUT, int DT>
__device__ __forceinline__ int score_token(int q4, int s, int i) {
  if constexpr (LAYOUT == KV_LAYOUT_PRESHUFFLED && DT == KV_DTYPE_BF16) return 16 * s + 4 * q4 + i;
  else if constexpr (LAYOUT == KV_LAYOUT_PRESHUFFLED) return 16 * (q4 >> 1) + 8 * s + 4 * (q4 & 1) + i;
  else return 8 * q4 + 4 * s + i;
}

// K/V bytes are read once per call: non-temporal loads (the `nt` cache
// policy) stream them past the caches instead of filling L2 with lines that
// are never read again, which lets the decode's loads reach a higher rate.
__device__ __forceinline__ u32x4_t stream_load(const u32x4_t* p) {
  return __builtin_nontemporal_load(p);
}

// Raw bytes of one wave's 32-token tile, as loaded (fp8 uses the low halves).
struct TileRaw {
  u32x4_t k[8];
  u32x4_t v[8];
};

// Issue every load of the tile starting at token t0.  Tokens at or past t_end
// are clamped to t_end - 1: their addresses stay inside the request and they
// repeat a row already being fetched (cache hits), so tiles past the end can be
// prefetched unconditionally.
template <int LAYOUT, int DT>
__device__ __forceinline__ void issue_tile(const DecodeArgs& a, const int32_t* s_tab, int32_t ib0,
                                           int hkv, int32_t t0, int32_t t_end, int lane,
                                           TileRaw& R) {
  const int q4 = lane >> 4, r = lane & 15;
  if constexpr (LAYOUT == KV_LAYOUT_NHD && DT == KV_DTYPE_BF16) {
    // K and V rows of token t0 + 4 j + lane / 16, 16-byte chunk lane % 16:
    // every load instruction reads four whole 256-byte rows (K reaches the
    // MFMA layout through LDS in consume_tile)
    const int a4 = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int32_t tok = min(t0 + 4 * j + a4, t_end - 1);
      const int32_t blk = s_tab[(tok >> a.bs_log2) - ib0];
      const int64_t row = ((int64_t)blk * a.bs + (tok & (a.bs - 1))) * a.Hkv + hkv;
      R.k[j] = stream_load((const u32x4_t*)(a.kc + row * (kD * 2) + c16 * 16));
      R.v[j] = stream_load((const u32x4_t*)(a.vc + row * (kD * 2) + c16 * 16));
    }
    return;
  }
  if constexpr (LAYOUT == KV_LAYOUT_NHD) {
    // fp8: K and V rows of token t0 + 8 j + lane / 8, 16-byte chunk lane % 8
    // (eight whole 128-byte rows per instruction)
    const int a8 = lane >> 3, c8 = lane & 7;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int32_t tok = min(t0 + 8 * j + a8, t_end - 1);
      const int32_t blk = s_tab[(tok >> a.bs_log2) - ib0];
      const int64_t row = ((int64_t)blk * a.bs + (tok & (a.bs - 1))) * a.Hkv + hkv;
      R.k[j] = stream_load((const u32x4_t*)(a.kc + row * kD + c8 * 16));
      R.v[j] = stream_load((const u32x4_t*)(a.vc + row * kD + c8 * 16));
    }
    return;
  }
  // Preshuffled K: A-operand row r of subtile s = token t0 + k_row_token(s, r)
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int32_t tok = min(t0 + k_row_token<LAYOUT, DT>(s, r), t_end - 1);
    const int32_t blk = s_tab[(tok >> a.bs_log2) - ib0];
    const int32_t off = tok & (a.bs - 1);
    const int64_t bh = (int64_t)blk * a.Hkv + hkv;
    if constexpr (DT == KV_DTYPE_BF16) {     // [blk][h][D/8][bs][8]
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int64_t e = ((bh * (kD / 8) + (4 * kk + q4)) * a.bs + off) * 8;
        R.k[4 * s + kk] = stream_load((const u32x4_t*)(a.kc + e * 2));
      }
    } else {                                  // [blk][h][D/16][bs][16]
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int64_t e = ((bh * (kD / 16) + (4 * pp + q4)) * a.bs + off) * 16;
        R.k[2 * s + pp] = stream_load((const u32x4_t*)(a.kc + e));
      }
    }
  }
  // V as the V^T operand (bf16: 8 tokens of dim 16n + r; fp8: see below).
  if constexpr (DT == KV_DTYPE_FP8_E4M3) {
    // 16-byte loads: lane (q4, r), load j takes the 16 tokens of tile half
    // q4 / 2 for dim 16 (2 j + q4 % 2) + r; consume_tile trades words between
    // lanes q4 and q4 ^ 1 so that each ends with its P^T tokens of dims
    // 16 (2 j) + r and 16 (2 j + 1) + r.
    const int32_t tb = min(t0 + 16 * (q4 >> 1), (t_end - 1) & ~15);   // aligned to 16
    const int32_t blk = s_tab[(tb >> a.bs_log2) - ib0];
    const int32_t off = tb & (a.bs - 1);
    const int64_t base = (((int64_t)blk * a.Hkv + hkv) * (a.bs / 16) + off / 16) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      R.v[j] = stream_load((const u32x4_t*)(a.vc + (base + 16 * (2 * j + (q4 & 1)) + r) * 16));
  } else {
    constexpr int X = 8;                                        // bf16
    // 8-token group ((q4 & 1) << 1) | (q4 >> 1): lane rows q4 and q4 ^ 1 hold
    // groups g and g + 2 (the same 4-token quarters of both 16-token blocks)
    const int grp = ((q4 & 1) << 1) | (q4 >> 1);
    const int32_t tb = min(t0 + 8 * grp, (t_end - 1) & ~7);   // 8 tokens, aligned to 8
    const int32_t blk = s_tab[(tb >> a.bs_log2) - ib0];
    const int32_t off = tb & (a.bs - 1);
    const int64_t base = (((int64_t)blk * a.Hkv + hkv) * (a.bs / X) + off / X) * kD;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int64_t e = (base + 16 * n + r) * X + (off % X);
      R.v[n] = stream_load((const u32x4_t*)(a.vc + e * 2));
    }
  }
}

// Running state of one wave: O^T accumulators (element i of o[n] is dim
// 16n + 4*q4 + i of query head r) and the exp2-domain max / lane-partial sum.
struct WaveState {
  f32x4_t o[8];
  float m, l;
};

template <int LAYOUT, int DT>
__device__ __forceinline__ void consume_tile(const DecodeArgs& a, const TileRaw& R,
                                             const bf16x8_t (&qb)[4], int32_t t0, int32_t t_end,
                                             int lane, uint8_t* vt, WaveState& st) {
  const int q4 = lane >> 4, r = lane & 15;
  const bool partial = t0 + kTile > t_end;
  bf16x8_t ka[2][4];
  if constexpr (LAYOUT == KV_LAYOUT_NHD) {
    // K rows (fp8 decoded) as bf16 into the wave's LDS slice (256-byte rows,
    // 16-byte chunk c of row x at position c ^ kfold(x)), then the A-operand
    // fragments out: row 8 (r / 4) + 4 s + r % 4, chunk 4 kk + q4.  kfold
    // differs between the 16 rows of one fragment read and permutes the
    // chunks of each row written, so neither access pattern has bank
    // conflicts.  The V rows written next reuse the slice; one wave's LDS
    // requests are served in order.
    auto kfold = [](int x) { return (x & 3) | (((x >> 3) & 3) << 2); };
    if constexpr (DT == KV_DTYPE_BF16) {
      const int a4 = lane >> 4, c16 = lane & 15;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int x = 4 * j + a4;
        *(u32x4_t*)(vt + x * 256 + 16 * (c16 ^ kfold(x))) = R.k[j];
      }
    } else {
      const int a8 = lane >> 3, c8 = lane & 7;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = 8 * j + a8;
        const u32x4_t w = R.k[j];
        *(bf16x8_t*)(vt + x * 256 + 16 * ((2 * c8) ^ kfold(x))) = fp8x8_to_bf16(u32x2_t{w[0], w[1]});
        *(bf16x8_t*)(vt + x * 256 + 16 * ((2 * c8 + 1) ^ kfold(x))) = fp8x8_to_bf16(u32x2_t{w[2], w[3]});
      }
    }
    order_lds();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int x = 8 * (r >> 2) + 4 * s + (r & 3);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        ka[s][kk] = *(const bf16x8_t*)(vt + x * 256 + 16 * ((4 * kk + q4) ^ kfold(x)));
    }
    order_lds();
  } else {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (DT == KV_DTYPE_BF16) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[s][kk] = __builtin_bit_cast(bf16x8_t, R.k[4 * s + kk]);
      } else {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const u32x4_t w = R.k[2 * s + pp];
          ka[s][2 * pp] = fp8x8_to_bf16(u32x2_t{w[0], w[1]});
          ka[s][2 * pp + 1] = fp8x8_to_bf16(u32x2_t{w[2], w[3]});
        }
      }
    }
  }
  bf16x8_t va[8];
  if constexpr (LAYOUT == KV_LAYOUT_NHD) {
    if constexpr (DT == KV_DTYPE_BF16) {
      const int a4 = lane >> 4, c16 = lane & 15;
#pragma unroll
      for (int j4 = 0; j4 < 8; ++j4)
        *(u32x4_t*)(vt + (4 * j4 + a4) * kVRowBytes + c16 * 16) = R.v[j4];
    } else {
      const int a8 = lane >> 3, c8 = lane & 7;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t w = R.v[j];
        uint8_t* dst = vt + (8 * j + a8) * kVRowBytes + c8 * 32;
        *(bf16x8_t*)dst = fp8x8_to_bf16(u32x2_t{w[0], w[1]});
        *(bf16x8_t*)(dst + 16) = fp8x8_to_bf16(u32x2_t{w[2], w[3]});
      }
    }
  } else {
    if constexpr (DT == KV_DTYPE_BF16) {
      // Load n of lane (q4, r) holds the 8 tokens of group g = 2 (q4 & 1) +
      // q4 / 2 (tokens 8 g .. 8 g + 7) of dim 16 n + r, two per word.  The
      // lane's P^T k-slots are tokens 4 q4 .. + 3 and 16 + 4 q4 .. + 3: the
      // first or second halves of groups q4 / 2 and q4 / 2 + 2, which lane rows
      // q4 and q4 ^ 1 hold between them.  Swapping (w0, w1) of the odd rows of
      // 16 lanes with (w2, w3) of the even rows leaves exactly those, in
      // k-slot order.
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        uint32_t w0 = R.v[n][0], w1 = R.v[n][1], w2 = R.v[n][2], w3 = R.v[n][3];
        asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3"
                     : "+v"(w0), "+v"(w2), "+v"(w1), "+v"(w3));
        va[n] = __builtin_bit_cast(bf16x8_t, u32x4_t{w0, w1, w2, w3});
      }
    } else {
      // Load j of lane (q4, r) holds the 16 tokens of tile half q4 / 2 of dim
      // 16 (2 j + q4 % 2) + r as words w0..w3 (4 tokens each).  The lane's
      // P^T k-slots are tokens {0-3, 8-11} (even q4) or {4-7, 12-15} (odd q4)
      // of that half: words 0 and 2, or 1 and 3.  Swapping w0 of the odd rows
      // of 16 lanes with w1 of the even rows, and w2 with w3, leaves in every
      // lane (w0, w2) of dim 16 (2 j) + r and (w1, w3) of dim 16 (2 j + 1) + r
      // for exactly those tokens (v_permlane16_swap_b32: odd rows of the first
      // operand <-> even rows of the second).
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w0 = R.v[j][0], w1 = R.v[j][1], w2 = R.v[j][2], w3 = R.v[j][3];
        asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3"
                     : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
        va[2 * j] = fp8x8_to_bf16(u32x2_t{w0, w2});
        va[2 * j + 1] = fp8x8_to_bf16(u32x2_t{w1, w3});
      }
    }
    if (partial) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (t0 + score_token<LAYOUT, DT>(q4, jj >> 2, jj & 3) >= t_end) {
#pragma unroll
          for (int n = 0; n < 8; ++n) va[n][jj] = (__bf16)0.f;
        }
    }
  }

  // ---- S^T = K Q^T: element i of acc[s] is token t0 + score_token(q4, s, i), head r
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
      const int32_t tok = t0 + score_token<LAYOUT, DT>(q4, s, i);
      sc[4 * s + i] = (partial && tok >= t_end) ? kNegInf : acc[s][i] * a.qk_mult;
    }

  // ---- online softmax for query head r (exp2 domain)
  float mt = sc[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sc[i]);
  mt = fmaxf(mt, __shfl_xor(mt, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float m_new = fmaxf(st.m, mt);      // finite: a wave's first tile has a valid token
  const float alpha = fast_exp2(st.m - m_new);
  float p[8], psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = fast_exp2(sc[i] - m_new);
    psum += p[i];
  }
  st.l = st.l * alpha + psum;               // lane-partial; reduced at the end
  st.m = m_new;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.o[n] *= alpha;
  const bf16x8_t pb = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                       (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};

  // ---- O^T += V^T P^T
  if constexpr (LAYOUT == KV_LAYOUT_NHD) {
    order_lds();
    const int row0 = 8 * q4 + (r >> 2);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int colb = (16 * n + 4 * (r & 3)) * 2;
      const s16x4_t lo = lds_read_tr16(vt + row0 * kVRowBytes + colb);
      const s16x4_t hi = lds_read_tr16(vt + (row0 + 4) * kVRowBytes + colb);
      st.o[n] = mfma16(cat_tr(lo, hi), pb, st.o[n]);
    }
    order_lds();
  } else {
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = mfma16(va[n], pb, st.o[n]);
  }
}

__device__ __forceinline__ int32_t clamp_len(int32_t L, int32_t cap) {
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Piece length from the padded stream length T (same rule in both planners).
// Pieces are 1/4 longer than an even share per wave: about one wave in five
// then has no piece, but HBM stays saturated and the kernel has fewer
// per-piece start-ups and partials to write and merge.
__device__ __forceinline__ int32_t piece_len(const DecodeArgs& a, int32_t T) {
  if (a.fixed_len > 0) return a.fixed_len;
  int32_t len = (T + a.target_pieces - 1) / a.target_pieces;
  len += len / 4;
  len = (len + 31) & ~31;
  return len < a.len_min ? a.len_min : (len > a.len_max ? a.len_max : len);
}

// Work plan (one workgroup): lengths rounded up to the 32-token tile are
// concatenated into one token stream of length T; the stream is cut into
// pieces of equal length (a multiple of 32), so every workgroup of the main
// kernel gets the same amount of KV to read however the lengths are spread.
// Writes cum[] (exclusive prefix sums), the header and, for every piece, the
// first request it touches.  Used for batches above kPlanLdsMax; smaller
// batches are planned by every main-pass workgroup in its own LDS.
__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a) {
  __shared__ int32_t s_part[1024];
  const int tid = threadIdx.x;
  const int32_t B = a.batch;
  const int32_t cap = a.max_len;
  const int32_t per = (B + 1023) / 1024;
  const int32_t b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int32_t sum = 0;
  for (int32_t b = b0; b < b1; ++b) sum += (clamp_len(a.seq_lens[b], cap) + 31) & ~31;
  s_part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {       // inclusive scan
    const int32_t v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int32_t run = tid ? s_part[tid - 1] : 0;
  for (int32_t b = b0; b < b1; ++b) {
    a.cum[b] = run;
    run += (clamp_len(a.seq_lens[b], cap) + 31) & ~31;
  }
  const int32_t T = s_part[1023];
  const int32_t len = piece_len(a, T);
  const int32_t NP = (T + len - 1) / len;
  if (tid == 0) {
    a.cum[B] = T;
    a.hdr[0] = T;
    a.hdr[1] = len;
    a.hdr[2] = NP;
  }
  __threadfence();
  __syncthreads();
  // first request of piece p: the largest b with cum[b] <= p*len (empty
  // requests share their successor's offset, so the largest one is non-empty)
  const volatile int32_t* cum = a.cum;
  for (int32_t p = tid; p < NP; p += 1024) {
    const int32_t start = p * len;
    int32_t lo = 0, hi = B - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (cum[mid] <= start) lo = mid; else hi = mid - 1;
    }
    a.first_seq[p] = lo;
  }
}

// Main pass.  Every wave is an independent worker for one (KV head,
// query-head group): the workgroup's gpw groups are consecutive, and the
// 4 / gpw waves of one group take pieces x*(4/gpw) + sub, stepping by
// gridDim.x * (4/gpw).  With gpw = 4 the four waves of a CU read four heads of
// the same tokens at about the same time (1 KB of each token's K and V rows
// instead of four scattered 256-byte slices), which keeps DRAM rows open.
// For each request its piece overlaps, a wave stages the segment's block ids in its own LDS slice,
// streams the segment's 32-token tiles through a two-deep register pipeline,
// and writes either the final output (a request covered by one piece) or an
// fp32 partial (o, lse) in row p + b.  No
// barrier is taken after the plan, so the waves of a CU drift apart and each
// one's request boundaries are covered by the others' streaming.
//
// The plan (prefix sums of the rounded lengths, piece length, first request
// of a piece) comes from LDS, computed by every workgroup for itself when the
// batch is small, else from decode_plan_kernel's output in the workspace.
template <int LAYOUT, int DT>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void decode_piece_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wpg = kWaves / a.gpw;                  // waves per head group
  const int32_t grp = blockIdx.y * a.gpw + wave % a.gpw;
  const int sub = wave / a.gpw;
  const int32_t hkv = grp / a.n_gchunks;
  const int32_t gc = grp - hkv * a.n_gchunks;
  const int q4 = lane >> 4, r = lane & 15;
  const int g0 = gc * 16;
  const int gcnt = min(16, a.G - g0);
  const int32_t h_base = hkv * a.G + g0;
  const int32_t cap = a.max_len;

  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves * kVTileBytes];
  __shared__ int32_t s_tab[kWaves][kTabCap];
  __shared__ int32_t s_cum[kPlanLdsMax + 1];
  __shared__ int32_t s_wsum[kWaves];
  __shared__ int32_t s_prog[kWaves];     // tiles consumed so far, per wave
  uint8_t* vt = smem + wave * kVTileBytes;
  int32_t* tab = s_tab[wave];

  // Waves w and w ^ 4 share a SIMD, and its arbiter favours the older one:
  // left alone, waves 0-3 finish their (equal) pieces far ahead of waves 4-7
  // and the SIMD then streams with half the loads in flight.  Each wave
  // publishes its progress and raises its priority while it trails its
  // partner, which keeps the pair level.
  int32_t my_prog = 0;
  if (lane == 0) s_prog[wave] = 0;

  int32_t T, len, NP;
  if (a.lds_plan) {
    // exclusive prefix sums of the rounded lengths: 8 requests per thread,
    // a wave scan, then the 4 wave totals
    constexpr int kPer = kPlanLdsMax / kThreads;
    const int32_t b0 = (int32_t)threadIdx.x * kPer;
    int32_t v[kPer], sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      v[i] = b0 + i < a.batch ? (clamp_len(a.seq_lens[b0 + i], cap) + 31) & ~31 : 0;
      sum += v[i];
    }
    int32_t inc = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t t = __shfl_up(inc, off);
      if (lane >= off) inc += t;
    }
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    int32_t run = inc - sum;
    T = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      run += w < wave ? s_wsum[w] : 0;
      T += s_wsum[w];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (b0 + i < a.batch) s_cum[b0 + i] = run;
      run += v[i];
    }
    if (threadIdx.x == 0) s_cum[a.batch] = T;
    __syncthreads();
    T = uniform(T);
    len = piece_len(a, T);
    NP = (T + len - 1) / len;
    if (blockIdx.x == 0 && blockIdx.y == 0) {   // the plan the combine pass reads
      for (int32_t b = threadIdx.x; b <= a.batch; b += kThreads) a.cum[b] = s_cum[b];
      if (threadIdx.x == 0) {
        a.hdr[0] = T;
        a.hdr[1] = len;
        a.hdr[2] = NP;
      }
    }
  } else {
    T = uniform(a.hdr[0]);
    len = uniform(a.hdr[1]);
    NP = uniform(a.hdr[2]);
    __syncthreads();                          // s_prog is initialised
  }
  auto cum_at = [&](int32_t b) -> int32_t { return a.lds_plan ? s_cum[b] : a.cum[b]; };

  for (int32_t p = blockIdx.x * wpg + sub; p < NP; p += gridDim.x * wpg) {
    const int32_t pstart = p * len, pend = min(T, pstart + len);
    int32_t b_first;
    if (a.lds_plan) {
      // largest b with cum[b] <= pstart (empty requests share their
      // successor's offset, so the largest one is non-empty)
      int32_t lo = 0, hi = a.batch - 1;
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (s_cum[mid] <= pstart) lo = mid; else hi = mid - 1;
      }
      b_first = uniform(lo);
    } else {
      b_first = uniform(a.first_seq[p]);
    }
    for (int32_t b = b_first; b < a.batch; ++b) {
      const int32_t cb = uniform(cum_at(b));
      if (cb >= pend) break;
      const int32_t L = uniform(clamp_len(a.seq_lens[b], cap));
      const int32_t t_begin = max(pstart, cb) - cb;      // multiple of 32
      const int32_t t_end = min(pend - cb, L);
      if (t_begin >= t_end) continue;                    // only padding of b
      const int32_t first_piece = cb / len;
      const int32_t n_b = (cb + L - 1) / len - first_piece + 1;

      // segment prologue: this wave's block-id slice and Q, issued together.
      // The slice goes to the wave's own LDS rows; a wave's LDS accesses
      // complete in order, so no barrier is needed before reading them.
      const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
      const int32_t ib0 = t_begin >> a.bs_log2;
      const int32_t nent = ((t_end - 1) >> a.bs_log2) - ib0 + 1;   // <= kTabCap
      int32_t tb[kTabCap / 64];
#pragma unroll
      for (int j = 0; j < kTabCap / 64; ++j)
        tb[j] = lane + 64 * j < nent ? trow[ib0 + lane + 64 * j] : 0;
      bf16x8_t qb[4];
      {
        const bf16x8_t zero = {};
        const __bf16* qrow = a.q + ((int64_t)b * a.Hq + h_base + r) * kD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          qb[kk] = (r < gcnt) ? *(const bf16x8_t*)(qrow + dmap<LAYOUT, DT>(kk, q4)) : zero;
      }
#pragma unroll
      for (int j = 0; j < kTabCap / 64; ++j)
        if (lane + 64 * j < nent) tab[lane + 64 * j] = clamp_block(tb[j], a.num_blocks);
      order_lds();

      WaveState st;
#pragma unroll
      for (int n = 0; n < 8; ++n) st.o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      st.m = kNegInf;
      st.l = 0.f;

      // Two register buffers: the next tile's loads are in flight while the
      // current tile is consumed (the scheduling barriers keep the compiler
      // from sinking them).  Tiles go in pairs: a second tile past the end has
      // every token masked (scores -inf, weights 0, rows clamped to the last
      // valid token) and changes nothing.  An early exit between the two
      // halves would leave the second buffer's loads in flight on one path
      // into the loop head, and the compiler then waits on them there in
      // every iteration, which serialises the prefetch.
      const int32_t n_tiles = (t_end - t_begin + kTile - 1) / kTile;
      TileRaw A, B;
      issue_tile<LAYOUT, DT>(a, tab, ib0, hkv, t_begin, t_end, lane, A);
      for (int32_t it = 0; it < n_tiles; it += 2) {
        my_prog += 2;
        if (lane == 0) s_prog[wave] = my_prog;
        if (my_prog <= uniform(s_prog[wave ^ 4])) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(0);
        issue_tile<LAYOUT, DT>(a, tab, ib0, hkv, t_begin + (it + 1) * kTile, t_end, lane, B);
        __builtin_amdgcn_sched_barrier(0);
        consume_tile<LAYOUT, DT>(a, A, qb, t_begin + it * kTile, t_end, lane, vt, st);
        issue_tile<LAYOUT, DT>(a, tab, ib0, hkv, t_begin + (it + 2) * kTile, t_end, lane, A);
        __builtin_amdgcn_sched_barrier(0);
        consume_tile<LAYOUT, DT>(a, B, qb, t_begin + (it + 1) * kTile, t_end, lane, vt, st);
      }
      __builtin_amdgcn_s_waitcnt(0);     // the last prefetch (past the end) lands

      // ---- this wave's result for the segment: query head r, dims 16n + 4*q4 + i
      float l_sum = st.l;
      l_sum += __shfl_xor(l_sum, 16);
      l_sum += __shfl_xor(l_sum, 32);
      if (r < gcnt) {
        const int64_t bh = (int64_t)b * a.Hq + h_base + r;
        const float f = a.v_scale / l_sum;       // l_sum > 0: the segment has a token
        const float lse_v = (st.m + __log2f(l_sum)) * kLn2;
        if (n_b == 1) {
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const f32x4_t o = st.o[n] * f;
            const bf16x4_t v4 = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
            *(bf16x4_t*)(a.out + bh * kD + 16 * n + 4 * q4) = v4;
          }
          if (q4 == 0 && a.lse) a.lse[bh] = lse_v;
        } else {
          const int64_t prow = (int64_t)(p + b) * a.Hq + h_base + r;
          float* po = a.part_o + prow * kD;
#pragma unroll
          for (int n = 0; n < 8; ++n) *(f32x4_t*)(po + 16 * n + 4 * q4) = st.o[n] * f;
          if (q4 == 0) a.part_lse[prow] = lse_v;
        }
      }
    }
  }
}

// Second pass: o = sum_i w_i o_i / sum_i w_i with w_i = exp(lse_i - max lse),
// lse = max + ln sum_i w_i, over the pieces of each request that spans more
// than one piece.  One wave per (request, query head).  A request of length 0
// has no visible key: its output is 0 and its lse -inf.
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + wave;
  if (bh >= (int64_t)a.batch * a.Hq) return;
  const int32_t b = (int32_t)(bh / a.Hq);
  const int32_t h = (int32_t)(bh - (int64_t)b * a.Hq);
  const int32_t L = clamp_len(a.seq_lens[b], a.max_len);
  if (L == 0) {
    *(bf16x2_t*)(a.out + bh * kD + 2 * lane) = bf16x2_t{(__bf16)0.f, (__bf16)0.f};
    if (lane == 0 && a.lse) a.lse[bh] = kNegInf;
    return;
  }
  const int32_t len = a.hdr[1];
  const int32_t cb = a.cum[b];
  const int32_t n_b = (cb + L - 1) / len - cb / len + 1;
  if (n_b <= 1) return;                      // written by the main pass
  // partial rows (first piece + i + b), i < n_b; consecutive rows are Hq apart
  const int64_t row0 = (int64_t)(cb / len + b) * a.Hq + h;
  const float* pl = a.part_lse + row0;
  const f32x2_t* po = (const f32x2_t*)(a.part_o + row0 * kD) + lane;
  const int64_t ostride = (int64_t)a.Hq * (kD / 2);   // in f32x2 units
  float M = kNegInf;
  f32x2_t acc = {0.f, 0.f};
  float wsum = 0.f;
  // Chunks of kU partials, every load of a chunk issued up front; the
  // running maximum and weights are carried across chunks (requests spanning
  // more than kU pieces are common when lengths are short and many).
  constexpr int kU = 8;
  for (int c0 = 0; c0 < n_b; c0 += kU) {
    float lv[kU];
    f32x2_t ov[kU];
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      lv[i] = c0 + i < n_b ? pl[(c0 + i) * a.Hq] : kNegInf;
      ov[i] = c0 + i < n_b ? po[(c0 + i) * ostride] : f32x2_t{0.f, 0.f};
    }
    float Mc = M;
#pragma unroll
    for (int i = 0; i < kU; ++i) Mc = fmaxf(Mc, lv[i]);
    if (c0 > 0) {
      const float sc = fast_exp2((M - Mc) * kLog2e);
      wsum *= sc;
      acc *= sc;
    }
    M = Mc;
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const float w = c0 + i < n_b ? fast_exp2((lv[i] - M) * kLog2e) : 0.f;
      wsum += w;
      acc += w * ov[i];
    }
  }
  const float inv = 1.f / wsum;
  const __bf16 o0 = (__bf16)(acc[0] * inv), o1 = (__bf16)(acc[1] * inv);
  *(bf16x2_t*)(a.out + bh * kD + 2 * lane) = bf16x2_t{o0, o1};
  if (lane == 0 && a.lse) a.lse[bh] = M + __log2f(wsum) * kLn2;
}

}  // namespace

static int32_t log2_ceil(int32_t v) {
  int32_t l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

DecodePlan plan_decode(const kv_cache_t& c, int32_t batch, int32_t num_q_heads,
                       int32_t max_seq_len, int32_t split_tokens, hipStream_t stream) {
  DecodePlan p;
  const int32_t G = num_q_heads / c.num_kv_heads;
  p.n_gchunks = (G + 15) / 16;
  const int32_t groups = c.num_kv_heads * p.n_gchunks;
  // a piece's block ids must fit a wave's LDS slice: len/bs + 1 <= kTabCap
  int64_t len_max = ((int64_t)(kTabCap - 1) << log2_ceil(c.block_size)) & ~(int64_t)31;
  if (len_max > 16384) len_max = 16384;
  p.len_max = (int32_t)len_max;
  if (split_tokens > 0) {
    p.fixed_len = split_tokens < p.len_max ? split_tokens : p.len_max;
    p.len_min = p.fixed_len;
  } else {
    p.fixed_len = 0;
    p.len_min = 256 < p.len_max ? 256 : p.len_max;
  }
  // head groups per workgroup: as many of the 8 as divide evenly, so a
  // workgroup's waves read the heads of the same tokens together
  p.gpw = groups % 8 == 0 ? 8 : (groups % 4 == 0 ? 4 : (groups % 2 == 0 ? 2 : 1));
  // grid: one round of one resident workgroup per CU
  const int32_t slots = device_cu_count(stream);
  const int32_t rows = groups / p.gpw;
  p.pieces_per_group = slots / rows > 0 ? slots / rows : 1;   // grid x
  p.split_tokens = p.fixed_len;
  p.target_pieces = p.pieces_per_group * (kWaves / p.gpw);
  // Pieces of the padded stream (T <= batch * max_seq_len rounded up to 32):
  // a fixed length gives ceil(T / len); the automatic length is at least
  // T / target_pieces unless clamped to len_max, so at most
  // max(target_pieces, ceil(T / len_max)).
  const int64_t padded = (int64_t)batch * ((max_seq_len + 31) & ~31);
  int64_t np;
  if (p.fixed_len > 0) {
    np = (padded + p.fixed_len - 1) / p.fixed_len;
  } else {
    np = (padded + p.len_max - 1) / p.len_max;
    if (np < p.target_pieces) np = p.target_pieces;
  }
  p.max_pieces = (int32_t)(np + 1);
  p.part_rows = p.max_pieces + batch;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(const DecodePlan& p, int32_t batch, int32_t num_q_heads,
                              int32_t head_dim) {
  const size_t rows = (size_t)p.part_rows * num_q_heads;
  return 256 + align256((size_t)(batch + 1) * 4) + align256((size_t)p.max_pieces * 4) +
         align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float));
}


hipError_t launch_decode(const kv_cache_t& c, const DecodePlan& p, const void* q,
                         int32_t batch, int32_t num_q_heads, const int32_t* tables,
                         int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                         float scale, void* out, float* lse, void* workspace, hipStream_t s) {
  DecodeArgs a;
  a.kc = (const uint8_t*)c.k_cache;
  a.vc = (const uint8_t*)c.v_cache;
  a.q = (const __bf16*)q;
  a.tables = tables;
  a.seq_lens = seq_lens;
  a.out = (__bf16*)out;
  a.lse = lse;
  uint8_t* w = (uint8_t*)workspace;
  a.hdr = (int32_t*)w;
  w += 256;
  a.cum = (int32_t*)w;
  w += align256((size_t)(batch + 1) * 4);
  a.first_seq = (int32_t*)w;
  w += align256((size_t)p.max_pieces * 4);
  const size_t rows = (size_t)p.part_rows * num_q_heads;
  a.part_o = (float*)w;
  w += align256(rows * c.head_dim * sizeof(float));
  a.part_lse = (float*)w;
  a.max_blocks = max_blocks;
  a.num_blocks = c.num_blocks;
  a.bs = c.block_size;
  a.bs_log2 = log2_ceil(c.block_size);
  const int64_t capacity = (int64_t)max_blocks << a.bs_log2;
  a.max_len = (int32_t)(capacity < max_seq_len ? capacity : max_seq_len);
  a.Hkv = c.num_kv_heads;
  a.Hq = num_q_heads;
  a.G = num_q_heads / c.num_kv_heads;
  a.n_gchunks = p.n_gchunks;
  a.batch = batch;
  a.fixed_len = p.fixed_len;
  a.len_min = p.len_min;
  a.len_max = p.len_max;
  a.gpw = p.gpw;
  a.target_pieces = p.target_pieces;
  a.qk_mult = scale * c.k_scale * kLog2e;
  a.v_scale = c.v_scale;
  a.lds_plan = batch <= kPlanLdsMax ? 1 : 0;
  hipError_t e;
  if (!a.lds_plan) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)p.pieces_per_group, (unsigned)(c.num_kv_heads * p.n_gchunks / p.gpw));
#define PKV_LAUNCH(L, T) \
  hipLaunchKernelGGL((decode_piece_kernel<L, T>), grid, dim3(kThreads), 0, s, a)
  if (c.layout == KV_LAYOUT_NHD) {
    if (c.dtype == KV_DTYPE_BF16) PKV_LAUNCH(KV_LAYOUT_NHD, KV_DTYPE_BF16);
    else PKV_LAUNCH(KV_LAYOUT_NHD, KV_DTYPE_FP8_E4M3);
  } else {
    if (c.dtype == KV_DTYPE_BF16) PKV_LAUNCH(KV_LAYOUT_PRESHUFFLED, KV_DTYPE_BF16);
    else PKV_LAUNCH(KV_LAYOUT_PRESHUFFLED, KV_DTYPE_FP8_E4M3);
  }
#undef PKV_LAUNCH
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t bh = (int64_t)batch * num_q_heads;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((bh + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv

namespace pkv {

// Device address of `scratch` on the device `stream` runs on, looked up once
// per device with that device current.  Returns nullptr (and the HIP error in
// *err) when the lookup fails.
void* decode_scratch(hipStream_t stream, hipError_t* err) {
  static std::mutex mu;
  static void* addr[64] = {};
  int cur = 0;
  *err = hipGetDevice(&cur);
  if (*err != hipSuccess) return nullptr;
  int dev = cur;
  if (stream != nullptr) {
    *err = hipStreamGetDevice(stream, &dev);
    if (*err != hipSuccess) return nullptr;
  }
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    if (dev != cur && (*err = hipSetDevice(dev)) != hipSuccess) return nullptr;
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (*err == hipSuccess) *err = e2;
    }
    if (*err != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  *err = hipSuccess;
  return addr[dev];
}

}  // namespace pkv
