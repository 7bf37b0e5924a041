// Absorbed MLA decode for gfx950: one query token per request against a paged
// cache of 576-dim latent rows shared by every query head.
//
// "Beyond just running: native inference optimisation in vLLM on AMD ROCm",
// section "AITER MLA backend: optimised for DeepSeek": MLA compresses the KV
// cache to one 576-dim latent row per token; decode works directly in that
// latent space ("absorbed") and stays bound by memory bandwidth, so the
// kernel's job is to stream the latent rows at HBM speed.  The score of head
// h against token j is scale * <q_h, row_j> over all 576 dims; the value is
// the row's first 512 dims (the compressed KV; the last 64 carry the rotary
// key), so each head's output is a 512-dim latent.
//
// Work split as in the MHA decode: the requests' lengths (rounded up to the
// 16-token tile) are concatenated into one token stream cut into equal
// pieces; every wave independently owns (piece, group of up to 16 heads) and
// runs one segment per request the piece overlaps.  A tile is 16 tokens of
// one block (block sizes >= 16): 16 rows x 1152 bytes, contiguous in the
// cache, moved by the LDS copy engine (global_load_lds_dwordx4) into the
// wave's own LDS buffer -- 19 copy instructions per tile, rows padded to 73
// 16-byte slots so the operand reads below hit distinct banks -- while the
// previous tile is consumed (two buffers per wave, no barriers):
//   S^T (16 tokens x 16 heads) = K Q^T     18 x v_mfma_f32_16x16x32_bf16
//                                          (K rows from LDS, Q^T in registers)
//   online softmax per head                (4 tokens per lane + 2 shuffles)
//   O^T (512 dims x 16 heads) += V^T P^T   32 x v_mfma_f32_16x16x16_bf16
//                                          (V^T by transposed LDS reads;
//                                          P^T is the S^T accumulator)
// A segment that is a whole request writes the bf16 output; others write an
// fp32 partial (o, lse) in row p + b, merged by a log-sum-exp combine pass
// ("Processing details of the three paths": partial results carry the log of
// their softmax denominator).
#include "common.h"
#include "internal.h"

namespace pkv {
namespace {

constexpr int kLat = 576;                      // latent row (dims)
constexpr int kVal = 512;                      // value part
constexpr int kRowBytes = kLat * 2;            // 1152
constexpr int kTileTok = 16;
constexpr int kSlots = 73;                     // 72 16-byte chunks + 1 pad per LDS row
constexpr int kCopies = (kTileTok * kSlots + 63) / 64;   // 19 copy instructions per tile
constexpr int kBufBytes = kCopies * 1024;      // 19456
constexpr int kMWaves = 4;                     // one wave per SIMD (LDS: 8 buffers)
constexpr int kMlaPlanLds = 2000;              // batches up to this size plan in LDS
constexpr int kMThreads = 64 * kMWaves;
constexpr float kNegInf = -__builtin_huge_valf();

typedef short s16x4v_t __attribute__((ext_vector_type(4)));

struct MlaArgs {
  const uint8_t* cache;       // [num_blocks][bs][576] bf16
  const __bf16* q;            // [B][H][576]
  const int32_t* tables;
  const int32_t* seq_lens;
  __bf16* out;                // [B][H][512]
  float* lse;                 // [B][H] or null
  float* part_o;              // [part_rows][H][512]: row p + b for piece p of request b
  float* part_lse;            // [part_rows][H]
  int32_t* hdr;               // [0] padded total T, [1] piece length, [2] pieces
  int32_t* cum;               // [B+1] prefix sums of lengths rounded up to 16
  int32_t* first_seq;         // [max_pieces]
  int32_t max_blocks, num_blocks, bs, bs_log2, H, n_gchunks, batch, max_len;
  int32_t fixed_len, len_min, len_max, target_pieces;
  float qk_mult;              // scale * log2(e)
  int32_t lds_plan;           // 1: every workgroup plans in LDS (batch <= kMlaPlanLds)
};

__device__ __forceinline__ int32_t clamp_len16(int32_t L, int32_t cap) {
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ __forceinline__ int32_t mla_piece_len(const MlaArgs& a, int32_t T) {
  if (a.fixed_len > 0) return a.fixed_len;
  int32_t len = (T + a.target_pieces - 1) / a.target_pieces;
  len = (len + 15) & ~15;
  return len < a.len_min ? a.len_min : (len > a.len_max ? a.len_max : len);
}

// Plan (one workgroup): prefix sums of the lengths rounded up to 16, the
// piece length, and the first request of every piece.
__global__ __launch_bounds__(1024) void mla_plan_kernel(MlaArgs a) {
  __shared__ int32_t s_part[1024];
  const int tid = threadIdx.x;
  const int32_t B = a.batch;
  const int32_t per = (B + 1023) / 1024;
  const int32_t b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int32_t sum = 0;
  for (int32_t b = b0; b < b1; ++b) sum += (clamp_len16(a.seq_lens[b], a.max_len) + 15) & ~15;
  s_part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int32_t run = tid ? s_part[tid - 1] : 0;
  for (int32_t b = b0; b < b1; ++b) {
    a.cum[b] = run;
    run += (clamp_len16(a.seq_lens[b], a.max_len) + 15) & ~15;
  }
  const int32_t T = s_part[1023];
  const int32_t len = mla_piece_len(a, T);
  const int32_t NP = (T + len - 1) / len;
  if (tid == 0) {
    a.cum[B] = T;
    a.hdr[0] = T;
    a.hdr[1] = len;
    a.hdr[2] = NP;
  }
  __threadfence_block();
  __syncthreads();
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

// One copy instruction of a tile: 64 lanes x 16 bytes from sbase + voff into
// the 1 KB of LDS at lds (lane i at lds + 16 i).  m0 is saved and restored
// around it (a reserved register the compiler may not list as clobbered).
// Every latent row is read once per call, so the copy is non-temporal (`nt`):
// the rows stream past the caches instead of filling L2.
__device__ __forceinline__ void copy16(uint32_t lds, uint32_t voff, const void* sbase) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(sbase)
      : "memory");
}

__device__ __forceinline__ f32x4_t mfma16k16(s16x4v_t a, s16x4v_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Main pass: one wave = one worker (see the file comment).  Launched with one
// workgroup of 4 waves per CU.
__global__ __attribute__((amdgpu_flat_work_group_size(kMThreads, kMThreads), amdgpu_waves_per_eu(1, 1)))
void mla_piece_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves * 2 * kBufBytes];
  __shared__ int32_t s_cum[kMlaPlanLds + 1];
  __shared__ int32_t s_wsum[kMWaves];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int q4 = lane >> 4, r = lane & 15;
  uint8_t* buf0 = smem + wave * 2 * kBufBytes;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)buf0);

  // This lane's slot of each copy instruction: slot s = 64 j + lane holds
  // chunk s % 73 of row s / 73 (pad slots and slots past the tile re-read
  // chunk 0 of the row, or of row 0).
  uint32_t row_of[kCopies], chunk_of[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int s = 64 * j + lane;
    const int rr = s / kSlots, cc = s - rr * kSlots;
    row_of[j] = rr < kTileTok ? rr : 0;
    chunk_of[j] = (rr < kTileTok && cc < 72) ? cc : 0;
  }

  // The plan: prefix sums of the lengths rounded up to 16, the piece length
  // and the number of pieces.  Small batches plan in every workgroup's LDS
  // (8 requests per thread, a wave scan, then the wave totals), with no
  // dependent loads before the first copy; workgroup 0 also leaves the plan
  // in the workspace for the combine pass.  Larger batches read what
  // mla_plan_kernel left there.
  int32_t T, len, NP;
  if (a.lds_plan) {
    constexpr int kPer = (kMlaPlanLds + kMThreads - 1) / kMThreads;
    const int32_t b0 = (int32_t)threadIdx.x * kPer;
    int32_t v[kPer], sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      v[i] = b0 + i < a.batch ? (clamp_len16(a.seq_lens[b0 + i], a.max_len) + 15) & ~15 : 0;
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
    for (int w = 0; w < kMWaves; ++w) {
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
    len = mla_piece_len(a, T);
    NP = (T + len - 1) / len;
    if (blockIdx.x == 0) {
      for (int32_t b = threadIdx.x; b <= a.batch; b += kMThreads) a.cum[b] = s_cum[b];
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
  }
  auto cum_at = [&](int32_t b) -> int32_t { return a.lds_plan ? s_cum[b] : a.cum[b]; };
  // first request of piece p: the largest b with cum[b] <= p * len (empty
  // requests share their successor's offset, so the largest one is non-empty)
  auto first_of = [&](int32_t p) -> int32_t {
    if (!a.lds_plan) return a.first_seq[p];
    const int32_t start = p * len;
    int32_t lo = 0, hi = a.batch - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (s_cum[mid] <= start) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  const int64_t total_waves = (int64_t)gridDim.x * kMWaves;
  const int64_t n_items = (int64_t)NP * a.n_gchunks;

  for (int64_t item = (int64_t)blockIdx.x * kMWaves + wave; item < n_items; item += total_waves) {
    const int32_t p = (int32_t)(item / a.n_gchunks);
    const int32_t gc = (int32_t)(item - (int64_t)p * a.n_gchunks);
    const int32_t h_base = gc * 16;
    const int gcnt = min(16, a.H - h_base);
    const int32_t pstart = p * len, pend = min(T, pstart + len);
    for (int32_t b = uniform(first_of(p)); b < a.batch; ++b) {
      const int32_t cb = uniform(cum_at(b));
      if (cb >= pend) break;
      const int32_t L = uniform(clamp_len16(a.seq_lens[b], a.max_len));
      const int32_t t_begin = max(pstart, cb) - cb;       // multiple of 16
      const int32_t t_end = min(pend - cb, L);
      if (t_begin >= t_end) continue;
      const int32_t n_b = (cb + L - 1) / len - cb / len + 1;
      const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;

      // Q^T as the B operand: lane (q4, r) holds head h_base + r, dims
      // 32 kk + 8 q4 .. + 7
      bf16x8_t qb[18];
      {
        const bf16x8_t zero = {};
        const __bf16* qrow = a.q + ((int64_t)b * a.H + h_base + r) * kLat + 8 * q4;
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) qb[kk] = r < gcnt ? *(const bf16x8_t*)(qrow + 32 * kk) : zero;
      }

      // the block holding token t0 (looked up one tile ahead of its copies)
      auto lookup = [&](int32_t t0) -> int32_t { return trow[t0 >> a.bs_log2]; };
      // copies of the tile starting at token t0 (in block `blk`) into buffer
      // `bi`; rows past t_end repeat the last valid row (finite values for
      // masked keys)
      auto copy_tile = [&](int32_t t0, int bi, int32_t blk) {
        blk = __builtin_amdgcn_readfirstlane(blk);
        blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
        const uint8_t* base = a.cache + ((int64_t)blk * a.bs + (t0 & (a.bs - 1))) * kRowBytes;
        const uint32_t rmax = (uint32_t)min(kTileTok - 1, t_end - 1 - t0);
        const uint32_t lds = lds0 + bi * kBufBytes;
#pragma unroll
        for (int j = 0; j < kCopies; ++j) {
          const uint32_t rr = row_of[j] < rmax ? row_of[j] : rmax;
          copy16(lds + j * 1024, rr * kRowBytes + chunk_of[j] * 16, base);
        }
      };

      f32x4_t o[32];
#pragma unroll
      for (int n = 0; n < 32; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      float m_run = kNegInf, l_run = 0.f;

      const int32_t n_tiles = (t_end - t_begin + kTileTok - 1) / kTileTok;
      const int32_t blk0 = lookup(t_begin);
      int32_t blk_next = n_tiles > 1 ? lookup(t_begin + kTileTok) : 0;
      copy_tile(t_begin, 0, blk0);
      // The first tile, Q and the look-ahead lookup have landed.  The lookup
      // passes through the wait as an operand: otherwise the compiler, which
      // does not see the copies, waits on the vector-memory counter before
      // its first use -- and with it on the copies issued since.
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(blk_next)::"memory");
      // Q^T has landed with the first tile; tell the compiler, so it does not
      // wait on the vector-memory counter (and with it on the next tile's
      // copies) before the first MFMA of every tile.
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) asm volatile("" : "+v"(qb[kk]));

      for (int32_t it = 0; it < n_tiles; ++it) {
        const int32_t t0 = t_begin + it * kTileTok;
        const int bi = it & 1;
        if (it + 1 < n_tiles) {
          const int32_t blk1 = blk_next;
          if (it + 2 < n_tiles) blk_next = lookup(t0 + 2 * kTileTok);
          copy_tile(t0 + kTileTok, bi ^ 1, blk1);
          // this tile's copies (and the lookup issued before the new ones)
          // have landed; only the 19 copies of the next tile may be in flight
          asm volatile("s_waitcnt vmcnt(19)" : "+v"(blk_next)::"memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const uint8_t* tl = buf0 + bi * kBufBytes;

        // ---- S^T = K Q^T: element i of acc is token t0 + 4 q4 + i, head r
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 18; ++kk)
          acc = mfma16(*(const bf16x8_t*)(tl + (r * kSlots + 4 * kk + q4) * 16), qb[kk], acc);

        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[i] = t0 + 4 * q4 + i < t_end ? acc[i] * a.qk_mult : kNegInf;
        float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // lazy rescale: the reference only moves when a head's maximum grew
        // by more than 8 (log2 domain), so p <= 2^8 and most tiles skip it
        if (__builtin_amdgcn_ballot_w64(mt > m_run + 8.f) != 0) {
          const float m_new = fmaxf(m_run, mt);
          const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
          l_run *= alpha;
#pragma unroll
          for (int n = 0; n < 32; ++n) o[n] *= alpha;
          m_run = m_new;
        }
        const float m_use = m_run == kNegInf ? 0.f : m_run;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = fast_exp2(sc[i] - m_use);
          l_run += pv[i];
        }
        const bf16x4_t pb4 = {(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
        const s16x4v_t pb = __builtin_bit_cast(s16x4v_t, pb4);

        // ---- O^T += V^T P^T: lane (q4, r) of the transposed read gets dim
        // 16 n + r of tokens 4 q4 .. 4 q4 + 3
        const int e = r >> 2, m = r & 3;
        const uint8_t* vb = tl + ((4 * q4 + e) * kSlots + (m >> 1)) * 16 + (m & 1) * 8;
#pragma unroll
        for (int n = 0; n < 32; ++n) {
          const s16x4_t vt = lds_read_tr16(vb + 32 * n);
          o[n] = mfma16k16(vt, pb, o[n]);
        }
      }

      // ---- result of the segment: head h_base + r, dims 16 n + 4 q4 + i
      float l_sum = l_run;
      l_sum += __shfl_xor(l_sum, 16);
      l_sum += __shfl_xor(l_sum, 32);
      if (r < gcnt) {
        const int64_t bh = (int64_t)b * a.H + h_base + r;
        const float f = 1.f / l_sum;
        const float lse_v = (m_run + __log2f(l_sum)) * kLn2;
        if (n_b == 1) {
#pragma unroll
          for (int n = 0; n < 32; ++n) {
            const f32x4_t v = o[n] * f;
            const bf16x4_t v4 = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            *(bf16x4_t*)(a.out + bh * kVal + 16 * n + 4 * q4) = v4;
          }
          if (q4 == 0 && a.lse) a.lse[bh] = lse_v;
        } else {
          const int64_t prow = (int64_t)(p + b) * a.H + h_base + r;
          float* po = a.part_o + prow * kVal;
#pragma unroll
          for (int n = 0; n < 32; ++n) *(f32x4_t*)(po + 16 * n + 4 * q4) = o[n] * f;
          if (q4 == 0) a.part_lse[prow] = lse_v;
        }
      }
    }
  }
}

// LSE merge of the pieces of every request that spans several pieces; one
// wave per (request, head); a request of length 0 gets out = 0, lse = -inf.
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaArgs a) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + wave;
  if (bh >= (int64_t)a.batch * a.H) return;
  const int32_t b = (int32_t)(bh / a.H);
  const int32_t h = (int32_t)(bh - (int64_t)b * a.H);
  const int32_t L = clamp_len16(a.seq_lens[b], a.max_len);
  bf16x8_t* dst = (bf16x8_t*)(a.out + bh * kVal) + lane;
  if (L == 0) {
    *dst = bf16x8_t{};
    if (lane == 0 && a.lse) a.lse[bh] = kNegInf;
    return;
  }
  const int32_t len = a.hdr[1];
  const int32_t cb = a.cum[b];
  const int32_t n_b = (cb + L - 1) / len - cb / len + 1;
  if (n_b <= 1) return;                        // written by the main pass
  const int64_t row0 = (int64_t)(cb / len + b) * a.H + h;
  // chunks of 8 partials, every load of a chunk issued up front; the running
  // maximum and weights are carried across chunks
  float M = kNegInf;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  float wsum = 0.f;
  constexpr int kU = 8;
  for (int c0 = 0; c0 < n_b; c0 += kU) {
    float lv[kU];
    f32x4_t o0[kU], o1[kU];
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int64_t row = row0 + (int64_t)(c0 + i) * a.H;
      const bool ok = c0 + i < n_b;
      const f32x4_t* po = (const f32x4_t*)(a.part_o + row * kVal) + 2 * lane;
      lv[i] = ok ? a.part_lse[row] : kNegInf;
      o0[i] = ok ? po[0] : f32x4_t{0.f, 0.f, 0.f, 0.f};
      o1[i] = ok ? po[1] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float Mc = M;
#pragma unroll
    for (int i = 0; i < kU; ++i) Mc = fmaxf(Mc, lv[i]);
    if (c0 > 0) {
      const float sc = fast_exp2((M - Mc) * kLog2e);
      wsum *= sc;
      acc0 *= sc;
      acc1 *= sc;
    }
    M = Mc;
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const float wgt = c0 + i < n_b ? fast_exp2((lv[i] - M) * kLog2e) : 0.f;
      wsum += wgt;
      acc0 += wgt * o0[i];
      acc1 += wgt * o1[i];
    }
  }
  const float inv = 1.f / wsum;
  *dst = bf16x8_t{(__bf16)(acc0[0] * inv), (__bf16)(acc0[1] * inv), (__bf16)(acc0[2] * inv),
                  (__bf16)(acc0[3] * inv), (__bf16)(acc1[0] * inv), (__bf16)(acc1[1] * inv),
                  (__bf16)(acc1[2] * inv), (__bf16)(acc1[3] * inv)};
  if (lane == 0 && a.lse) a.lse[bh] = M + __log2f(wsum) * kLn2;
}

int32_t log2_of(int32_t v) {
  int32_t l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

MlaPlan plan_mla(int32_t batch, int32_t num_heads, int32_t max_seq_len, hipStream_t stream) {
  MlaPlan p;
  p.n_gchunks = (num_heads + 15) / 16;
  p.waves = device_cu_count(stream) * kMWaves;
  p.target_pieces = p.waves / p.n_gchunks > 0 ? p.waves / p.n_gchunks : 1;
  p.len_min = 64;
  p.len_max = 16384;
  const int64_t padded = (int64_t)batch * ((max_seq_len + 15) & ~15);
  int64_t np = (padded + p.len_max - 1) / p.len_max;
  if (np < p.target_pieces) np = p.target_pieces;
  p.max_pieces = (int32_t)(np + 1);
  p.part_rows = p.max_pieces + batch;
  return p;
}

size_t mla_workspace_bytes(const MlaPlan& p, int32_t batch, int32_t num_heads) {
  const size_t rows = (size_t)p.part_rows * num_heads;
  return 256 + align256((size_t)(batch + 1) * 4) + align256((size_t)p.max_pieces * 4) +
         align256(rows * kVal * sizeof(float)) + align256(rows * sizeof(float));
}

hipError_t launch_mla_decode(const MlaPlan& p, const void* cache, int32_t num_blocks,
                             int32_t block_size, const void* q, int32_t batch, int32_t num_heads,
                             const int32_t* tables, int32_t max_blocks, const int32_t* seq_lens,
                             int32_t max_seq_len, float scale, void* out, float* lse,
                             void* workspace, hipStream_t s) {
  MlaArgs a;
  a.cache = (const uint8_t*)cache;
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
  const size_t rows = (size_t)p.part_rows * num_heads;
  a.part_o = (float*)w;
  w += align256(rows * kVal * sizeof(float));
  a.part_lse = (float*)w;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.bs = block_size;
  a.bs_log2 = log2_of(block_size);
  const int64_t capacity = (int64_t)max_blocks << a.bs_log2;
  a.max_len = (int32_t)(capacity < max_seq_len ? capacity : max_seq_len);
  a.H = num_heads;
  a.n_gchunks = p.n_gchunks;
  a.batch = batch;
  a.fixed_len = 0;
  a.len_min = p.len_min;
  a.len_max = p.len_max;
  a.target_pieces = p.target_pieces;
  a.qk_mult = scale * kLog2e;
  a.lds_plan = batch <= kMlaPlanLds ? 1 : 0;
  hipError_t e;
  if (!a.lds_plan) {
    hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(1024), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mla_piece_kernel, dim3((unsigned)(p.waves / kMWaves)), dim3(kMThreads), 0, s,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t bh = (int64_t)batch * num_heads;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((bh + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
