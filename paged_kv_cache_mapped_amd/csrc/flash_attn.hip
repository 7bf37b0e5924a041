// Prefill and extend attention for gfx950: an MFMA flash-attention tile core.
//
// "Beyond just running: native inference optimisation in vLLM on AMD ROCm":
// * section "Every batch handles a mixed workload": prefill is large matrix
//   products (compute bound, wants big tiles and high ALU use); extend attends
//   both to the cached context and to this round's new tokens;
// * section "ROCM_AITER_FA": prefill runs a variable-length flash-attention
//   kernel on the matrix cores; long contexts are processed in chunks under a
//   per-iteration token budget (about 32K) shared by the extend requests and
//   merged by log-sum-exp;
// * section "Processing details of the three paths": prefill Q/K/V use the
//   [num_tokens, num_heads, head_dim] layout; extend = (1) new tokens among
//   themselves, (2) per context chunk: attention of the new tokens to the chunk
//   and an LSE merge, (3) a final merge.  Each chunk yields an output and an
//   LSE that records its softmax denominator.
//
// Tile core.  A workgroup of 8 waves owns 256 query rows that read the same
// keys -- P = gcd(G, 8) query heads of one KV head over 256 / P consecutive
// tokens, each wave one head over 32 tokens -- and walks the key range in
// tiles of 64 keys staged in LDS (double buffered: the next tile is moved from
// global memory straight into the other LDS buffer by global_load_lds_dwordx4
// while the current one is consumed, with no staging registers).  Each tile
// copied serves 256 query rows.  Per tile each wave computes
//     S^T (64 keys x 32 rows) = K Q^T         16 x v_mfma_f32_32x32x16_bf16
//     online softmax per row in registers     (a row's 64 scores live in two
//                                              lanes: in-lane max/sum + one
//                                              cross-lane exchange)
//     O^T (128 dims x 32 rows) += V^T P^T      16 x v_mfma_f32_32x32x16_bf16
// Q^T stays in registers as the B operand; K rows are read from LDS as the A
// operand; V^T comes out of the natural row-major V tile through
// ds_read_b64_tr_b16 (transposing LDS read); rows are unpadded, their 16-byte
// chunks permuted per row so both read patterns are free of bank conflicts;
// P^T is the S^T accumulator converted to bf16 in place (its lane layout
// already is the B-operand layout once the 16 keys of an MFMA k-step are taken
// in the order the accumulator holds them).  Scores are kept in the exp2
// domain (scale * log2 e folded in).
//
// Keys are read either from contiguous [tokens, H_kv, D] tensors (prefill, and
// the new tokens of an extend) or straight from the paged NHD cache through
// the block table (extend context chunks) -- no gather copy.
//
// Prefill runs persistent: one workgroup per CU walks a fixed serpentine
// list of work items and, during the last key tile of each, copies the next
// item's Q rows and first K/V tile into LDS, so consecutive items follow each
// other without a start-up wait; outputs leave through LDS as whole rows.
// The extend kernels are launched one workgroup per work item.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace pkv {
namespace {

constexpr int kD = 128;
constexpr int kBM = 128;                   // query tile of the work-size heuristics
constexpr int kWGRows = 256;               // query rows (token, head) per workgroup
constexpr int kWaves = 8;                  // one query head x 32 tokens each
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;                    // keys per tile
constexpr int kRowB = 256;                 // LDS bytes per K or V row (unpadded)
constexpr int kKTile = kBN * kRowB;
constexpr int kVTile = kBN * kRowB;
constexpr int kStage = kKTile + kVTile;    // 32768 bytes
constexpr float kNegInf = -__builtin_huge_valf();

struct AttnArgs {
  const __bf16* q;          // [rows][Hq][D]
  const __bf16* k;          // [rows][Hkv][D]  (prefill keys / extend new keys)
  const __bf16* v;
  const int32_t* cu;        // [num_seqs+1] row offsets
  const uint8_t* kc;        // paged NHD cache (extend context)
  const uint8_t* vc;
  const int32_t* tables;
  const int32_t* ctx_lens;
  __bf16* out;
  float* lse;
  float* part_o;            // [n_parts][rows][Hq][D]
  float* part_lse;          // [n_parts][rows][Hq]
  int32_t max_blocks, num_blocks, bs, bs_log2;
  int32_t Hq, Hkv, G, num_seqs, n_parts, chunk_tokens, rows;
  int32_t P;                // query heads per workgroup (gcd(G, 8)): wave w takes head
                            // w % P of the lane's P heads, tokens 32 (w / P) .. + 31
  int32_t TW;               // tokens per workgroup: kWGRows / P
  int32_t Gs;               // lanes per KV head: G / P
  int32_t n_qitems;         // query items per lane: TW-token slices of the sequence
  int64_t items;            // lanes (work items = lanes x query items)
  int64_t grid_pad;         // launched workgroups (multiple of 8)
  int32_t qt_major;         // work order inside an XCD's share of lanes
  int32_t lchunk;           // lanes kept together on one XCD (query heads sharing a KV head)
  float qk_mult;            // scale * log2(e)
  // context scores and values of an fp8 cache: code * k_scale, code * v_scale
  float ctx_qk_mult;        // scale * k_scale * log2(e)
  float ctx_vexp;           // log2(v_scale): added to the exponent of p
  float ctx_linv;           // 1 / v_scale: takes it back out of the row sum
  // hybrid extend (see extend_plan_kernel): the plan and the work list in
  // the workspace
  const int32_t* plan;
  const struct ListEntry* list;
  int32_t max_split;        // split request slots
  int32_t list_cap;         // work-list entries the workspace holds
  int32_t plan_slots;       // workgroups the GPU holds at once (one per CU)
};

// Work order.  A work item is (lane, query item), lanes being the
// (sequence[, part], KV head, group of P query heads) combinations in that
// order.  A workgroup of 8 waves runs 256 query rows that share every K/V tile
// it copies into LDS: P query heads of one KV head over TW = 256 / P
// consecutive tokens, each wave one head over 32 tokens (P = gcd(G, 8): eight
// heads over 32 tokens for groups of 8 or 16, one head over 256 tokens for an
// odd group).  Short requests then fill their rows, and a workgroup's causal
// diagonal is TW tokens long.
// Launched workgroup L runs on XCD L % 8, and the hardware hands workgroups
// out in launch order as CUs free up.  Lanes are dealt to the XCDs in chunks
// of lchunk consecutive lanes (half the head groups of one KV head): the
// heads of a chunk share its K/V tiles in that XCD's L2, and the lanes of one
// request -- 2 * H_kv chunks -- are spread over the XCDs, so a request that
// is much longer than the others (a heavy-tailed batch) is worked on by the
// whole GPU rather than by one or two XCDs.  Inside an XCD's share the order
// is either query-tile-major with
// the last query tiles (the heaviest under a causal mask) first, so the
// in-order hand-out is a longest-first schedule (causal prefill, short
// extends), or lane-major (a lane's tiles back to back, last first), which
// keeps the workgroups of an XCD on fewer K/V streams when every tile costs
// about the same (long non-causal work).  grid_pad = 8 * hx * n_qitems, hx a
// multiple of lchunk.
struct WorkItem {
  int64_t lane;
  int32_t qi;
};
template <class Args>
__device__ __forceinline__ WorkItem work_item_in(const Args& a, int64_t L, int64_t grid_pad,
                                                 int32_t n_qitems) {
  const int64_t hx = grid_pad / (8 * (int64_t)n_qitems);
  const int64_t j = L >> 3;
  WorkItem w;
  int64_t l;                    // this XCD's l-th lane
  if (a.qt_major) {
    w.qi = n_qitems - 1 - (int32_t)(j / hx);
    l = j % hx;
  } else {
    w.qi = n_qitems - 1 - (int32_t)(j % n_qitems);
    l = j / n_qitems;
  }
  // chunks of lchunk consecutive lanes are dealt to the XCDs in turn
  const int64_t c = a.lchunk;
  w.lane = ((l / c) * 8 + (L & 7)) * c + l % c;
  return w;
}
template <class Args>
__device__ __forceinline__ WorkItem work_item(const Args& a, int64_t L) {
  return work_item_in(a, L, a.grid_pad, a.n_qitems);
}
static int64_t work_grid(int64_t lanes, int32_t n_qitems, int32_t lchunk) {
  return 8 * (((lanes + 8 * lchunk - 1) / (8 * lchunk)) * lchunk) * (int64_t)n_qitems;
}
// Persistent walk: the launched grid holds one workgroup per CU (a multiple of
// 8); launched workgroup b runs the virtual workgroups 8m + (b & 7) of its
// XCD, m = r J + j in even rounds r and r J + J - 1 - j in odd ones (j = b / 8,
// J = workgroups per XCD): a serpentine over the heaviest-first order.
// Returns -1 past the end.
template <class Args>
__device__ __forceinline__ int64_t virtual_wg(const Args& a, int32_t r) {
  const int32_t J = gridDim.x >> 3, j = blockIdx.x >> 3;
  const int64_t m = (int64_t)r * J + ((r & 1) ? J - 1 - j : j);
  return m < (a.grid_pad >> 3) ? 8 * m + (blockIdx.x & 7) : -1;
}
static unsigned persistent_grid(int64_t grid_pad, hipStream_t stream) {
  const int64_t slots = 8 * (int64_t)(device_cu_count(stream) / 8);
  return (unsigned)(grid_pad < slots ? grid_pad : slots);
}

// This wave's rows of work item (KV head hkv, head group gsel, query item qi):
// query head h over tokens q0w .. q0w + 31; the workgroup's tokens are
// [q0_lo, q_end) (they bound the keys it needs under a causal mask).
struct RowBlock {
  int32_t h, q0w, q0_lo, q_end;
};
template <class Args>
__device__ __forceinline__ RowBlock row_block(const Args& a, int32_t hkv, int32_t gsel,
                                              int32_t qi) {
  const int w = wave_id();
  RowBlock r;
  r.h = hkv * a.G + gsel * a.P + (w & (a.P - 1));
  r.q0_lo = qi * a.TW;
  r.q_end = r.q0_lo + a.TW;
  r.q0w = r.q0_lo + 32 * (w / a.P);
  return r;
}

struct KeySrc {
  const uint8_t* kb;        // contiguous: K of key 0; paged: cache base
  const uint8_t* vb;
  const int32_t* trow;      // paged only
  int32_t hkv;
};

template <bool PAGED, class Args>
__device__ __forceinline__ int64_t key_row_bytes(const Args& a, const KeySrc& s, int32_t key) {
  if constexpr (PAGED) {
    int32_t blk = s.trow[key >> a.bs_log2];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    const int64_t slot = (int64_t)blk * a.bs + (key & (a.bs - 1));
    return (slot * a.Hkv + s.hkv) * (kD * 2);
  } else {
    return ((int64_t)key * a.Hkv + s.hkv) * (kD * 2);
  }
}




// Rows are stored unpadded with their 16-byte chunks permuted: K chunk c of
// row r at position c ^ (r & 15) (the 32 rows of an MFMA operand read hit
// distinct banks), V chunk c at c ^ 4(r & 3) (the transposed reads touch 4
// rows x 4 chunks at a time).
__device__ __forceinline__ int kswz(int row, int c) { return row * kRowB + ((c ^ (row & 15)) << 4); }
__device__ __forceinline__ int vswz(int row, int c) { return row * kRowB + ((c ^ ((row & 3) << 2)) << 4); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)p);
}
// The lane index through an asm the compiler cannot move, so that per-lane
// address arithmetic at item boundaries is not hoisted out of the item loop
// (it would hold registers during the whole key loop).
__device__ __forceinline__ int lane_here() {
  uint32_t lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return (int)lane;
}

// 64 lanes' 16-byte global pieces into one contiguous 1 KB of LDS (lane i at
// m0 + 16 i), with no staging registers.  Not known to the compiler: the
// caller waits for them (vmcnt) before the barrier that publishes the stage.
// m0 is a reserved register the compiler may not list as clobbered, so each
// copy saves it into a scratch SGPR and restores it afterwards: whatever the
// compiler keeps in m0 survives the copy.
__device__ __forceinline__ void dma16(uint32_t lds_base, const void* g) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(g)
      : "memory");
}
__device__ __forceinline__ void dma16s(uint32_t lds_base, uint32_t voff, const void* sbase) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(sbase)
      : "memory");
}
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Whether the tile starting at k0 is one whose wave rows are contiguous in
// memory: contiguous keys, or (paged) one 16-token block per wave.
template <bool PAGED, class Args>
__device__ __forceinline__ bool whole_tile(const Args& a, int32_t k0, int32_t k_end) {
  return PAGED ? (a.bs == 16 && (k0 & 15) == 0 && k0 + kBN <= k_end) : (k0 + kBN <= k_end);
}

// The block-table entry of this wave's 8 rows of the whole paged tile at k0
// (0 when the tile is not such a tile).  Looked up one tile ahead of the copy
// that uses it: the value is first read by the next tile's copy, after the
// current tile's wait, so neither the lookup nor the copy stalls.
template <bool PAGED, class Args>
__device__ __forceinline__ int32_t tile_block(const Args& a, const KeySrc& s, int32_t k0,
                                              int32_t k_end) {
  if constexpr (PAGED) {
    return whole_tile<PAGED>(a, k0, k_end) ? s.trow[(k0 >> 4) + (wave_id() >> 1)] : 0;
  } else {
    return 0;
  }
}

// Wait for this wave's copies, and tell the compiler that the look-ahead
// lookup issued with them has landed too (it takes the value as an operand).
// Without that, the compiler still counts the lookup as in flight and, before
// the register is next written, waits on the vector-memory counter -- which
// then also waits for the copy just issued for the following tile.
__device__ __forceinline__ void dma_wait_for(int32_t& lookup) {
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(lookup)::"memory");
}

// Cache kinds of the extend's cached context.  NHD bf16 rows already are the
// LDS rows the core reads, so the copy engine moves them as they are.  The
// other kinds are loaded into registers one tile ahead (issued at the start
// of a tile, stored at its end), decoded to bf16 -- exact: every e4m3fn value
// is a bf16 value -- and written into the same LDS rows, so the core is the
// same for every cache ("Beyond just running: native inference optimisation
// in vLLM on AMD ROCm", section "ROCM_AITER_FA": the preshuffled layout
// k [block][head][D/x][block_size][x], v [block][head][block_size/x][D][x];
// the pages gather it into a contiguous copy first, this reads it in place).
enum : int { kCtxNhdBf16 = 0, kCtxNhdFp8 = 1, kCtxPreBf16 = 2, kCtxPreFp8 = 3 };

// One thread's share of a context tile in flight (raw cache bytes).
struct Staged {
  u32x4_t k[2], v[2];
};

// Issue the loads of this thread's share of the 64-key context tile at k0.
//  NHD fp8: thread t takes 16 dims (16 bytes) of K and V of key t / 8; keys
//    past kend repeat the last key, as in the copy-engine path.
//  preshuffled (block size 16): thread t works in the tile's block t / 128
//    (a block wholly past kend is read from block 0 and zeroed when stored,
//    so no table entry past the range is read).  bf16: K pieces (one token x
//    8 dims) t % 128 and t % 128 + 128; V dims 2p and 2p + 1 of tokens 8g ..
//    8g + 7 (p = t % 64, g = t % 128 / 64).  fp8: the K piece (one token x 16
//    dims) t % 128; V dims 2p, 2p + 1 of tokens 8g .. 8g + 7 (8 bytes each).
template <int KIND, class Args>
__device__ __forceinline__ void stage_load(const Args& a, const KeySrc& s, int32_t k0,
                                           int32_t kend, Staged& R) {
  const int th = threadIdx.x;
  if constexpr (KIND == kCtxNhdFp8) {
    const int r = th >> 3, j = th & 7;
    const int32_t key = min(k0 + r, kend - 1);
    int32_t blk = s.trow[key >> a.bs_log2];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    const int64_t row = ((int64_t)blk * a.bs + (key & (a.bs - 1))) * a.Hkv + s.hkv;
    R.k[0] = *(const u32x4_t*)(s.kb + row * kD + 16 * j);
    R.v[0] = *(const u32x4_t*)(s.vb + row * kD + 16 * j);
  } else {
    const int b4 = th >> 7, i = th & 127;
    const int32_t kb = k0 + 16 * b4;
    int32_t blk = 0;
    if (kb < kend) blk = s.trow[kb >> 4];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    const int p = i & 63, g = i >> 6;
    if constexpr (KIND == kCtxPreBf16) {
      const int64_t base = ((int64_t)blk * a.Hkv + s.hkv) * 4096;
      R.k[0] = *(const u32x4_t*)(s.kb + base + 16 * i);
      R.k[1] = *(const u32x4_t*)(s.kb + base + 16 * (i + 128));
      R.v[0] = *(const u32x4_t*)(s.vb + base + (g * 128 + 2 * p) * 16);
      R.v[1] = *(const u32x4_t*)(s.vb + base + (g * 128 + 2 * p + 1) * 16);
    } else {
      const int64_t base = ((int64_t)blk * a.Hkv + s.hkv) * 2048;
      R.k[0] = *(const u32x4_t*)(s.kb + base + 16 * i);
      const u32x2_t v0 = *(const u32x2_t*)(s.vb + base + (2 * p) * 16 + 8 * g);
      const u32x2_t v1 = *(const u32x2_t*)(s.vb + base + (2 * p + 1) * 16 + 8 * g);
      R.v[0] = u32x4_t{v0[0], v0[1], v1[0], v1[1]};
    }
  }
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// Decode this thread's share (loaded by stage_load) into the LDS rows of the
// tile at k0 in `stage` (K rows kswz, V rows vswz, bf16).  Keys at or past
// kend are stored as zeros (their scores are masked; their values must be
// finite).
template <int KIND>
__device__ __forceinline__ void stage_store(const Staged& R, uint8_t* stage, int32_t k0,
                                            int32_t kend) {
  const int th = threadIdx.x;
  uint8_t* kl = stage;
  uint8_t* vl = stage + kKTile;
  if constexpr (KIND == kCtxNhdFp8) {
    const int r = th >> 3, j = th & 7;
    *(bf16x8_t*)(kl + kswz(r, 2 * j)) = fp8x8_to_bf16(u32x2_t{R.k[0][0], R.k[0][1]});
    *(bf16x8_t*)(kl + kswz(r, 2 * j + 1)) = fp8x8_to_bf16(u32x2_t{R.k[0][2], R.k[0][3]});
    *(bf16x8_t*)(vl + vswz(r, 2 * j)) = fp8x8_to_bf16(u32x2_t{R.v[0][0], R.v[0][1]});
    *(bf16x8_t*)(vl + vswz(r, 2 * j + 1)) = fp8x8_to_bf16(u32x2_t{R.v[0][2], R.v[0][3]});
  } else {
    const int b4 = th >> 7, i = th & 127;
    const int p = i & 63, g = i >> 6;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    if constexpr (KIND == kCtxPreBf16) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int piece = i + 128 * u, row = 16 * b4 + (piece & 15);
        *(u32x4_t*)(kl + kswz(row, piece >> 4)) = k0 + row < kend ? R.k[u] : zero;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 16 * b4 + 8 * g + j;
        const uint32_t lo = (R.v[0][j >> 1] >> (16 * (j & 1))) & 0xffffu;
        const uint32_t hi = (R.v[1][j >> 1] >> (16 * (j & 1))) & 0xffffu;
        *(uint32_t*)(vl + vswz(row, p >> 2) + 4 * (p & 3)) = k0 + row < kend ? (lo | (hi << 16)) : 0u;
      }
    } else {
      const int row = 16 * b4 + (i & 15), c16 = i >> 4;
      const bool ok = k0 + row < kend;
      const bf16x8_t zb = {};
      const bf16x8_t lo = fp8x8_to_bf16(u32x2_t{R.k[0][0], R.k[0][1]});
      const bf16x8_t hi = fp8x8_to_bf16(u32x2_t{R.k[0][2], R.k[0][3]});
      *(bf16x8_t*)(kl + kswz(row, 2 * c16)) = ok ? lo : zb;
      *(bf16x8_t*)(kl + kswz(row, 2 * c16 + 1)) = ok ? hi : zb;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        // tokens 8g + 4 h2 .. + 3 of dims 2p (word h2) and 2p + 1 (word 2 + h2)
        const f32x2_t d0a = __builtin_amdgcn_cvt_pk_f32_fp8((int)R.v[0][h2], false);
        const f32x2_t d0b = __builtin_amdgcn_cvt_pk_f32_fp8((int)R.v[0][h2], true);
        const f32x2_t d1a = __builtin_amdgcn_cvt_pk_f32_fp8((int)R.v[0][2 + h2], false);
        const f32x2_t d1b = __builtin_amdgcn_cvt_pk_f32_fp8((int)R.v[0][2 + h2], true);
        const uint32_t w[4] = {bf16_pair(d0a[0], d1a[0]), bf16_pair(d0a[1], d1a[1]),
                               bf16_pair(d0b[0], d1b[0]), bf16_pair(d0b[1], d1b[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rw = 16 * b4 + 8 * g + 4 * h2 + e;
          *(uint32_t*)(vl + vswz(rw, p >> 2) + 4 * (p & 3)) = k0 + rw < kend ? w[e] : 0u;
        }
      }
    }
  }
}

// Tile starting at key k0 (keys past k_end clamped to the last key) into the
// stage at `stage`: wave w moves rows 8w..8w+7 of K and of V.  Whole tiles
// whose wave rows are contiguous in memory (contiguous keys, or half of one
// 16-token block of the paged cache, `blk` its table entry from tile_block)
// use a uniform base and per-lane 32-bit offsets.
template <bool PAGED, class Args>
__device__ __forceinline__ void dma_tile(const Args& a, const KeySrc& s, uint8_t* stage,
                                         int32_t k0, int32_t k_end, int32_t blk) {
  uint32_t lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int wave = wave_id();
  const int pc = lane & 15;
  const uint32_t kb = lds_addr(stage), vb = lds_addr(stage + kKTile);
  if (whole_tile<PAGED>(a, k0, k_end)) {
    const int64_t row_stride = (int64_t)a.Hkv * (kD * 2);
    int64_t tb;
    if constexpr (PAGED) {
      blk = __builtin_amdgcn_readfirstlane(blk);
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
      tb = ((int64_t)blk * 16 - 16 * (wave >> 1)) * row_stride + s.hkv * (kD * 2);
    } else {
      tb = (int64_t)k0 * row_stride + s.hkv * (kD * 2);
    }
    const uint8_t* kbase = s.kb + tb;
    const uint8_t* vbase = s.vb + tb;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 8 * wave + 4 * j + (lane >> 4);
      const uint32_t ro = (uint32_t)(row * row_stride);
      const uint32_t off = __builtin_amdgcn_readfirstlane((2 * wave + j) * 1024);
      dma16s(kb + off, ro + ((pc ^ (row & 15)) << 4), kbase);
      dma16s(vb + off, ro + ((pc ^ ((row & 3) << 2)) << 4), vbase);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = 2 * wave + j;
    const int row = 4 * q + (lane >> 4);
    int32_t key = k0 + row;
    key = key < k_end ? key : k_end - 1;
    const int64_t rb = key_row_bytes<PAGED>(a, s, key);
    const uint32_t off = __builtin_amdgcn_readfirstlane(q * 1024);
    dma16(kb + off, s.kb + rb + ((pc ^ (row & 15)) << 4));
    dma16(vb + off, s.vb + rb + ((pc ^ ((row & 3) << 2)) << 4));
  }
}

// Per-wave state of its 32 query rows: Q^T (B operand), O^T accumulators
// and the running exp2-domain max / lane-partial sum of each lane's row.
struct RowState {
  bf16x8_t qb[8];
  f32x16_t o[4];
  float m_run, l_run;
};

// Load Q (this wave's rows q0w .. q0w + 31 of a sequence whose row 0 is
// global row qbase) and clear the running state.
__device__ __forceinline__ void init_rows(const AttnArgs& a, int32_t h, int64_t qbase, int32_t q0w,
                                          int32_t qn, RowState& S) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int32_t row = q0w + r;
  // Q^T as the B operand: lane holds q[row][16*ks + 8*hh .. +8], ks = 0..7
  const bf16x8_t zero = {};
  const __bf16* qp = a.q + ((qbase + row) * a.Hq + h) * kD + 8 * hh;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) S.qb[ks] = row < qn ? *(const bf16x8_t*)(qp + 16 * ks) : zero;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) S.o[dt][i] = 0.f;
  S.m_run = kNegInf;
  S.l_run = 0.f;
}

// The tile loop folding keys [k_begin, kend) (n_tiles tiles of kBN) into the
// running state of this wave's rows (tokens q0w .. q0w + 31; the workgroup's
// first token is q0_lo).  CAUSAL: key j is visible to row i iff j <= i
// (keys and rows indexed within the sequence).  On entry the first tile is in
// LDS buffer SB, published by a barrier, and blk_next holds the table entry
// of the second one (paged keys).  Tile t is in buffer (t + SB) & 1; each step
// copies the next tile into the other buffer.  hooks.last(buffer) runs at the
// start of the last tile, when the other buffer is free: a persistent
// workgroup copies its next work item's first tile there.
struct NoHooks {
  __device__ __forceinline__ void last(uint8_t*) const {}
};
template <bool PAGED, bool CAUSAL, int SB, class Hooks, class Args, int KIND = kCtxNhdBf16>
__device__ __forceinline__ void key_loop(const Args& a, uint8_t* smem, const KeySrc& src,
                                         int32_t q0w, int32_t q0_lo, int32_t k_begin, int32_t kend,
                                         int32_t n_tiles, int32_t blk_next, RowState& S,
                                         const Hooks& hooks) {
  const int lane = lane_here();
  const int r = lane & 31, hh = lane >> 5;      // MFMA column (query row) / k-half
  const int g16 = lane >> 4, l16 = lane & 15;   // 16-lane group for transposed reads
  const int32_t row = q0w + r;                  // this lane's query row (in sequence)
  const float qk = KIND == kCtxNhdBf16 ? a.qk_mult : a.ctx_qk_mult;
  const float vexp = a.ctx_vexp, linv = a.ctx_linv;

  // One key tile.  MASK = false for tiles that no row of the workgroup needs
  // masked (the whole tile is inside the key range and, for causal blocks,
  // below the diagonal of the first row); the mask code is not emitted there.
  // This lane's LDS byte offsets of its K fragments (k-step ks, rows r and
  // r + 32 differ by a constant) and V^T fragments (dims 32 dt + ..; key
  // steps and the +8 row half differ by constants), computed once.
  uint32_t koff[8], voff[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = kswz(r, 2 * ks + hh);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int colb = (32 * dt + 16 * (g16 & 1) + 4 * (l16 & 3)) * 2;
    voff[dt] = kKTile + vswz(4 * (g16 >> 1) + (l16 >> 2), colb >> 4) + (colb & 15);
  }

  // One key tile in LDS buffer `par` (a compile-time 0/1 in the main loop,
  // so buffer offsets fold into the LDS instructions' immediates).
  auto step = [&](int32_t t, auto mask_tag, auto par, auto last_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool LAST = decltype(last_tag)::value;
    const int32_t k0 = k_begin + t * kBN;
    uint8_t* st = smem + par * kStage;
    Staged R;
    if constexpr (!LAST) {
      if constexpr (KIND == kCtxNhdBf16) {
        dma_tile<PAGED>(a, src, smem + (1 - par) * kStage, k0 + kBN, kend, blk_next);
        if (t + 2 < n_tiles) blk_next = tile_block<PAGED>(a, src, k0 + 2 * kBN, kend);
      } else {
        stage_load<KIND>(a, src, k0 + kBN, kend, R);
      }
    }

    // A diagonal tile whose first key lies past every row of this wave
    // contributes nothing to it: the wave only takes part in the copy and the
    // barrier.
    const bool skip = MASK && CAUSAL && k0 > q0w + 31;
    if (!skip) {
      // ---- S^T = K Q^T
      f32x16_t s[2];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[ks2][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
          s[ks2] = mfma32(*(const bf16x8_t*)(st + 8192 * ks2 + koff[ks]), S.qb[ks], s[ks2]);

      // ---- mask, online softmax on raw scores (row = this lane's query row)
      if constexpr (MASK) {
        // score (ks2, i) is key k0 + 4 hh + e, e = 32 ks2 + 8 (i / 4) + i % 4; it is
        // dead past the key range and, causal, past this lane's row
        int32_t lim = kend - 1 - (k0 + 4 * hh);
        if constexpr (CAUSAL) lim = min(lim, row - (k0 + 4 * hh));
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * ks2 + 8 * (i >> 2) + (i & 3) > lim) s[ks2][i] = kNegInf;
      }
      float mt = s[0][0];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[ks2][i]);
      mt = xor32_max(mt) * qk;                            // exp2 domain
      // Lazy rescale: the reference max only moves when some row's max grew by
      // more than 8, so probabilities stay <= 2^8 and most tiles skip the O^T
      // rescale.  Any reference works: numerator and denominator share it.
      if (__builtin_amdgcn_ballot_w64(mt > S.m_run + 8.f) != 0) {
        const float m_new = fmaxf(S.m_run, mt);
        const float alpha = fast_exp2(S.m_run - (m_new == kNegInf ? 0.f : m_new));
        S.l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) S.o[dt] *= alpha;
        S.m_run = m_new;
      }
      const float m_use = (S.m_run == kNegInf) ? 0.f : S.m_run;
      // fp8 context: p carries the factor v_scale (added to its exponent) so
      // the products with the decoded codes are p * value; the row sum does not
      float psum = 0.f;
      const float shift = KIND == kCtxNhdBf16 ? -m_use : vexp - m_use;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[ks2][i] = fast_exp2(__builtin_fmaf(s[ks2][i], qk, shift));
          psum += s[ks2][i];
        }
      if constexpr (KIND == kCtxNhdBf16) S.l_run += psum;
      else S.l_run = __builtin_fmaf(psum, linv, S.l_run);

      // P^T as B operand: k-step kk covers keys 16kk + {4hh..4hh+3, 8+4hh..8+4hh+3}
      bf16x8_t pb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[kk][j] = (__bf16)s[kk >> 1][8 * (kk & 1) + j];

      // ---- O^T += V^T P^T
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4_t lo = lds_read_tr16(st + 4096 * kk + voff[dt]);
          const s16x4_t hi = lds_read_tr16(st + 4096 * kk + 2048 + voff[dt]);
          S.o[dt] = mfma32(cat_tr(lo, hi), pb[kk], S.o[dt]);
        }
      }
    }

    if constexpr (KIND != kCtxNhdBf16 && !LAST)
      stage_store<KIND>(R, smem + (1 - par) * kStage, k0 + kBN, kend);
    dma_wait_for(blk_next);
    __syncthreads();
  };

  int32_t t_plain = (kend - k_begin) / kBN;             // tiles fully inside the key range
  if constexpr (CAUSAL) {
    const int32_t c = q0_lo - k_begin - (kBN - 1);       // last key of tile <= first row
    const int32_t tc = c >= 0 ? c / kBN + 1 : 0;
    t_plain = t_plain < tc ? t_plain : tc;
  }
  // tile t sits in buffer (t + SB) & 1
  using Par0 = std::integral_constant<int, SB>;
  using Par1 = std::integral_constant<int, 1 - SB>;
  using No = std::false_type;
  using Yes = std::true_type;
  const int32_t n_body = n_tiles - 1;                   // tiles followed by another one
  const int32_t tp = t_plain < n_body ? t_plain : n_body;
  int32_t t = 0;
  for (; t + 1 < tp; t += 2) {
    step(t, No{}, Par0{}, No{});
    step(t + 1, No{}, Par1{}, No{});
  }
  if (t < tp) {                                           // t is even here
    step(t, No{}, Par0{}, No{});
    ++t;
  }
  for (; t < n_body; ++t) step(t, Yes{}, (int)((t + SB) & 1), No{});
  // the last tile: the other buffer is free from here on
  const int par_last = (t + SB) & 1;
  hooks.last(smem + (1 - par_last) * kStage);
  __builtin_amdgcn_sched_barrier(0);    // keep the hook's code apart from the tile's
  // (buffer offsets as compile-time constants: with a run-time buffer the
  // compiler builds every LDS address in a register of its own)
  if (t < t_plain) {
    if (par_last == SB) step(t, No{}, Par0{}, Yes{});
    else step(t, No{}, Par1{}, Yes{});
  } else {
    if (par_last == SB) step(t, Yes{}, Par0{}, Yes{});
    else step(t, Yes{}, Par1{}, Yes{});
  }
}


// Fold keys [k_begin, k_end) of one source into the running state of this
// wave's rows (tokens q0w .. q0w + 31; the workgroup's tokens are [q0_lo,
// q_end)): copy the first tile, then the tile loop.  The LDS double buffer is
// filled and drained inside, so phases with different sources can follow
// each other.
template <bool PAGED, bool CAUSAL, bool FIRST = false, int KIND = kCtxNhdBf16>
__device__ __forceinline__ void run_keys(const AttnArgs& a, uint8_t* smem, const KeySrc& src,
                                         int32_t q0w, int32_t q0_lo, int32_t q_end, int32_t qn,
                                         int32_t k_begin, int32_t k_end, RowState& S) {
  // key range actually needed by the workgroup
  int32_t kend = k_end;
  if constexpr (CAUSAL) kend = min(kend, min(q_end, qn));
  if (kend <= k_begin) return;               // uniform over the workgroup
  const int32_t n_tiles = (kend - k_begin + kBN - 1) / kBN;

  if constexpr (!FIRST) __syncthreads();      // a previous phase may still read the buffers
  int32_t blk_next = 0;
  if constexpr (KIND == kCtxNhdBf16) {
    dma_tile<PAGED>(a, src, smem, k_begin, kend, tile_block<PAGED>(a, src, k_begin, kend));
    // table entry of the next tile's rows (the step copying tile t+1 looks up t+2)
    blk_next = n_tiles > 1 ? tile_block<PAGED>(a, src, k_begin + kBN, kend) : 0;
  } else {
    Staged R;
    stage_load<KIND>(a, src, k_begin, kend, R);
    stage_store<KIND>(R, smem, k_begin, kend);
  }
  dma_wait_for(blk_next);
  // Q^T was loaded before this wait; passing it through an empty asm tells the
  // compiler so.  Otherwise its wait insertion treats the Q loads as possibly
  // outstanding at the loop head and waits on the vector-memory counter before
  // the first MFMA of every tile -- which also waits for the next tile's copy
  // issued just before, and serialises the double buffer.
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(S.qb[ks]));
  __syncthreads();
  key_loop<PAGED, CAUSAL, 0, NoHooks, AttnArgs, KIND>(a, smem, src, q0w, q0_lo, k_begin, kend,
                                                     n_tiles, blk_next, S, NoHooks{});
}

// Write this wave's rows: bf16 output + lse, or an fp32 partial (normalised
// o and its lse) of part `part`.
template <bool PARTIAL>
__device__ __forceinline__ void finish_rows(const AttnArgs& a, int32_t h, int64_t qbase,
                                            int32_t q0w, int32_t qn, int32_t part, RowState& S) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int32_t row = q0w + r;
  const float l_run = xor32_sum(S.l_run);
  if (row >= qn) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse_v = l_run > 0.f ? (S.m_run + __log2f(l_run)) * kLn2 : kNegInf;
  const int64_t grow = qbase + row;
  if constexpr (PARTIAL) {
    float* op = a.part_o + (((int64_t)part * a.rows + grow) * a.Hq + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4_t v4 = {S.o[dt][4 * i4] * inv, S.o[dt][4 * i4 + 1] * inv,
                            S.o[dt][4 * i4 + 2] * inv, S.o[dt][4 * i4 + 3] * inv};
        *(f32x4_t*)(op + 32 * dt + 8 * i4 + 4 * hh) = v4;
      }
    if (hh == 0) a.part_lse[((int64_t)part * a.rows + grow) * a.Hq + h] = lse_v;
  } else {
    __bf16* op = a.out + (grow * a.Hq + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const bf16x4_t v4 = {(__bf16)(S.o[dt][4 * i4] * inv), (__bf16)(S.o[dt][4 * i4 + 1] * inv),
                             (__bf16)(S.o[dt][4 * i4 + 2] * inv), (__bf16)(S.o[dt][4 * i4 + 3] * inv)};
        *(bf16x4_t*)(op + 32 * dt + 8 * i4 + 4 * hh) = v4;
      }
    if (hh == 0 && a.lse) a.lse[grow * a.Hq + h] = lse_v;
  }
}

template <class Args>
__device__ __forceinline__ KeySrc contiguous_keys(const Args& a, int32_t s0, int32_t hkv) {
  KeySrc src;
  src.kb = (const uint8_t*)(a.k + (int64_t)s0 * a.Hkv * kD);
  src.vb = (const uint8_t*)(a.v + (int64_t)s0 * a.Hkv * kD);
  src.trow = nullptr;
  src.hkv = hkv;
  return src;
}

template <class Args>
__device__ __forceinline__ KeySrc paged_keys(const Args& a, int32_t seq, int32_t hkv) {
  KeySrc src;
  src.kb = a.kc;
  src.vb = a.vc;
  src.trow = a.tables + (int64_t)seq * a.max_blocks;
  src.hkv = hkv;
  return src;
}

template <class Args>
__device__ __forceinline__ int32_t context_len(const Args& a, int32_t seq) {
  int32_t C = a.ctx_lens[seq];
  const int32_t cap = a.max_blocks << a.bs_log2;
  C = C > cap ? cap : C;
  return C < 0 ? 0 : C;
}

// ---- Streamed prefill: one persistent workgroup per CU runs its work items
// back to back.  During the last key tile of an item it decodes the next item,
// copies that item's first K/V tile into the free LDS buffer, and each wave
// copies its next 32 query rows into its own 8 KB region of a Q area, so an
// item starts with nothing to wait for.  The output of an item is staged
// through the same region (after the next Q has been read from it) and
// written as whole 256-byte rows.
constexpr int kQRegion = 32 * kRowB;                     // one wave's 32 query rows
constexpr int kQArea = 2 * kStage;                       // Q / output area
constexpr int kSlotArea = kQArea + kWaves * kQRegion;    // per wave: the next item (64 bytes)
constexpr int kStreamSmem = kSlotArea + kWaves * 64;

struct StreamItem {
  int32_t valid, h, q0w, q0_lo, qn, s0, hkv, kend, n_tiles;
};
constexpr int kItemWords = 9;

// The kernel argument block as a constant-memory pointer the compiler cannot
// see through: fields read through it are loaded where they are used
// (scalar loads) instead of being hoisted to the kernel entry and held in
// registers across the whole item loop.
typedef const __attribute__((address_space(4))) AttnArgs* ArgsPtr;
__device__ __forceinline__ ArgsPtr args_here() {
  // the kernels take the argument block as their only argument, at offset 0
  ArgsPtr p = (ArgsPtr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

// Next valid work item of this workgroup's walk, from round r on (this
// wave's rows: q0w is its first row; keys [0, kend) in n_tiles tiles).
template <bool CAUSAL>
__device__ __forceinline__ StreamItem next_item(int32_t& r) {
  const auto& a = *args_here();
  StreamItem it = {};
  for (;; ++r) {
    const int64_t L = virtual_wg(a, r);
    if (L < 0) return it;
    const WorkItem w = work_item(a, L);
    if (w.lane >= a.items) continue;
    int64_t rest = w.lane;
    const int32_t gsel = (int32_t)(rest % a.Gs);
    rest /= a.Gs;
    const int32_t hkv = (int32_t)(rest % a.Hkv);
    const int32_t seq = (int32_t)(rest / a.Hkv);
    const int32_t s0 = a.cu[seq];
    const int32_t qn = a.cu[seq + 1] - s0;
    const RowBlock rb = row_block(a, hkv, gsel, w.qi);
    if (rb.q0_lo >= qn) continue;
    it.valid = 1;
    it.h = uniform(rb.h);
    it.q0w = uniform(rb.q0w);
    it.q0_lo = uniform(rb.q0_lo);
    it.qn = uniform(qn);
    it.s0 = uniform(s0);
    it.hkv = uniform(hkv);
    it.kend = uniform(CAUSAL ? min(rb.q_end, qn) : qn);
    it.n_tiles = uniform((it.kend + kBN - 1) / kBN);
    ++r;
    return it;
  }
}

// The item through this wave's LDS slot (lane i < kItemWords holds word i).
__device__ __forceinline__ void put_item(uint8_t* smem, const StreamItem& it) {
  const int lane = lane_here();
  const int32_t w[kItemWords] = {it.valid, it.h,    it.q0w,    it.q0_lo, it.qn,
                                 it.s0,    it.hkv,  it.kend,   it.n_tiles};
  int32_t v = 0;
#pragma unroll
  for (int i = 0; i < kItemWords; ++i) v = lane == i ? w[i] : v;
  if (lane < kItemWords) ((int32_t*)(smem + kSlotArea + wave_id() * 64))[lane] = v;
}
__device__ __forceinline__ StreamItem get_item(const uint8_t* smem) {
  const int32_t* p = (const int32_t*)(smem + kSlotArea + wave_id() * 64);
  const int lane = lane_here();
  const int32_t v = lane < kItemWords ? p[lane] : 0;
  StreamItem it;
  it.valid = __builtin_amdgcn_readlane(v, 0);
  it.h = __builtin_amdgcn_readlane(v, 1);
  it.q0w = __builtin_amdgcn_readlane(v, 2);
  it.q0_lo = __builtin_amdgcn_readlane(v, 3);
  it.qn = __builtin_amdgcn_readlane(v, 4);
  it.s0 = __builtin_amdgcn_readlane(v, 5);
  it.hkv = __builtin_amdgcn_readlane(v, 6);
  it.kend = __builtin_amdgcn_readlane(v, 7);
  it.n_tiles = __builtin_amdgcn_readlane(v, 8);
  return it;
}

// This wave's 32 query rows of `it` into its Q region: row i at 256 i, its
// 16-byte chunk c at position c ^ (i & 15) (rows past the sequence repeat its
// last row; their results are never stored).
template <class Args>
__device__ __forceinline__ void dma_q(const Args& a, uint8_t* smem, const StreamItem& it) {
  const int lane = lane_here();
  const int wave = wave_id();
  const uint32_t base = lds_addr(smem + kQArea + wave * kQRegion);
  const int pc = lane & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rw = 4 * j + (lane >> 4);
    int32_t row = it.q0w + rw;
    row = row < it.qn ? row : it.qn - 1;
    const uint8_t* g = (const uint8_t*)a.q + ((int64_t)(it.s0 + row) * a.Hq + it.h) * (kD * 2) +
                       ((pc ^ (rw & 15)) << 4);
    dma16(base + __builtin_amdgcn_readfirstlane(j * 1024), g);
  }
}

__device__ __forceinline__ void read_q(const uint8_t* smem, RowState& S) {
  const int lane = lane_here(), r = lane & 31, hh = lane >> 5;
  const uint8_t* reg = smem + kQArea + wave_id() * kQRegion;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) S.qb[ks] = *(const bf16x8_t*)(reg + kswz(r, 2 * ks + hh));
}

__device__ __forceinline__ void clear_rows(RowState& S) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) S.o[dt][i] = 0.f;
  S.m_run = kNegInf;
  S.l_run = 0.f;
}

// Output rows (bf16) and lse of this wave's rows q0w.. of head h, staged
// through its Q region so that every store writes whole rows.
template <class Args>
__device__ __forceinline__ void store_rows(const Args& a, uint8_t* smem, int32_t h, int32_t s0,
                                           int32_t q0w, int32_t qn, RowState& S) {
  const int lane = lane_here(), r = lane & 31, hh = lane >> 5;
  uint8_t* reg = smem + kQArea + wave_id() * kQRegion;
  const float l_run = xor32_sum(S.l_run);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const bf16x4_t v4 = {(__bf16)(S.o[dt][4 * i4] * inv), (__bf16)(S.o[dt][4 * i4 + 1] * inv),
                           (__bf16)(S.o[dt][4 * i4 + 2] * inv), (__bf16)(S.o[dt][4 * i4 + 3] * inv)};
      *(bf16x4_t*)(reg + kswz(r, 4 * dt + i4) + 8 * hh) = v4;
    }
  if (hh == 0 && q0w + r < qn && a.lse) {
    const float lse_v = l_run > 0.f ? (S.m_run + __log2f(l_run)) * kLn2 : kNegInf;
    a.lse[(int64_t)(s0 + q0w + r) * a.Hq + h] = lse_v;
  }
  order_lds();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rw = 4 * j + (lane >> 4), c = lane & 15;
    const bf16x8_t v = *(const bf16x8_t*)(reg + kswz(rw, c));
    const int32_t row = q0w + rw;
    if (row < qn) *(bf16x8_t*)(a.out + ((int64_t)(s0 + row) * a.Hq + h) * kD + 8 * c) = v;
  }
}

// Copies that start item n: its Q rows and its first key tile (into buf).
template <class Args>
__device__ __forceinline__ void start_item(const Args& a, uint8_t* smem, uint8_t* buf,
                                           const StreamItem& n) {
  dma_q(a, smem, n);
  dma_tile<false>(a, contiguous_keys(a, n.s0, n.hkv), buf, 0, n.kend, 0);
}

// Hooks of an item's key loop: at its last tile, decode the next item, leave
// it in the slot and start its copies.
template <bool CAUSAL>
struct NextItem {
  ArgsPtr a;
  uint8_t* smem;
  int32_t* r;
  __device__ __forceinline__ void last(uint8_t* buf) const {
    const StreamItem n = next_item<CAUSAL>(*r);
    put_item(smem, n);
    if (n.valid) start_item(*a, smem, buf, n);
  }
};

// Prefill as a stream of work items per persistent workgroup.
template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void prefill_stream_kernel(AttnArgs) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStreamSmem];
  int32_t r = 0;
  StreamItem cur = next_item<CAUSAL>(r);
  if (!cur.valid) return;
  start_item(*args_here(), smem, smem, cur);
  dma_wait();
  __syncthreads();
  RowState S;
  read_q(smem, S);
  clear_rows(S);
  int32_t sb = 0;                                   // LDS buffer of the item's first tile
  for (;;) {
    {
      const ArgsPtr A = args_here();
      const NextItem<CAUSAL> hooks = {A, smem, &r};
      const KeySrc src = contiguous_keys(*A, cur.s0, cur.hkv);
      if (sb == 0)
        key_loop<false, CAUSAL, 0>(*A, smem, src, cur.q0w, cur.q0_lo, 0, cur.kend, cur.n_tiles, 0,
                                   S, hooks);
      else
        key_loop<false, CAUSAL, 1>(*A, smem, src, cur.q0w, cur.q0_lo, 0, cur.kend, cur.n_tiles, 0,
                                   S, hooks);
    }
    sb = (sb + cur.n_tiles) & 1;
    // The last tile's barrier has passed: the next item's Q and first tile are in LDS.
    const StreamItem nxt = get_item(smem);
    RowState N;
    if (nxt.valid) read_q(smem, N);
    store_rows(*args_here(), smem, cur.h, cur.s0, cur.q0w, cur.qn, S);
    if (!nxt.valid) break;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) S.qb[ks] = N.qb[ks];
    clear_rows(S);
    cur = nxt;
  }
}

// Split extend.  Lanes: (seq, part, kv head, group of P query heads).  Part 0: the new
// tokens among themselves (causal).  Part
// p >= 1: the new tokens against context chunk p-1 = cached tokens
// [(p-1)*chunk, p*chunk), read through the block table.  Every part writes an
// fp32 partial (row pbase + i for new token i); extend_merge_kernel combines
// them.
// Hybrid plan, in the workspace (int32): [0] requests run split, [1] compact
// partial rows they use, [2] work-list entries, [3] unused, then max_split
// request ids and max_split first compact rows; after it (256-byte aligned)
// the work list, one ListEntry per (request, query item) of a fused request
// and per (request, part, query item) of a split one, heaviest first.
constexpr int kPlanHead = 4;
constexpr int kHybridMaxSeqs = 1024;          // requests the plan takes
constexpr int kHybridMaxSplit = 16;           // requests that may run split
constexpr int64_t kHybridPartialBytes = 64ll << 20;
struct ListEntry {
  int32_t seq, slot, part, qi;                // slot -1: fused
};

template <int KIND>
__device__ __forceinline__ void split_item(const AttnArgs& a, uint8_t* smem, int32_t seq,
                                           int32_t part, int32_t hkv, int32_t gsel, int32_t qi,
                                           int32_t slot) {
  const int32_t s0 = a.cu[seq];
  const int32_t qn = a.cu[seq + 1] - s0;
  const RowBlock rb = row_block(a, hkv, gsel, qi);
  if (rb.q0_lo >= qn) return;                            // uniform over the workgroup
  RowState S;
  if (part == 0) {
    init_rows(a, rb.h, s0, rb.q0w, qn, S);
    run_keys<false, true, true>(a, smem, contiguous_keys(a, s0, hkv), rb.q0w, rb.q0_lo, rb.q_end,
                                qn, 0, qn, S);
  } else {
    const int32_t C = context_len(a, seq);
    const int32_t kb = (part - 1) * a.chunk_tokens;
    if (kb >= C) return;
    init_rows(a, rb.h, s0, rb.q0w, qn, S);
    run_keys<true, false, true, KIND>(a, smem, paged_keys(a, seq, hkv), rb.q0w, rb.q0_lo, rb.q_end,
                                      qn, kb, min(C, kb + a.chunk_tokens), S);
  }
  // partial rows: the request's own rows, or (hybrid, slot >= 0) its compact rows
  const int64_t pbase = slot < 0 ? s0 : uniform(a.plan[kPlanHead + a.max_split + slot]);
  finish_rows<true>(a, rb.h, pbase, rb.q0w, qn, part, S);
}

template <int KIND>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void extend_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
  const WorkItem w = work_item(a, blockIdx.x);
  if (w.lane >= a.items) return;
  int64_t rest = w.lane;
  const int32_t gsel = (int32_t)(rest % a.Gs);
  rest /= a.Gs;
  const int32_t hkv = (int32_t)(rest % a.Hkv);
  rest /= a.Hkv;
  const int32_t part = (int32_t)(rest % a.n_parts);
  const int32_t seq = (int32_t)(rest / a.n_parts);
  split_item<KIND>(a, smem, seq, part, hkv, gsel, w.qi, -1);
}

// Fused extend, used when the batch has enough query tiles to fill the GPU
// without splitting along the context.  Logical order: (seq, kv head, head
// group, query item descending).  One workgroup runs the cached
// context of its rows and then the new tokens, carrying one running softmax
// state: the LSE merge of the context into the running output is done in
// registers (rescaling by the exponential of the max difference), so no
// partials are written and no merge pass is needed.  The context is walked as
// one key range: its 64-key tiles are the ones a walk chunk by chunk would
// take (chunk lengths are whole tiles), in the same order, so the result is
// the same, without a pipeline restart per chunk.  Q comes in through the
// per-wave LDS regions and the output leaves through them, as in the
// persistent prefill.
template <int KIND>
__device__ __forceinline__ void fused_item(const AttnArgs& a, uint8_t* smem, int32_t seq,
                                           int32_t hkv, int32_t gsel, int32_t qi) {
  const int32_t s0 = a.cu[seq];
  const int32_t qn = a.cu[seq + 1] - s0;
  const RowBlock rb = row_block(a, hkv, gsel, qi);
  if (rb.q0_lo >= qn) return;                            // uniform over the workgroup
  const int32_t C = context_len(a, seq);
  StreamItem it = {};
  it.valid = 1;
  it.h = rb.h;
  it.q0w = rb.q0w;
  it.qn = qn;
  it.s0 = s0;
  const int32_t kend = min(rb.q_end, qn);                // new tokens, causal
  const KeySrc ctx = paged_keys(a, seq, hkv);
  const KeySrc fresh = contiguous_keys(a, s0, hkv);
  dma_q(a, smem, it);
  int32_t blk1 = 0;
  if (C > 0) {
    if constexpr (KIND == kCtxNhdBf16) {
      dma_tile<true>(a, ctx, smem, 0, C, tile_block<true>(a, ctx, 0, C));
      blk1 = C > kBN ? tile_block<true>(a, ctx, kBN, C) : 0;
    } else {
      Staged R;
      stage_load<KIND>(a, ctx, 0, C, R);
      stage_store<KIND>(R, smem, 0, C);
    }
  } else {
    dma_tile<false>(a, fresh, smem, 0, kend, 0);
  }
  dma_wait_for(blk1);
  __syncthreads();
  RowState S;
  read_q(smem, S);
  clear_rows(S);
  if (C > 0) {
    const int32_t nt = (C + kBN - 1) / kBN;
    key_loop<true, false, 0, NoHooks, AttnArgs, KIND>(a, smem, ctx, rb.q0w, rb.q0_lo, 0, C, nt,
                                                      blk1, S, NoHooks{});
    run_keys<false, true>(a, smem, fresh, rb.q0w, rb.q0_lo, rb.q_end, qn, 0, qn, S);
  } else {
    const int32_t nt_new = (kend + kBN - 1) / kBN;
    key_loop<false, true, 0>(a, smem, fresh, rb.q0w, rb.q0_lo, 0, kend, nt_new, 0, S, NoHooks{});
  }
  store_rows(a, smem, rb.h, s0, it.q0w, qn, S);
}

template <int KIND>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void extend_fused_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kQArea + kWaves * kQRegion];
  const WorkItem w = work_item(a, blockIdx.x);
  if (w.lane >= a.items) return;
  int64_t rest = w.lane;
  const int32_t gsel = (int32_t)(rest % a.Gs);
  rest /= a.Gs;
  const int32_t hkv = (int32_t)(rest % a.Hkv);
  const int32_t seq = (int32_t)(rest / a.Hkv);
  fused_item<KIND>(a, smem, seq, hkv, gsel, w.qi);
}

// Hybrid extend over the plan's work list: lanes are the (KV head, head
// group) combinations, query items the list positions (heaviest first, the
// positions past the list's length empty and launched last).  An entry runs
// fused (its request's context and new tokens, one running state) or as one
// part of a split request (partials in compact rows, merged afterwards).
template <int KIND>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void extend_list_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kQArea + kWaves * kQRegion];
  const WorkItem w = work_item(a, blockIdx.x);
  if (w.lane >= a.items) return;
  const int32_t pos = a.n_qitems - 1 - w.qi;
  if (pos >= uniform(a.plan[2])) return;
  const ListEntry* e = a.list + pos;
  const int32_t seq = uniform(e->seq), slot = uniform(e->slot);
  const int32_t part = uniform(e->part), qi = uniform(e->qi);
  const int32_t gsel = (int32_t)(w.lane % a.Gs);
  const int32_t hkv = (int32_t)(w.lane / a.Gs);
  if (slot < 0) fused_item<KIND>(a, smem, seq, hkv, gsel, qi);
  else split_item<KIND>(a, smem, seq, part, hkv, gsel, qi, slot);
}

// Final merge of the extend parts of each (row, head), one wave each:
// o = sum_p w_p o_p / sum_p w_p, w_p = exp(lse_p - max_p lse_p),
// lse = max + ln sum_p w_p.
__global__ __launch_bounds__(256) void extend_merge_kernel(AttnArgs a) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * 4 + wave;
  if (rh >= (int64_t)a.rows * a.Hq) return;
  const int32_t grow = (int32_t)(rh / a.Hq);
  // the request owning this row (cu is sorted)
  int32_t lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (a.cu[mid] <= grow) lo = mid; else hi = mid - 1;
  }
  int32_t C = a.ctx_lens[lo];
  const int32_t cap = a.max_blocks << a.bs_log2;
  C = C > cap ? cap : C;
  C = C < 0 ? 0 : C;
  int32_t np = 1 + (C + a.chunk_tokens - 1) / a.chunk_tokens;
  np = np > a.n_parts ? a.n_parts : np;
  const int64_t stride = (int64_t)a.rows * a.Hq;
  float M = kNegInf;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_lse[p * stride + rh]);
  f32x2_t acc = {0.f, 0.f};
  float wsum = 0.f;
  for (int p = 0; p < np; ++p) {
    const float lp = a.part_lse[p * stride + rh];
    const float w = lp == kNegInf ? 0.f : fast_exp2((lp - M) * kLog2e);
    wsum += w;
    acc += w * *((const f32x2_t*)(a.part_o + (p * stride + rh) * kD) + lane);
  }
  const float inv = 1.f / wsum;
  *(bf16x2_t*)(a.out + rh * kD + 2 * lane) = bf16x2_t{(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv)};
  if (lane == 0 && a.lse) a.lse[rh] = M + __log2f(wsum) * kLn2;
}

// Exclusive prefix sum over the 1024 threads of a workgroup (v of thread t
// -> sum of v over threads < t); *total gets the sum over all of them.
__device__ __forceinline__ int32_t block_scan_1024(int32_t v, int32_t* s_tmp, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t inc = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(inc, off);
    if (lane >= off) inc += u;
  }
  __syncthreads();                                        // s_tmp free
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int32_t base = 0, all = 0;
  for (int i = 0; i < 16; ++i) {
    const int32_t x = s_tmp[i];
    base += i < wave ? x : 0;
    all += x;
  }
  *total = all;
  return base + inc - v;
}

// Plan of the hybrid extend (one workgroup, one request per thread).  A fused
// work item of request b (n_b new tokens, C_b cached) with tokens [i R, (i+1) R)
// walks ceil(C_b/64) context tiles and ceil(min((i+1) R, n_b)/64) new-token
// tiles (R = TW tokens per workgroup); its
// longest item walks walk_b = ceil(C_b/64) + ceil(n_b/64).  The batch's work,
// summed over every item, spread over the resident workgroups gives the mean
// load D.  A request with walk_b > D / 2 holds workgroups for a large part of
// the kernel's time by itself, and late if they start late; if its context
// spans more than one chunk it is a candidate to run split (its chunks in
// parallel), and candidates are taken in request order while the running
// count stays within max_split and their running rows within the compact
// partial rows (rows).  Then the work list: every query item of a fused
// request and every (part, query item) of a split one, requests sorted by
// their heaviest entry (heaviest first, ties in request order), each
// request's entries heaviest first (context chunks before the new-token
// part, later query items first).
__global__ __launch_bounds__(1024) void extend_plan_kernel(AttnArgs a) {
  __shared__ int32_t s_tmp[16];
  __shared__ int64_t s_w[16];
  __shared__ uint32_t s_key[kHybridMaxSeqs];
  __shared__ int32_t s_cnt[kHybridMaxSeqs];
  __shared__ int32_t s_slot[kHybridMaxSeqs];
  __shared__ int32_t s_off[kHybridMaxSeqs + 1];   // first list entry of sorted position q
  __shared__ int32_t s_req[kHybridMaxSeqs];       // request at sorted position q
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int32_t R = a.TW;
  int32_t* plan = (int32_t*)a.plan;
  const bool mine = t < a.num_seqs;
  const int32_t n = mine ? a.cu[t + 1] - a.cu[t] : 0;
  const int32_t C = mine ? context_len(a, t) : 0;
  const int32_t k = (n + R - 1) / R;                      // query items per lane
  const int32_t ct = (C + kBN - 1) / kBN, nt = (n + kBN - 1) / kBN;
  int64_t w = n > 0 ? (int64_t)a.Hkv * a.Gs *
                          ((int64_t)k * ct + (int64_t)R * (k - 1) * k / 2 / kBN + nt)
                    : 0;
  for (int off = 32; off > 0; off >>= 1) w += __shfl_xor(w, off);
  if (lane == 0) s_w[wave] = w;
  __syncthreads();
  int64_t tot = 0;
  for (int i = 0; i < 16; ++i) tot += s_w[i];
  const int64_t D = tot / (a.plan_slots > 0 ? a.plan_slots : 1);
  // split candidates, taken in request order while slots and rows last
  const bool cand = n > 0 && 2 * (int64_t)(ct + nt) > D && C > a.chunk_tokens;
  int32_t all_c, all_r;
  const int32_t before_c = block_scan_1024(cand ? 1 : 0, s_tmp, &all_c);
  const int32_t before_r = block_scan_1024(cand ? n : 0, s_tmp, &all_r);
  const bool split = cand && before_c < a.max_split && before_r + n <= a.rows;
  int32_t n_split, used;
  const int32_t slot_of = block_scan_1024(split ? 1 : 0, s_tmp, &n_split);
  const int32_t row_off = block_scan_1024(split ? n : 0, s_tmp, &used);
  const int32_t slot = split ? slot_of : -1;
  if (split) {
    plan[kPlanHead + slot] = t;
    plan[kPlanHead + a.max_split + slot] = row_off;
  }
  // entries and the request order
  int32_t np = 1 + (C + a.chunk_tokens - 1) / a.chunk_tokens;
  np = np > a.n_parts ? a.n_parts : np;
  const int32_t cnt = n == 0 ? 0 : (slot < 0 ? k : np * k);
  const int32_t cht = ((C < a.chunk_tokens ? C : a.chunk_tokens) + kBN - 1) / kBN;
  const int32_t rcost = slot < 0 ? ct + nt : (nt > cht ? nt : cht);
  int32_t N = 1;
  while (N < a.num_seqs) N <<= 1;
  if (t < N) {
    s_key[t] = cnt > 0 ? ((0xFFFFu - (uint32_t)(rcost < 0xFFFF ? rcost : 0xFFFF)) << 10) | (uint32_t)t
                       : 0xFFFFFFFFu;
    if (mine) {
      s_cnt[t] = cnt;
      s_slot[t] = slot;
    }
  }
  __syncthreads();
  for (int32_t kk = 2; kk <= N; kk <<= 1) {
    for (int32_t jj = kk >> 1; jj > 0; jj >>= 1) {
      if (t < N) {
        const int32_t ixj = t ^ jj;
        if (ixj > t) {
          const uint32_t x = s_key[t], y = s_key[ixj];
          if ((x > y) == ((t & kk) == 0)) {
            s_key[t] = y;
            s_key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  // offsets of the sorted requests' entries, then every thread writes entries
  // j = t, t + 1024, ...: entry j belongs to the last sorted position whose
  // first entry is <= j (positions without entries share their successor's
  // offset)
  const uint32_t key = t < N ? s_key[t] : 0xFFFFFFFFu;
  const int32_t b = key != 0xFFFFFFFFu ? (int32_t)(key & 0x3FFu) : -1;
  const int32_t bcnt = b >= 0 ? s_cnt[b] : 0;
  int32_t total;
  const int32_t off = block_scan_1024(bcnt, s_tmp, &total);
  const int32_t E = total < a.list_cap ? total : a.list_cap;
  if (t < N) {
    s_off[t] = off;
    s_req[t] = b;
  }
  __syncthreads();
  ListEntry* list = (ListEntry*)a.list;
  for (int32_t j = t; j < E; j += 1024) {
    int32_t lo = 0, hi = N - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= j) lo = mid; else hi = mid - 1;
    }
    const int32_t rb = s_req[lo], i = j - s_off[lo];
    const int32_t bn = a.cu[rb + 1] - a.cu[rb];
    const int32_t bk = (bn + R - 1) / R;
    const int32_t bslot = s_slot[rb];
    const int32_t bparts = s_cnt[rb] / bk;
    ListEntry e;
    e.seq = rb;
    e.slot = bslot;
    e.qi = bk - 1 - i % bk;                               // later query items first
    const int32_t pi = i / bk;                            // context chunks first, new tokens last
    e.part = bslot < 0 ? 0 : (pi + 1 < bparts ? pi + 1 : 0);
    list[j] = e;
  }
  if (t == 0) {
    plan[0] = n_split;
    plan[1] = used;
    plan[2] = E;
  }
}

// Merge of the hybrid extend's split requests: one wave per compact (row,
// head), as extend_merge_kernel.
__global__ __launch_bounds__(256) void extend_merge_compact_kernel(AttnArgs a) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * 4 + wave;
  const int32_t n_split = uniform(a.plan[0]), used = uniform(a.plan[1]);
  if (rh >= (int64_t)used * a.Hq) return;
  const int32_t cr = (int32_t)(rh / a.Hq), h = (int32_t)(rh % a.Hq);
  int32_t j = 0;                                          // the slot owning compact row cr
  while (j + 1 < n_split && a.plan[kPlanHead + a.max_split + j + 1] <= cr) ++j;
  const int32_t seq = a.plan[kPlanHead + j];
  const int64_t grow = (int64_t)a.cu[seq] + (cr - a.plan[kPlanHead + a.max_split + j]);
  const int32_t C = context_len(a, seq);
  int32_t np = 1 + (C + a.chunk_tokens - 1) / a.chunk_tokens;
  np = np > a.n_parts ? a.n_parts : np;
  const int64_t stride = (int64_t)a.rows * a.Hq;
  float M = kNegInf;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_lse[p * stride + rh]);
  f32x2_t acc = {0.f, 0.f};
  float wsum = 0.f;
  for (int p = 0; p < np; ++p) {
    const float lp = a.part_lse[p * stride + rh];
    const float wp = lp == kNegInf ? 0.f : fast_exp2((lp - M) * kLog2e);
    wsum += wp;
    acc += wp * *((const f32x2_t*)(a.part_o + (p * stride + rh) * kD) + lane);
  }
  const float inv = 1.f / wsum;
  const int64_t oh = grow * a.Hq + h;
  *(bf16x2_t*)(a.out + oh * kD + 2 * lane) = bf16x2_t{(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv)};
  if (lane == 0 && a.lse) a.lse[oh] = M + __log2f(wsum) * kLn2;
}

int32_t log2i(int32_t v) {
  int32_t l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

}  // namespace

// Query heads per workgroup: the largest power of two up to 8 dividing the
// group size G.
static int32_t heads_per_wg(int32_t G) {
  int32_t P = 1;
  while (P < 8 && G % (2 * P) == 0) P *= 2;
  return P;
}

// Rows of a work item: P query heads of one KV head over TW = 256 / P tokens;
// lanes per KV head and query items per lane for sequences of up to
// max_tokens tokens.
static void set_packing(AttnArgs& a, int32_t max_tokens) {
  a.P = heads_per_wg(a.G);
  a.TW = kWGRows / a.P;
  a.Gs = a.G / a.P;
  a.n_qitems = (max_tokens + a.TW - 1) / a.TW;
  a.lchunk = a.Gs >= 2 ? a.Gs / 2 : 1;
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                          int32_t num_seqs, int32_t max_seqlen, int32_t num_q_heads,
                          int32_t num_kv_heads, float scale, int32_t causal, void* out, float* lse,
                          hipStream_t s) {
  AttnArgs a = {};
  a.q = (const __bf16*)q;
  a.k = (const __bf16*)k;
  a.v = (const __bf16*)v;
  a.cu = cu_seqlens;
  a.out = (__bf16*)out;
  a.lse = lse;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.G = num_q_heads / num_kv_heads;
  a.num_seqs = num_seqs;
  set_packing(a, max_seqlen);
  a.n_parts = 1;
  a.qk_mult = scale * kLog2e;
  a.items = (int64_t)num_seqs * num_kv_heads * a.Gs;     // lanes
  a.grid_pad = work_grid(a.items, a.n_qitems, a.lchunk);
  a.qt_major = causal ? 1 : 0;
  if (a.grid_pad > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(persistent_grid(a.grid_pad, s));
  if (causal)
    hipLaunchKernelGGL(prefill_stream_kernel<true>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_stream_kernel<false>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

ExtendPlan plan_extend(const kv_cache_t& c, int32_t num_seqs, int32_t total_new,
                       int32_t num_q_heads, int32_t max_ctx_len, int32_t chunk_budget_tokens,
                       int32_t mode, hipStream_t stream) {
  ExtendPlan p;
  // Per-request share of the budget, rounded down to whole key tiles and
  // blocks (at least one).
  const int32_t unit = c.block_size > kBN ? c.block_size : kBN;
  int64_t share = num_seqs > 0 ? (int64_t)chunk_budget_tokens / num_seqs : chunk_budget_tokens;
  share = share / unit * unit;
  if (share < unit) share = unit;
  if (share > (1 << 30)) share = 1 << 30;
  p.chunk_tokens = (int32_t)share;
  p.n_chunks = max_ctx_len > 0 ? (int32_t)((max_ctx_len + share - 1) / share) : 0;
  p.n_parts = p.n_chunks + 1;
  // Automatic: fused when the query tiles alone give every CU two rounds of
  // its two resident workgroups; otherwise the context chunks become extra
  // grid parallelism and a merge pass combines them.
  const int64_t tiles = (int64_t)num_q_heads * ((total_new + kBM - 1) / kBM);
  if (mode == KV_EXTEND_SPLIT)
    p.fused = 0;
  else if (mode == KV_EXTEND_FUSED)
    p.fused = 1;
  else
    p.fused = (p.n_chunks == 0 || tiles >= (int64_t)4 * device_cu_count(stream)) ? 1 : 0;
  // Automatic and fused with a context of two or more chunks: hybrid, whose
  // device-side plan may still run some requests split (their partials in at
  // most kHybridPartialBytes of compact rows).
  p.hybrid = 0;
  p.max_split = 0;
  p.cap_rows = 0;
  p.list_cap = 0;
  if (mode == KV_EXTEND_AUTO && p.fused && p.n_chunks >= 2 && num_seqs <= kHybridMaxSeqs) {
    const int64_t per_row = (int64_t)p.n_parts * num_q_heads * (kD + 1) * (int64_t)sizeof(float);
    const int64_t cap = kHybridPartialBytes / per_row;
    p.cap_rows = (int32_t)(cap < total_new ? cap : total_new);
    p.max_split = num_seqs < kHybridMaxSplit ? num_seqs : kHybridMaxSplit;
    // list length bound: a fused request has at most n/R + 1 query items, a
    // split one n_parts times that, and the split requests' rows are at most
    // cap_rows
    const int64_t R = kWGRows / heads_per_wg(num_q_heads / c.num_kv_heads);
    const int64_t cap_list = (total_new + R - 1) / R + num_seqs +
                             (int64_t)p.n_parts * ((p.cap_rows + R - 1) / R + p.max_split);
    p.list_cap = (int32_t)(cap_list < (1 << 24) ? cap_list : 0);
    p.hybrid = p.cap_rows > 0 && p.list_cap > 0 && p.n_parts < (1 << 15) ? 1 : 0;
  }
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t hybrid_plan_bytes(const ExtendPlan& p) {
  return align256(sizeof(int32_t) * ((size_t)kPlanHead + 2 * (size_t)p.max_split)) +
         align256(sizeof(ListEntry) * (size_t)p.list_cap);
}

size_t extend_workspace_bytes(const ExtendPlan& p, int32_t num_seqs, int32_t total_new,
                              int32_t num_q_heads, int32_t head_dim) {
  if (p.fused && !p.hybrid) return 0;
  const int32_t rows_cap = p.fused ? p.cap_rows : total_new;
  const size_t rows = (size_t)p.n_parts * rows_cap * num_q_heads;
  return (p.fused ? hybrid_plan_bytes(p) : 0) + align256(rows * head_dim * sizeof(float)) +
         align256(rows * sizeof(float));
}

hipError_t launch_extend(const kv_cache_t& c, const ExtendPlan& p, const void* q,
                         const void* k_new, const void* v_new, const int32_t* cu_q_lens,
                         const int32_t* ctx_lens, const int32_t* tables, int32_t max_blocks,
                         int32_t num_seqs, int32_t total_new, int32_t max_q_len,
                         int32_t num_q_heads, float scale, void* out, float* lse,
                         void* workspace, hipStream_t s) {
  AttnArgs a = {};
  a.q = (const __bf16*)q;
  a.k = (const __bf16*)k_new;
  a.v = (const __bf16*)v_new;
  a.cu = cu_q_lens;
  a.kc = (const uint8_t*)c.k_cache;
  a.vc = (const uint8_t*)c.v_cache;
  a.tables = tables;
  a.ctx_lens = ctx_lens;
  a.out = (__bf16*)out;
  a.lse = lse;
  const size_t plan_bytes = p.fused && p.hybrid ? hybrid_plan_bytes(p) : 0;
  const size_t prow = (size_t)p.n_parts * (p.fused ? p.cap_rows : total_new) * num_q_heads;
  a.plan = (const int32_t*)workspace;
  a.list = (const ListEntry*)((uint8_t*)workspace +
                              align256(sizeof(int32_t) * ((size_t)kPlanHead + 2 * (size_t)p.max_split)));
  a.part_o = (float*)((uint8_t*)workspace + plan_bytes);
  a.part_lse = (float*)((uint8_t*)workspace + plan_bytes + align256(prow * c.head_dim * sizeof(float)));
  a.max_blocks = max_blocks > 0 ? max_blocks : 1;
  a.num_blocks = c.num_blocks;
  a.bs = c.block_size;
  a.bs_log2 = log2i(c.block_size);
  a.Hq = num_q_heads;
  a.Hkv = c.num_kv_heads;
  a.G = num_q_heads / c.num_kv_heads;
  a.num_seqs = num_seqs;
  const int32_t n_qtiles = (max_q_len + kBM - 1) / kBM;
  set_packing(a, max_q_len);
  a.n_parts = p.n_parts;
  a.chunk_tokens = p.chunk_tokens;
  a.rows = total_new;
  a.qk_mult = scale * kLog2e;
  a.ctx_qk_mult = scale * c.k_scale * kLog2e;
  a.ctx_vexp = __builtin_log2f(c.v_scale);
  a.ctx_linv = 1.0f / c.v_scale;
  a.qt_major = n_qtiles <= 16 ? 1 : 0;
  const int kind = c.layout == KV_LAYOUT_NHD ? (c.dtype == KV_DTYPE_BF16 ? kCtxNhdBf16 : kCtxNhdFp8)
                                             : (c.dtype == KV_DTYPE_BF16 ? kCtxPreBf16 : kCtxPreFp8);
  if (p.fused && p.hybrid) {
    a.rows = p.cap_rows;
    a.max_split = p.max_split;
    a.list_cap = p.list_cap;
    a.plan_slots = device_cu_count(s);
    a.items = (int64_t)a.Hkv * a.Gs;                     // lanes: (KV head, head group)
    a.n_qitems = p.list_cap;                             // list positions
    a.qt_major = 1;
    // an XCD's share of the lanes: an eighth of them, within one KV head or
    // whole KV heads, so that its workgroups stream one context at a time
    {
      const int32_t target = a.items >= 8 ? (int32_t)(a.items / 8) : 1;
      int32_t c = 1;
      if (target >= a.Gs) c = (target / a.Gs) * a.Gs;
      else for (int32_t d = target; d >= 1; --d) if (a.Gs % d == 0) { c = d; break; }
      a.lchunk = c;
    }
    a.grid_pad = work_grid(a.items, a.n_qitems, a.lchunk);
    if (a.grid_pad > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(extend_plan_kernel, dim3(1), dim3(1024), 0, s, a);
    const dim3 grid((unsigned)a.grid_pad);
    switch (kind) {
      case kCtxNhdBf16: hipLaunchKernelGGL(extend_list_kernel<kCtxNhdBf16>, grid, dim3(kThreads), 0, s, a); break;
      case kCtxNhdFp8: hipLaunchKernelGGL(extend_list_kernel<kCtxNhdFp8>, grid, dim3(kThreads), 0, s, a); break;
      case kCtxPreBf16: hipLaunchKernelGGL(extend_list_kernel<kCtxPreBf16>, grid, dim3(kThreads), 0, s, a); break;
      default: hipLaunchKernelGGL(extend_list_kernel<kCtxPreFp8>, grid, dim3(kThreads), 0, s, a); break;
    }
    const int64_t rh = (int64_t)p.cap_rows * num_q_heads;
    hipLaunchKernelGGL(extend_merge_compact_kernel, dim3((unsigned)((rh + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (p.fused) {
    a.items = (int64_t)num_seqs * a.Hkv * a.Gs;          // lanes
    a.grid_pad = work_grid(a.items, a.n_qitems, a.lchunk);
    if (a.grid_pad > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.grid_pad);
    switch (kind) {
      case kCtxNhdBf16: hipLaunchKernelGGL(extend_fused_kernel<kCtxNhdBf16>, grid, dim3(kThreads), 0, s, a); break;
      case kCtxNhdFp8: hipLaunchKernelGGL(extend_fused_kernel<kCtxNhdFp8>, grid, dim3(kThreads), 0, s, a); break;
      case kCtxPreBf16: hipLaunchKernelGGL(extend_fused_kernel<kCtxPreBf16>, grid, dim3(kThreads), 0, s, a); break;
      default: hipLaunchKernelGGL(extend_fused_kernel<kCtxPreFp8>, grid, dim3(kThreads), 0, s, a); break;
    }
    return hipGetLastError();
  }
  a.items = (int64_t)num_seqs * p.n_parts * a.Hkv * a.Gs;  // lanes
  a.grid_pad = work_grid(a.items, a.n_qitems, a.lchunk);
  if (a.grid_pad > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.grid_pad);
  switch (kind) {
    case kCtxNhdBf16: hipLaunchKernelGGL(extend_kernel<kCtxNhdBf16>, grid, dim3(kThreads), 0, s, a); break;
    case kCtxNhdFp8: hipLaunchKernelGGL(extend_kernel<kCtxNhdFp8>, grid, dim3(kThreads), 0, s, a); break;
    case kCtxPreBf16: hipLaunchKernelGGL(extend_kernel<kCtxPreBf16>, grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(extend_kernel<kCtxPreFp8>, grid, dim3(kThreads), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rh = (int64_t)total_new * num_q_heads;
  hipLaunchKernelGGL(extend_merge_kernel, dim3((unsigned)((rh + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
