"""Seeded synthetic inputs shaped like the serving workloads of the pages.

This module only draws random inputs and lays them out; it holds none of the
attention or cache arithmetic.  Both the CPU oracle and the HIP path consume
exactly the arrays produced here (numpy; bf16 as uint16 bit patterns, fp8 as
uint8 codes).  Random source: numpy PCG64 via ``default_rng(seed)``; large
tensors are drawn in fixed 4M-element chunks, each from a stream spawned off a
seed taken from the workload's generator (threaded, thread-count independent).

Recipe (shared by every workload):
* activations and cache contents: float32 N(0, 1), rounded to bf16 with
  round-half-to-even;
* block tables: one random permutation of the physical blocks, sliced
  consecutively per request, so every request is fully fragmented;
* lengths: uniform integers over the stated inclusive ranges;
* fp8 caches: per-tensor scale = amax / 448 over the drawn N(0,1) values, codes
  from torch's float8_e4m3fn cast of value / scale (a library conversion);
* one physical block (the last) is kept out of every table: tests fill it with
  NaN and point padding table entries at it, so an over-read shows up as NaN
  instead of touching memory outside the cache.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)


# ----------------------------------------------------------------------------
# random bf16 tensors
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-half-to-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


_CHUNK = 1 << 22


def _parallel_normal(rng: np.random.Generator, n: int, sink) -> None:
    """Draw n N(0,1) float32 values in fixed chunks of 4M, each from its own
    stream spawned off a seed taken from ``rng``; ``sink(start, values)``
    receives them.  Chunks run on threads; the values do not depend on the
    thread count."""
    from concurrent.futures import ThreadPoolExecutor

    seed = int(rng.integers(0, 2**63 - 1))
    nch = (n + _CHUNK - 1) // _CHUNK
    seqs = np.random.SeedSequence(seed).spawn(max(nch, 1))

    def job(i):
        s = i * _CHUNK
        e = min(n, s + _CHUNK)
        g = np.random.default_rng(seqs[i])
        sink(s, g.standard_normal(e - s, dtype=np.float32))

    if nch <= 1:
        for i in range(nch):
            job(i)
        return
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(job, range(nch)))


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) values rounded to bf16."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def sink(s, vals):
        out[s:s + vals.size] = f32_to_bf16_bits(vals)

    _parallel_normal(rng, n, sink)
    return out.reshape(shape)


def normal_fp8(rng: np.random.Generator, shape):
    """N(0,1) values as fp8 e4m3fn codes with a per-tensor scale amax/448.

    Returns (codes uint8, scale float)."""
    import torch

    n = int(np.prod(shape))
    vals = np.empty(n, dtype=np.float32)

    def sink(s, v):
        vals[s:s + v.size] = v

    _parallel_normal(rng, n, sink)
    amax = float(np.abs(vals).max())
    scale = float(np.float32(amax / 448.0))
    out = np.empty(n, dtype=np.uint8)
    inv = np.float32(1.0 / scale)
    for s in range(0, n, _CHUNK * 8):
        e = min(n, s + _CHUNK * 8)
        t = torch.from_numpy(vals[s:e] * inv).clamp_(-448.0, 448.0)
        out[s:e] = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out.reshape(shape), scale


# ----------------------------------------------------------------------------
# cache and tables
# ----------------------------------------------------------------------------
@dataclass
class CacheSpec:
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    layout: str = "nhd"          # "nhd" | "preshuffled"
    dtype: str = "bf16"          # "bf16" | "fp8"

    @property
    def x(self) -> int:
        return 16 // (1 if self.dtype == "fp8" else 2) if self.layout == "preshuffled" else 0

    def shapes(self):
        nb, bs, H, D = self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim
        if self.layout == "nhd":
            return (nb, bs, H, D), (nb, bs, H, D)
        x = self.x
        return (nb, H, D // x, bs, x), (nb, H, bs // x, D, x)


@dataclass
class CacheData:
    spec: CacheSpec
    k: np.ndarray
    v: np.ndarray
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def poison_block(self) -> int:
        return self.spec.num_blocks - 1


def random_cache(rng, spec: CacheSpec) -> CacheData:
    ks, vs = spec.shapes()
    if spec.dtype == "bf16":
        return CacheData(spec, normal_bf16(rng, ks), normal_bf16(rng, vs))
    k, ksc = normal_fp8(rng, ks)
    v, vsc = normal_fp8(rng, vs)
    return CacheData(spec, k, v, ksc, vsc)


def block_tables_for(rng, capacities, block_size: int, num_blocks: int, pad_to: Optional[int] = None):
    """Fully fragmented tables: a permutation of blocks 0..num_blocks-2 (the
    last block is the poison block) sliced consecutively, one slice per
    request, long enough for ``capacities[i]`` tokens.  Padding entries point
    at the poison block."""
    need = [(int(c) + block_size - 1) // block_size for c in capacities]
    total = sum(need)
    if total > num_blocks - 1:
        raise ValueError(f"workload needs {total} blocks, cache has {num_blocks - 1}")
    perm = rng.permutation(num_blocks - 1).astype(np.int32)
    width = max(pad_to or 0, max(need) if need else 1, 1)
    tables = np.full((len(need), width), num_blocks - 1, dtype=np.int32)
    s = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[s:s + n]
        s += n
    return tables


def slots_for(tables, seq_idx, positions, block_size: int) -> np.ndarray:
    """Physical slot (block * block_size + offset) of logical positions."""
    seq_idx = np.asarray(seq_idx, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    blk = tables[seq_idx, positions // block_size].astype(np.int64)
    return blk * block_size + positions % block_size


def poison_cache(cache: CacheData, tables, lengths) -> None:
    """NaN-fill the poison block and every slot of each request past its
    length (in the blocks its table lists), in place."""
    sp = cache.spec
    nanv = BF16_NAN if sp.dtype == "bf16" else FP8_NAN
    cache.k[cache.poison_block] = nanv
    cache.v[cache.poison_block] = nanv
    bs = sp.block_size
    for i, L in enumerate(lengths):
        L = int(L)
        nblk = (L + bs - 1) // bs
        for j in range(nblk, tables.shape[1]):      # blocks reserved for growth
            blk = int(tables[i, j])
            cache.k[blk] = nanv
            cache.v[blk] = nanv
        if nblk == 0 or L % bs == 0:
            continue
        blk = int(tables[i, nblk - 1])
        for off in range(L % bs, bs):
            if sp.layout == "nhd":
                cache.k[blk, off] = nanv
                cache.v[blk, off] = nanv
            else:
                x = sp.x
                cache.k[blk, :, :, off, :] = nanv
                cache.v[blk, :, off // x, :, off % x] = nanv


# ----------------------------------------------------------------------------
# decode workloads
# ----------------------------------------------------------------------------
@dataclass
class DecodeStep:
    """One decode step: write the new token of every request at position
    seq_lens-1, then attend over seq_lens tokens."""
    cache: CacheData
    num_q_heads: int
    q: np.ndarray             # [B, H_q, D] bf16 bits
    k_new: np.ndarray         # [B, H_kv, D] bf16 bits
    v_new: np.ndarray
    slot_mapping: np.ndarray  # [B] int64
    block_tables: np.ndarray  # [B, max_blocks] int32
    seq_lens: np.ndarray      # [B] int32 (includes the new token)
    scale: float

    @property
    def batch(self) -> int:
        return self.q.shape[0]


def decode_workload(seed, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                    num_blocks, len_lo, len_hi, layout="nhd", dtype="bf16",
                    growth: int = 0, max_blocks: Optional[int] = None,
                    fixed_lens=None) -> DecodeStep:
    """``growth`` reserves table room for that many further tokens per request
    (multi-step decode); ``fixed_lens`` overrides the first lengths drawn."""
    rng = np.random.default_rng(seed)
    spec = CacheSpec(num_blocks, block_size, num_kv_heads, head_dim, layout, dtype)
    lens = rng.integers(len_lo, len_hi + 1, size=batch).astype(np.int32)
    if fixed_lens is not None:
        lens[:len(fixed_lens)] = fixed_lens
    tables = block_tables_for(rng, lens + growth, block_size, num_blocks, max_blocks)
    cache = random_cache(rng, spec)
    q = normal_bf16(rng, (batch, num_q_heads, head_dim))
    k_new = normal_bf16(rng, (batch, num_kv_heads, head_dim))
    v_new = normal_bf16(rng, (batch, num_kv_heads, head_dim))
    slots = slots_for(tables, np.arange(batch), lens - 1, block_size)
    return DecodeStep(cache, num_q_heads, q, k_new, v_new, slots, tables, lens,
                      float(1.0 / np.sqrt(head_dim)))


def next_decode_step(rng, step: DecodeStep) -> DecodeStep:
    """The following decode step: every request grows by one token."""
    sp = step.cache.spec
    B = step.batch
    lens = (step.seq_lens + 1).astype(np.int32)
    q = normal_bf16(rng, (B, step.num_q_heads, sp.head_dim))
    k_new = normal_bf16(rng, (B, sp.num_kv_heads, sp.head_dim))
    v_new = normal_bf16(rng, (B, sp.num_kv_heads, sp.head_dim))
    slots = slots_for(step.block_tables, np.arange(B), lens - 1, sp.block_size)
    return DecodeStep(step.cache, step.num_q_heads, q, k_new, v_new, slots,
                      step.block_tables, lens, step.scale)


def tiny_decode(seed=1):
    """Batch 4, 8:2 heads, D 128, block 16, 256 blocks, lengths [100, 512];
    eight consecutive steps are reserved in the tables."""
    return decode_workload(seed, 4, 8, 2, 128, 16, 256, 100, 512, growth=8)


def llama70b_decode_layer(seed=2, batch=64, len_lo=2048, len_hi=8192, num_blocks=32768):
    """Llama-3.1-70B-shaped decode layer: 64:8 heads, D 128, bf16, block 16."""
    return decode_workload(seed, batch, 64, 8, 128, 16, num_blocks, len_lo, len_hi)


def fp8_preshuffled_decode(seed=5, batch=128, len_lo=1000, len_hi=16000, num_blocks=131072):
    """fp8 e4m3 KV in the preshuffled layout (x = 16), 64:4 heads, D 128,
    block 16, Q and output bf16."""
    return decode_workload(seed, batch, 64, 4, 128, 16, num_blocks, len_lo, len_hi,
                           layout="preshuffled", dtype="fp8")


# ----------------------------------------------------------------------------
# layer pack / unpack
# ----------------------------------------------------------------------------
@dataclass
class PackJob:
    src_ids: np.ndarray      # [n] int32 distinct
    dst_ids: np.ndarray      # [n] int32 distinct (where the receiver unpacks)


def pack_job(seed, num_blocks, num_seqs=8, tokens_per_seq=10000, block_size=16) -> PackJob:
    """All blocks of ``num_seqs`` requests of ``tokens_per_seq`` tokens each:
    distinct random source ids, and a second random set of destination ids."""
    rng = np.random.default_rng(seed + 1000)
    n = num_seqs * ((tokens_per_seq + block_size - 1) // block_size)
    src = rng.permutation(num_blocks - 1)[:n].astype(np.int32)
    dst = rng.permutation(num_blocks - 1)[:n].astype(np.int32)
    return PackJob(src, dst)


# ----------------------------------------------------------------------------
# extend / prefill / mixed batches
# ----------------------------------------------------------------------------
@dataclass
class MixedBatch:
    """A batch already reordered [decode:extend:prefill].

    Token rows: decodes first (one row each), then the extends' new tokens,
    then the prefills' tokens.  Every row's K/V is written to the cache at
    ``slot_mapping`` before attention."""
    cache: CacheData
    num_q_heads: int
    scale: float
    q: np.ndarray             # [T, H_q, D]
    k_new: np.ndarray         # [T, H_kv, D]
    v_new: np.ndarray
    slot_mapping: np.ndarray  # [T] int64
    # decode part
    n_decode: int
    dec_tables: np.ndarray
    dec_seq_lens: np.ndarray  # includes the new token
    # extend part
    ext_cu_q: np.ndarray      # [E+1] int32, relative to the extend rows
    ext_ctx: np.ndarray       # [E] int32 cached tokens before this step
    ext_tables: np.ndarray
    # prefill part
    pre_cu: np.ndarray        # [P+1] int32, relative to the prefill rows
    # raw (arrival) order, for reorder tests
    raw_query_lens: np.ndarray = field(default=None)
    raw_ctx_lens: np.ndarray = field(default=None)

    @property
    def rows_decode(self):
        return 0, self.n_decode

    @property
    def rows_extend(self):
        return self.n_decode, self.n_decode + int(self.ext_cu_q[-1])

    @property
    def rows_prefill(self):
        s = self.n_decode + int(self.ext_cu_q[-1])
        return s, s + int(self.pre_cu[-1])


def mixed_batch(seed, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                dec_lens, ext_ctx, ext_new, pre_lens, layout="nhd", dtype="bf16") -> MixedBatch:
    """Build a reordered mixed batch from explicit per-request sizes."""
    rng = np.random.default_rng(seed)
    spec = CacheSpec(num_blocks, block_size, num_kv_heads, head_dim, layout, dtype)
    dec_lens = np.asarray(dec_lens, dtype=np.int32)
    ext_ctx = np.asarray(ext_ctx, dtype=np.int32)
    ext_new = np.asarray(ext_new, dtype=np.int32)
    pre_lens = np.asarray(pre_lens, dtype=np.int32)
    caps = list(dec_lens) + list(ext_ctx + ext_new) + list(pre_lens)
    all_tables = block_tables_for(rng, caps, block_size, num_blocks)
    nd, ne = len(dec_lens), len(ext_ctx)
    dec_tables = all_tables[:nd]
    ext_tables = all_tables[nd:nd + ne]
    pre_tables = all_tables[nd + ne:]
    cache = random_cache(rng, spec)
    T = nd + int(ext_new.sum()) + int(pre_lens.sum())
    q = normal_bf16(rng, (T, num_q_heads, head_dim))
    k_new = normal_bf16(rng, (T, num_kv_heads, head_dim))
    v_new = normal_bf16(rng, (T, num_kv_heads, head_dim))
    slots = []
    if nd:
        slots.append(slots_for(dec_tables, np.arange(nd), dec_lens - 1, block_size))
    for e in range(ne):
        pos = ext_ctx[e] + np.arange(ext_new[e])
        slots.append(slots_for(ext_tables, np.full(ext_new[e], e), pos, block_size))
    for p in range(len(pre_lens)):
        pos = np.arange(pre_lens[p])
        slots.append(slots_for(pre_tables, np.full(pre_lens[p], p), pos, block_size))
    slot_mapping = np.concatenate(slots).astype(np.int64) if slots else np.zeros(0, np.int64)
    ext_cu = np.concatenate([[0], np.cumsum(ext_new)]).astype(np.int32)
    pre_cu = np.concatenate([[0], np.cumsum(pre_lens)]).astype(np.int32)
    # arrival order: a random interleaving of the three kinds
    qlens = np.concatenate([np.ones(nd, np.int32), ext_new, pre_lens])
    ctxs = np.concatenate([dec_lens - 1, ext_ctx, np.zeros(len(pre_lens), np.int32)])
    arrival = rng.permutation(len(qlens))
    return MixedBatch(cache, num_q_heads, float(1.0 / np.sqrt(head_dim)), q, k_new, v_new,
                      slot_mapping, nd, dec_tables, dec_lens, ext_cu, ext_ctx, ext_tables,
                      pre_cu, qlens[arrival], ctxs[arrival])


def qwen3_mixed_batch(seed=3, n_decode=48, dec_lo=2000, dec_hi=3000, n_extend=4, ext_ctx=2000,
                      ext_new=512, n_prefill=2, pre_len=2000, num_blocks=12288) -> MixedBatch:
    """Qwen3-235B-A22B-shaped mixed batch: 64:4 heads, D 128, bf16, block 16;
    48 decodes with context in [2000, 3000], 4 extends of 512 new tokens on
    2000 cached tokens, 2 fresh 2000-token prefills."""
    rng = np.random.default_rng(seed + 7)
    dec_lens = rng.integers(dec_lo, dec_hi + 1, size=n_decode)
    return mixed_batch(seed, 64, 4, 128, 16, num_blocks, dec_lens, [ext_ctx] * n_extend,
                       [ext_new] * n_extend, [pre_len] * n_prefill)


def long_context_extend(seed=4, n_seq=2, ctx=100000, new=8192, num_blocks=16384) -> MixedBatch:
    """2 requests with 100000 cached tokens and 8192 new tokens each; 64:8
    heads, D 128, bf16, block 16 (an extend-only batch)."""
    return mixed_batch(seed, 64, 8, 128, 16, num_blocks, [], [ctx] * n_seq, [new] * n_seq, [])


def heavy_tailed_mixed_batch(seed=6, n_decode=64, n_extend=12, n_prefill=2,
                             num_blocks=20480) -> MixedBatch:
    """A serving batch with heavy-tailed lengths (prefix-cache hits and
    multi-turn requests: many short extends beside a few long ones), 64:4
    heads, D 128, bf16, block 16, reordered [decode:extend:prefill].
    Lengths are lognormal, rounded and clipped:
      decode contexts   median 2000, sigma 1.0, in [16, 32768]
      extend new tokens median 96,   sigma 1.3, in [2, 4096]
      extend contexts   median 3000, sigma 1.0, in [16, 32768]
      prefill lengths   median 1500, sigma 0.8, in [64, 8192]"""
    rng = np.random.default_rng(seed + 11)

    def lengths(n, median, sigma, lo, hi):
        x = rng.lognormal(np.log(median), sigma, size=n)
        return np.clip(np.rint(x), lo, hi).astype(np.int32)

    dec = lengths(n_decode, 2000, 1.0, 16, 32768)
    ext_new = lengths(n_extend, 96, 1.3, 2, 4096)
    ext_ctx = lengths(n_extend, 3000, 1.0, 16, 32768)
    pre = lengths(n_prefill, 1500, 0.8, 64, 8192)
    return mixed_batch(seed, 64, 4, 128, 16, num_blocks, dec, ext_ctx, ext_new, pre)


# ----------------------------------------------------------------------------
# MLA (absorbed latent) decode
# ----------------------------------------------------------------------------
@dataclass
class MlaDecode:
    cache: np.ndarray         # [num_blocks, block_size, 576] bf16 bits
    q: np.ndarray             # [B, H, 576] bf16 bits (absorbed queries)
    block_tables: np.ndarray  # [B, max_blocks] int32
    seq_lens: np.ndarray      # [B] int32
    block_size: int
    scale: float

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]


def mla_decode_workload(seed, batch, num_heads, block_size, num_blocks, len_lo, len_hi,
                        fixed_lens=None, latent=576) -> MlaDecode:
    """Latent rows and absorbed queries N(0,1) in bf16; fully fragmented
    tables (the last block is the poison block); scale 1/sqrt(576)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(len_lo, len_hi + 1, size=batch).astype(np.int32)
    if fixed_lens is not None:
        lens[:len(fixed_lens)] = fixed_lens
    tables = block_tables_for(rng, lens, block_size, num_blocks)
    cache = normal_bf16(rng, (num_blocks, block_size, latent))
    q = normal_bf16(rng, (batch, num_heads, latent))
    return MlaDecode(cache, q, tables, lens, block_size, float(1.0 / np.sqrt(latent)))


def deepseek_mla_decode(seed=7, batch=128, len_lo=10000, len_hi=11000,
                        num_blocks=90112) -> MlaDecode:
    """One GPU's share of DeepSeek-R1 MLA decode under TP8: 16 of the 128
    query heads over the (replicated) 576-dim latent cache, block 16, batch
    128 at ISL 10K + up to 1K generated tokens."""
    return mla_decode_workload(seed, batch, 16, 16, num_blocks, len_lo, len_hi)
