"""Paged KV cache model -- oracle side.  TEST INFRASTRUCTURE ONLY.

Block table ("From LLM performance optimisation to DeepSeek deployment",
section 3 "Paged Attention"): the KV cache is cut into fixed-size blocks that
need not be contiguous; each request owns a block table that maps its logical
block i (tokens i*bs .. i*bs+bs-1) to a physical block, like a page table.
So logical token t of a request lives in physical block table[t // bs] at
offset t % bs.

Layouts of one layer's cache (per "Beyond just running: native inference
optimisation in vLLM on AMD ROCm"):
* "nhd" -- the standard layout.  The page contrasts the preshuffled layout with
  a "standard" one without spelling it out; the reading taken is the paged form
  of its prefill layout [num_tokens, num_heads, head_dim] (section "Processing
  details of the three paths"): k, v = [num_blocks, block_size, H_kv, D].
* "preshuffled" -- section "ROCM_AITER_FA", hardware-oriented KV cache layout:
  k = [num_blocks, H_kv, D // x, block_size, x], v = [num_blocks, H_kv,
  block_size // x, D, x].  x is left undefined on the page; reading: x = 16
  bytes / element size (16 for fp8, 8 for bf16).

Element types: "bf16" (uint16 bit patterns) or "fp8" (OCP e4m3fn codes, uint8,
with per-tensor k_scale / v_scale; value = code * scale).

Slot mapping (the cache write of section "Unified attention backends", stage 1:
new K/V are written into the cache before attention): the pages only say that
the new key/value go into the cache.  Reading: slot = block_id * block_size +
offset as int64; a negative slot marks a padding token that is not written.

Layer pack / unpack ("Advanced inference: why your single-node vLLM setup needs
prefill/decode disaggregation", section "Architecture", write mode: after each
layer the prefill side pushes that layer's KV blocks into blocks preallocated on
the decode side; the handshake shares base address, block size and per-layer
stride).  Reading of the buffer format: [K of blocks ids[0..n) in id-list order]
followed by [V of the same blocks], each block's bytes verbatim.  One block of
one layer is contiguous in both layouts, so this is layout-agnostic.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from . import bf16, fp8


@dataclass
class Cache:
    k: np.ndarray
    v: np.ndarray
    layout: str            # "nhd" | "preshuffled"
    dtype: str             # "bf16" | "fp8"
    block_size: int
    num_kv_heads: int
    head_dim: int
    x: int = 0             # preshuffled only
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_blocks(self) -> int:
        return self.k.shape[0]

    def copy(self) -> "Cache":
        return replace(self, k=self.k.copy(), v=self.v.copy())


def _values(cache: Cache, raw: np.ndarray, scale: float) -> np.ndarray:
    if cache.dtype == "bf16":
        return bf16.to_f64(raw)
    return fp8.decode(raw) * np.float64(np.float32(scale))


def token_location(table_row, t, block_size):
    """Logical token t -> (physical block, offset) through the block table."""
    t = np.asarray(t, dtype=np.int64)
    blk = np.asarray(table_row, dtype=np.int64)[t // block_size]
    return blk, t % block_size


def gather(cache: Cache, table_row, length: int):
    """K and V of one request's first ``length`` tokens, float64 [L, H_kv, D].

    Reads nothing past token length-1 and no table entry past
    ceil(length / block_size) - 1.
    """
    t = np.arange(length, dtype=np.int64)
    blk, off = token_location(table_row[: (length + cache.block_size - 1) // cache.block_size],
                              t, cache.block_size)
    H, D = cache.num_kv_heads, cache.head_dim
    if cache.layout == "nhd":
        kraw = cache.k[blk, off]                      # [L, H, D]
        vraw = cache.v[blk, off]
    else:
        x = cache.x
        h = np.arange(H)[None, :, None]
        d = np.arange(D)[None, None, :]
        b3 = blk[:, None, None]
        o3 = off[:, None, None]
        kraw = cache.k[b3, h, d // x, o3, d % x]      # K[t,h,d] = k[blk,h,d//x,off,d%x]
        vraw = cache.v[b3, h, o3 // x, d, o3 % x]     # V[t,h,d] = v[blk,h,off//x,d,off%x]
    return _values(cache, kraw, cache.k_scale), _values(cache, vraw, cache.v_scale)


def write(cache: Cache, k_bits, v_bits, slot_mapping) -> Cache:
    """Slot-mapped store of new tokens' K/V ([T, H_kv, D] bf16 bits).

    bf16 caches receive the bf16 bits unchanged; fp8 caches receive
    fp8.quantize(value, scale) (an fp32 product, then round-half-even with
    saturation).  Returns an updated copy; slots < 0 are skipped.
    """
    out = cache.copy()
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    bs, x = cache.block_size, cache.x
    H, D = cache.num_kv_heads, cache.head_dim
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = int(s // bs), int(s % bs)
        if cache.dtype == "bf16":
            kv = (k_bits[i], v_bits[i])
        else:
            kf = (k_bits[i].astype(np.uint32) << 16).view(np.float32)
            vf = (v_bits[i].astype(np.uint32) << 16).view(np.float32)
            kv = (fp8.quantize(kf, cache.k_scale), fp8.quantize(vf, cache.v_scale))
        if cache.layout == "nhd":
            out.k[blk, off] = kv[0]
            out.v[blk, off] = kv[1]
        else:
            h = np.arange(H)[:, None]
            d = np.arange(D)[None, :]
            out.k[blk, h, d // x, off, d % x] = kv[0]
            out.v[blk, h, off // x, d, off % x] = kv[1]
    return out


def packed_bytes(cache: Cache, n: int) -> int:
    """Size of a packed layer: n blocks of K plus n blocks of V."""
    return 2 * n * int(cache.k[0].nbytes)


def pack_layer(cache: Cache, block_ids) -> np.ndarray:
    ids = np.asarray(block_ids, dtype=np.int64)
    kb = np.ascontiguousarray(cache.k[ids]).view(np.uint8).reshape(-1)
    vb = np.ascontiguousarray(cache.v[ids]).view(np.uint8).reshape(-1)
    return np.concatenate([kb, vb])


def unpack_layer(cache: Cache, block_ids, buf) -> Cache:
    ids = np.asarray(block_ids, dtype=np.int64)
    buf = np.asarray(buf, dtype=np.uint8)
    out = cache.copy()
    n = len(ids)
    per = int(cache.k[0].nbytes)
    if buf.size != 2 * n * per:
        raise ValueError("packed buffer size mismatch")
    kpart = buf[: n * per].view(cache.k.dtype).reshape((n,) + cache.k.shape[1:])
    vpart = buf[n * per:].view(cache.v.dtype).reshape((n,) + cache.v.shape[1:])
    out.k[ids] = kpart
    out.v[ids] = vpart
    return out
