"""Paged KV-cache attention for mixed serving batches on AMD Instinct MI355X.

Thin ctypes binding over ``libpagedkv.so`` (declared in ``include/pagedkv.h``):
argument marshalling only -- every step of the attention path runs in the
library's gfx950 HIP kernels.  PyTorch supplies device memory and the current
HIP stream.  The binding refuses to run when the library has not been built;
there is no fallback implementation.

Calls (same names as the C ABI):
    kv_write, paged_decode, paged_decode_noalloc, prefill_attn, extend_attn,
    mla_decode, kv_layer_packed_bytes, kv_pack_layer, kv_unpack_layer,
    reorder_batch
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

KV_OK, KV_EINVAL, KV_ENOSPC, KV_ENOTSUP, KV_EHIP = 0, -22, -28, -95, -1000
KV_DTYPE_BF16, KV_DTYPE_FP8_E4M3 = 0, 1
KV_LAYOUT_NHD, KV_LAYOUT_PRESHUFFLED = 0, 1
KV_EXTEND_AUTO, KV_EXTEND_SPLIT, KV_EXTEND_FUSED = 0, 1, 2
_EXTEND_MODES = {"auto": KV_EXTEND_AUTO, "split": KV_EXTEND_SPLIT, "fused": KV_EXTEND_FUSED}


class PagedKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class KVCacheT(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32), ("x", ctypes.c_int32),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
    ]


_P, _I32, _SZ, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
_PC = ctypes.POINTER(KVCacheT)
_SIGS = {
    "kv_write": (ctypes.c_int, [_PC, _P, _P, _P, _I32, _P]),
    "paged_decode_workspace_bytes": (_SZ, [_PC, _I32, _I32, _I32]),
    "paged_decode_workspace_bytes_ex": (_SZ, [_PC, _I32, _I32, _I32, _I32]),
    "paged_decode": (ctypes.c_int, [_PC, _P, _I32, _I32, _P, _I32, _P, _I32, _F, _P, _P, _P, _SZ, _P]),
    "paged_decode_ex": (ctypes.c_int, [_PC, _P, _I32, _I32, _P, _I32, _P, _I32, _F, _P, _P, _P, _SZ,
                                       _I32, _P]),
    "paged_decode_noalloc": (ctypes.c_int, [_PC, _P, _I32, _I32, _P, _I32, _P, _I32, _F, _P, _P,
                                            _P]),
    "prefill_attn": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F, _I32, _P, _P, _P]),
    "extend_attn_workspace_bytes": (_SZ, [_PC, _I32, _I32, _I32, _I32, _I32]),
    "extend_attn": (ctypes.c_int, [_PC, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                   _I32, _F, _P, _P, _P, _SZ, _P]),
    "extend_attn_workspace_bytes_ex": (_SZ, [_PC, _I32, _I32, _I32, _I32, _I32, _I32]),
    "extend_attn_ex": (ctypes.c_int, [_PC, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                      _I32, _I32, _F, _P, _P, _P, _SZ, _I32, _P]),
    "mla_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "mla_decode": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _I32, _I32, _P, _I32, _P, _I32, _F,
                                  _P, _P, _P, _SZ, _P]),
    "kv_layer_packed_bytes": (_SZ, [_PC, _I32]),
    "kv_pack_layer": (ctypes.c_int, [_PC, _P, _I32, _P, _SZ, _P]),
    "kv_unpack_layer": (ctypes.c_int, [_PC, _P, _I32, _P, _SZ, _P]),
    "kv_reorder_batch": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
    "kv_last_error": (ctypes.c_char_p, []),
    "kv_abi_version": (ctypes.c_int, []),
}
EXPORTS = tuple(_SIGS)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_mapped_amd.build` (no fallback exists)")
        # torch first: its wheel carries its own HIP runtime (soname
        # libamdhip64.so.7).  Loaded after it, the library binds to that same
        # runtime; loaded before it, the library would pull the system's copy
        # and the process would hold two runtimes, whose devices, streams and
        # allocations are not each other's (the library's calls then fail).
        _t()
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(code: int) -> None:
    if code != KV_OK:
        raise PagedKVError(code, lib().kv_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _want(t, name: str, dtypes, ndim: Optional[int] = None, optional: bool = False) -> None:
    """Refuse a tensor the C ABI would misread: wrong element type, wrong rank
    or not contiguous.  `dtypes` is a tuple of torch dtypes."""
    if t is None:
        if optional:
            return
        raise TypeError(f"{name} is required")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, "
                        f"got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors) -> None:
    """Every given tensor (None skipped) lives in GPU memory."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def _t():
    import torch
    return torch


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


class PagedKVCache:
    """One layer's paged KV cache: two device tensors plus their description.

    layout "nhd":         k, v [num_blocks, block_size, H_kv, D]
    layout "preshuffled": k [num_blocks, H_kv, D/x, block_size, x],
                          v [num_blocks, H_kv, block_size/x, D, x]
    dtype "bf16" (torch.bfloat16 tensors) or "fp8" (torch.uint8 codes,
    OCP e4m3fn, value = code * scale)."""

    def __init__(self, k, v, block_size: int, num_kv_heads: int, head_dim: int,
                 layout: str = "nhd", dtype: str = "bf16", k_scale: float = 1.0,
                 v_scale: float = 1.0):
        if layout not in ("nhd", "preshuffled") or dtype not in ("bf16", "fp8"):
            raise ValueError(f"unknown layout/dtype {layout}/{dtype}")
        t = _t()
        want = (t.bfloat16,) if dtype == "bf16" else (t.uint8, t.float8_e4m3fn)
        _want(k, "k_cache", want)
        _want(v, "v_cache", want)
        if k.numel() != v.numel() or k.shape[0] != v.shape[0]:
            raise ValueError("k_cache and v_cache must hold the same blocks")
        _on_gpu(k_cache=k, v_cache=v)
        self.k, self.v = k, v
        self.block_size, self.num_kv_heads, self.head_dim = block_size, num_kv_heads, head_dim
        self.layout, self.dtype = layout, dtype
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.num_blocks = int(k.shape[0])
        self.x = (16 if dtype == "fp8" else 8) if layout == "preshuffled" else 0

    def desc(self) -> KVCacheT:
        return KVCacheT(self.k.data_ptr(), self.v.data_ptr(), self.num_blocks, self.block_size,
                        self.num_kv_heads, self.head_dim,
                        KV_DTYPE_BF16 if self.dtype == "bf16" else KV_DTYPE_FP8_E4M3,
                        KV_LAYOUT_NHD if self.layout == "nhd" else KV_LAYOUT_PRESHUFFLED,
                        self.x, self.k_scale, self.v_scale)


def kv_write(cache: PagedKVCache, k, v, slot_mapping) -> None:
    """Store k, v [T, H_kv, D] bf16 at slot_mapping [T] int64 (negative = skip)."""
    t = _t()
    _want(k, "k", (t.bfloat16,), 3)
    _want(v, "v", (t.bfloat16,), 3)
    _want(slot_mapping, "slot_mapping", (t.int64,), 1)
    if k.shape != v.shape or slot_mapping.shape[0] != k.shape[0]:
        raise ValueError("k, v and slot_mapping disagree on the number of tokens")
    if k.shape[1] != cache.num_kv_heads or k.shape[2] != cache.head_dim:
        raise ValueError("k/v heads or head_dim do not match the cache")
    _on_gpu(k=k, v=v, slot_mapping=slot_mapping)
    d = cache.desc()
    _check(lib().kv_write(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(slot_mapping),
                          int(k.shape[0]), _stream(k)))


def paged_decode_workspace_bytes(cache: PagedKVCache, batch: int, num_q_heads: int,
                                 max_seq_len: int, split_tokens: int = 0) -> int:
    d = cache.desc()
    return int(lib().paged_decode_workspace_bytes_ex(ctypes.byref(d), batch, num_q_heads,
                                                     max_seq_len, split_tokens))


def paged_decode(cache: PagedKVCache, q, block_tables, seq_lens, max_seq_len: int, scale: float,
                 out=None, lse=None, workspace=None, split_tokens: int = 0):
    """q [B, H_q, D] bf16 -> (out [B, H_q, D] bf16, lse [B, H_q] fp32)."""
    import torch
    _want(q, "q", (torch.bfloat16,), 3)
    _want(block_tables, "block_tables", (torch.int32,), 2)
    _want(seq_lens, "seq_lens", (torch.int32,), 1)
    _want(out, "out", (torch.bfloat16,), 3, optional=True)
    _want(lse, "lse", (torch.float32,), 2, optional=True)
    _want(workspace, "workspace", (torch.uint8,), 1, optional=True)
    B, Hq, D = q.shape
    if block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_tables / seq_lens must have one row per request")
    _on_gpu(q=q, block_tables=block_tables, seq_lens=seq_lens, out=out, lse=lse,
            workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = paged_decode_workspace_bytes(cache, B, Hq, max_seq_len, split_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    d = cache.desc()
    _check(lib().paged_decode_ex(ctypes.byref(d), _ptr(q), B, Hq, _ptr(block_tables),
                                 int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len),
                                 float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                 int(workspace.numel() * workspace.element_size()),
                                 int(split_tokens), _stream(q)))
    return out, lse


def paged_decode_noalloc(cache: PagedKVCache, q, block_tables, seq_lens, max_seq_len: int,
                         scale: float, out, lse=None):
    """paged_decode into a caller-given `out` with the library's static
    scratch instead of a workspace (no allocation anywhere in the call)."""
    import torch
    _want(q, "q", (torch.bfloat16,), 3)
    _want(block_tables, "block_tables", (torch.int32,), 2)
    _want(seq_lens, "seq_lens", (torch.int32,), 1)
    _want(out, "out", (torch.bfloat16,), 3)
    _want(lse, "lse", (torch.float32,), 2, optional=True)
    B, Hq, D = q.shape
    if block_tables.shape[0] != B or seq_lens.shape[0] != B or out.shape != q.shape:
        raise ValueError("block_tables / seq_lens / out must match q's batch")
    _on_gpu(q=q, block_tables=block_tables, seq_lens=seq_lens, out=out, lse=lse)
    d = cache.desc()
    _check(lib().paged_decode_noalloc(ctypes.byref(d), _ptr(q), B, Hq, _ptr(block_tables),
                                      int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len),
                                      float(scale), _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def prefill_attn(q, k, v, cu_seqlens, max_seqlen: int, scale: float, causal: bool = True,
                 out=None, lse=None):
    """Varlen prefill: q [T, H_q, D], k/v [T, H_kv, D] bf16, cu_seqlens [N+1] int32."""
    import torch
    for name, x in (("q", q), ("k", k), ("v", v)):
        _want(x, name, (torch.bfloat16,), 3)
    _want(cu_seqlens, "cu_seqlens", (torch.int32,), 1)
    _want(out, "out", (torch.bfloat16,), 3, optional=True)
    _want(lse, "lse", (torch.float32,), 2, optional=True)
    T, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != T:
        raise ValueError("q, k and v disagree on the number of tokens")
    _on_gpu(q=q, k=k, v=v, cu_seqlens=cu_seqlens, out=out, lse=lse)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _check(lib().prefill_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                              int(cu_seqlens.shape[0]) - 1, int(max_seqlen), Hq, int(k.shape[1]), D,
                              float(scale), 1 if causal else 0, _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def extend_attn_workspace_bytes(cache: PagedKVCache, num_seqs: int, total_new: int,
                                num_q_heads: int, max_ctx_len: int, chunk_budget_tokens: int,
                                mode: str = "auto") -> int:
    d = cache.desc()
    return int(lib().extend_attn_workspace_bytes_ex(ctypes.byref(d), num_seqs, total_new,
                                                    num_q_heads, max_ctx_len, chunk_budget_tokens,
                                                    _EXTEND_MODES[mode]))


def extend_attn(cache: PagedKVCache, q, k_new, v_new, cu_q_lens, ctx_lens, block_tables,
                max_q_len: int, max_ctx_len: int, scale: float, chunk_budget_tokens: int = 32768,
                out=None, lse=None, workspace=None, mode: str = "auto"):
    """Extend: q [T, H_q, D], k_new/v_new [T, H_kv, D] bf16; cached context
    through block_tables.  mode: "auto", "split" (per-chunk partials + LSE
    merge pass) or "fused" (one running state per row block).
    Returns (out, lse)."""
    import torch
    for name, x in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        _want(x, name, (torch.bfloat16,), 3)
    _want(cu_q_lens, "cu_q_lens", (torch.int32,), 1)
    _want(ctx_lens, "ctx_lens", (torch.int32,), 1)
    _want(block_tables, "block_tables", (torch.int32,), 2, optional=True)
    _want(out, "out", (torch.bfloat16,), 3, optional=True)
    _want(lse, "lse", (torch.float32,), 2, optional=True)
    _want(workspace, "workspace", (torch.uint8,), 1, optional=True)
    if mode not in _EXTEND_MODES:
        raise ValueError(f"mode must be one of {sorted(_EXTEND_MODES)}")
    T, Hq, D = q.shape
    E = int(cu_q_lens.shape[0]) - 1
    if ctx_lens.shape[0] != E or (block_tables is not None and block_tables.shape[0] != E):
        raise ValueError("ctx_lens / block_tables must have one row per request")
    _on_gpu(q=q, k_new=k_new, v_new=v_new, cu_q_lens=cu_q_lens, ctx_lens=ctx_lens,
            block_tables=block_tables, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    need = extend_attn_workspace_bytes(cache, E, T, Hq, max_ctx_len, chunk_budget_tokens, mode)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    d = cache.desc()
    mb = int(block_tables.shape[1]) if block_tables is not None else 0
    _check(lib().extend_attn_ex(ctypes.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new),
                                _ptr(cu_q_lens), _ptr(ctx_lens), _ptr(block_tables), mb, E, T,
                                int(max_q_len), int(max_ctx_len), Hq, int(chunk_budget_tokens),
                                float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                int(workspace.numel() * workspace.element_size()),
                                _EXTEND_MODES[mode], _stream(q)))
    return out, lse


def mla_decode(kv_cache, q, block_tables, seq_lens, max_seq_len: int, scale: float,
               out=None, lse=None, workspace=None):
    """Absorbed MLA decode: kv_cache [num_blocks, block_size, 576] bf16 latent
    rows, q [B, H, 576] bf16 -> (out [B, H, 512] bf16, lse [B, H] fp32)."""
    import torch
    _want(kv_cache, "kv_cache", (torch.bfloat16,), 3)
    _want(q, "q", (torch.bfloat16,), 3)
    _want(block_tables, "block_tables", (torch.int32,), 2)
    _want(seq_lens, "seq_lens", (torch.int32,), 1)
    _want(out, "out", (torch.bfloat16,), 3, optional=True)
    _want(lse, "lse", (torch.float32,), 2, optional=True)
    _want(workspace, "workspace", (torch.uint8,), 1, optional=True)
    B, H, Dk = q.shape
    if block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_tables / seq_lens must have one row per request")
    _on_gpu(kv_cache=kv_cache, q=q, block_tables=block_tables, seq_lens=seq_lens, out=out,
            lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    need = int(lib().mla_decode_workspace_bytes(B, H, int(max_seq_len)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib().mla_decode(_ptr(kv_cache), int(kv_cache.shape[0]), int(kv_cache.shape[1]),
                            int(kv_cache.shape[2]), 512, _ptr(q), B, H, _ptr(block_tables),
                            int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len),
                            float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                            int(workspace.numel()), _stream(q)))
    return out, lse


def kv_layer_packed_bytes(cache: PagedKVCache, n: int) -> int:
    d = cache.desc()
    return int(lib().kv_layer_packed_bytes(ctypes.byref(d), n))


def kv_pack_layer(cache: PagedKVCache, block_ids, dst=None):
    """Gather blocks block_ids [n] int32 of this layer into dst (uint8)."""
    import torch
    _want(block_ids, "block_ids", (torch.int32,), 1)
    _want(dst, "dst", (torch.uint8,), 1, optional=True)
    _on_gpu(block_ids=block_ids, dst=dst)
    n = int(block_ids.shape[0])
    need = kv_layer_packed_bytes(cache, n)
    if dst is None:
        dst = torch.empty(need, dtype=torch.uint8, device=block_ids.device)
    d = cache.desc()
    _check(lib().kv_pack_layer(ctypes.byref(d), _ptr(block_ids), n, _ptr(dst),
                               int(dst.numel() * dst.element_size()), _stream(block_ids)))
    return dst


def kv_unpack_layer(cache: PagedKVCache, block_ids, src) -> None:
    """Scatter a packed buffer into blocks block_ids [n] int32 of this layer."""
    t = _t()
    _want(block_ids, "block_ids", (t.int32,), 1)
    _want(src, "src", (t.uint8,), 1)
    _on_gpu(block_ids=block_ids, src=src)
    d = cache.desc()
    _check(lib().kv_unpack_layer(ctypes.byref(d), _ptr(block_ids), int(block_ids.shape[0]),
                                 _ptr(src), int(src.numel() * src.element_size()), _stream(block_ids)))


def reorder_batch(query_lens: Sequence[int], ctx_lens: Sequence[int],
                  threshold: int = 1) -> Tuple[list, Tuple[int, int, int]]:
    """Host-side [decode:extend:prefill] reorder -> (perm, (n_decode, n_extend, n_prefill))."""
    n = len(query_lens)
    Q = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in query_lens])
    C = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in ctx_lens])
    P = (ctypes.c_int32 * max(n, 1))()
    K = (ctypes.c_int32 * 3)()
    _check(lib().kv_reorder_batch(ctypes.addressof(Q), ctypes.addressof(C), n, int(threshold),
                                  ctypes.addressof(P), ctypes.addressof(K)))
    return list(P)[:n], (K[0], K[1], K[2])
