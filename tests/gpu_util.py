"""Helpers for the GPU parity tests: move synthetic numpy workloads to the
device and build the matching oracle objects.  Not a test module."""
from __future__ import annotations

import sys

import numpy as np

import paged_kv_cache_mapped_amd as pk
from oracle import cache as oc

BF16_TOL = 1.5e-2     # max |err| of bf16 outputs
FP8_TOL = 5e-2        # max |err| with an fp8 KV cache
LSE_TOL = 1e-3        # max |err| of lse


def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need an MI355X (torch.cuda.is_available() is False)"
    return t


def say(msg: str) -> None:
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype=None):
    """numpy -> cuda tensor; uint16 bf16 bit patterns become torch.bfloat16."""
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).cuda()
    x = t.from_numpy(np.ascontiguousarray(a)).cuda()
    return x if dtype is None else x.to(dtype)


def host_bits(x) -> np.ndarray:
    """cuda tensor -> numpy (bf16 as uint16 bits, fp8 caches as uint8)."""
    t = torch()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def bf16_to_f64(x) -> np.ndarray:
    b = host_bits(x)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def device_cache(cd) -> pk.PagedKVCache:
    sp = cd.spec
    return pk.PagedKVCache(dev(cd.k), dev(cd.v), sp.block_size, sp.num_kv_heads, sp.head_dim,
                           sp.layout, sp.dtype, cd.k_scale, cd.v_scale)


def oracle_cache(cd) -> oc.Cache:
    sp = cd.spec
    return oc.Cache(cd.k, cd.v, sp.layout, sp.dtype, sp.block_size, sp.num_kv_heads,
                    sp.head_dim, sp.x, cd.k_scale, cd.v_scale)


def oracle_cache_from_device(dc: pk.PagedKVCache, like: oc.Cache) -> oc.Cache:
    return oc.Cache(host_bits(dc.k), host_bits(dc.v), like.layout, like.dtype, like.block_size,
                    like.num_kv_heads, like.head_dim, like.x, like.k_scale, like.v_scale)


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    assert got.shape == ref.shape
    assert not np.isnan(got).any(), "NaN in GPU output"
    return float(np.max(np.abs(got - ref))) if got.size else 0.0
