"""Exact softmax attention for the three request paths -- oracle side.
TEST INFRASTRUCTURE ONLY.

"Beyond just running: native inference optimisation in vLLM on AMD ROCm",
section "Every batch handles a mixed workload", names three kinds of request in
one batch:
* prefill -- a fresh prompt, all of whose tokens attend at once;
* extend  -- more prompt tokens for a request whose KV cache is already partly
  built; the new tokens attend both to the cached context and to this round's
  new tokens;
* decode  -- one new token that reads the request's whole KV cache.
Section "Processing details of the three paths" fixes the prefill layout
[num_tokens, num_heads, head_dim] and the extend method (new-token attention,
then per context chunk attention + LSE merge, then a final merge).  Chunking and
the LSE merge are exact rearrangements of one softmax, so the oracle computes
the plain definition over the full visible key set, with no chunking, no online
softmax and no tiling:

  s_j = scale * <q, k_j>  over the visible set S,  m = max_j s_j,
  l = sum_j exp(s_j - m),  o = sum_j exp(s_j - m) v_j / l,  lse = m + ln l.

Readings where the pages are silent (each listed with the other readings in the
design notes):
* scale = 1/sqrt(head_dim) unless given; lse is natural-log and includes scale.
* grouped-query heads: query head h uses KV head h // (H_q / H_kv).
* extend causality is bottom-right aligned: new token i of a request with C
  cached tokens sits at absolute position C + i and sees cached tokens 0..C-1
  and new tokens 0..i.
* prefill is causal within each sequence of the varlen batch; sequences are
  delimited by cu_seqlens (exclusive prefix sums of lengths).
All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np

from . import cache as cache_mod


def attend(q, K, V, scale, visible=None):
    """q [n, D], K/V [m, D] float64, visible [n, m] bool (None = all).

    Returns (o [n, D], lse [n]).  A row with nothing visible gets o = 0 and
    lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = scale * (q @ K.T)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True) if s.shape[1] else np.full((s.shape[0], 1), -np.inf)
    empty = ~np.isfinite(m[:, 0])
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)
    if visible is not None:
        e = np.where(visible, e, 0.0)
    l = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = (e @ V) / l[:, None]
        lse = m[:, 0] + np.log(l)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse


def paged_decode(q, cache: "cache_mod.Cache", block_tables, seq_lens, scale):
    """Decode path: q [B, H_q, D] float64; request b attends to its first
    seq_lens[b] cached tokens, gathered through block_tables[b].
    Returns out [B, H_q, D], lse [B, H_q]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // cache.num_kv_heads
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        K, V = cache_mod.gather(cache, block_tables[b], int(seq_lens[b]))
        for h in range(Hq):
            g = h // G
            o, l = attend(q[b, h][None, :], K[:, g, :], V[:, g, :], scale)
            out[b, h], lse[b, h] = o[0], l[0]
    return out, lse


def _rows_of(seq_start, seq_len, rows):
    if rows is None:
        return np.arange(seq_len)
    r = np.asarray([x - seq_start for x in rows if seq_start <= x < seq_start + seq_len],
                   dtype=np.int64)
    return r


def prefill(q, k, v, cu_seqlens, scale, causal=True, rows=None):
    """Prefill path over a varlen batch.

    q [T, H_q, D], k/v [T, H_kv, D] float64; sequence n owns tokens
    cu_seqlens[n] .. cu_seqlens[n+1]-1.  With ``rows`` (global token indices)
    only those rows are computed; the others are returned as NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for n in range(len(cu) - 1):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        L = s1 - s0
        ri = _rows_of(s0, L, rows)
        if L == 0 or ri.size == 0:
            continue
        j = np.arange(L)
        vis = (j[None, :] <= ri[:, None]) if causal else np.ones((ri.size, L), bool)
        for h in range(Hq):
            g = h // G
            o, l = attend(q[s0 + ri, h], k[s0:s1, g], v[s0:s1, g], scale, vis)
            out[s0 + ri, h], lse[s0 + ri, h] = o, l
    return out, lse


def extend(q, k_new, v_new, cu_q_lens, ctx_lens, cache: "cache_mod.Cache",
           block_tables, scale, rows=None):
    """Extend path: request e has ctx_lens[e] cached tokens (read through
    block_tables[e]) and new tokens cu_q_lens[e] .. cu_q_lens[e+1]-1 whose
    q/k/v are given.  New token i sees every cached token and new tokens 0..i.
    With ``rows`` only those global new-token rows are computed (others NaN)."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    G = Hq // cache.num_kv_heads
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    for e in range(len(cu) - 1):
        s0, s1 = int(cu[e]), int(cu[e + 1])
        n = s1 - s0
        C = int(ctx_lens[e])
        ri = _rows_of(s0, n, rows)
        if n == 0 or ri.size == 0:
            continue
        Kc, Vc = cache_mod.gather(cache, block_tables[e], C)
        K = np.concatenate([Kc, np.asarray(k_new[s0:s1], dtype=np.float64)], axis=0)
        V = np.concatenate([Vc, np.asarray(v_new[s0:s1], dtype=np.float64)], axis=0)
        j = np.arange(C + n)
        vis = (j[None, :] < C) | ((j[None, :] - C) <= ri[:, None])
        for h in range(Hq):
            g = h // G
            o, l = attend(q[s0 + ri, h], K[:, g], V[:, g], scale, vis)
            out[s0 + ri, h], lse[s0 + ri, h] = o, l
    return out, lse
