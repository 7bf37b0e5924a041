"""Absorbed multi-head latent attention (MLA) decode over a paged latent
cache -- oracle side.  TEST INFRASTRUCTURE ONLY.

"Beyond just running: native inference optimisation in vLLM on AMD ROCm",
section "AITER MLA backend: optimised for DeepSeek": DeepSeek / Kimi MLA
compress the KV cache to one 576-dimensional latent row per token (about 14x
less than the roughly 8K dimensions of standard MHA); decode is "absorbed":
it works directly in that latent space, one row shared by every query head,
and stays bound by memory bandwidth; the MLA benchmark runs with block size
16.  Paging follows "From LLM performance optimisation to DeepSeek
deployment", section 3 "Paged Attention" (block table).

Reading taken where the pages stop (each listed in the design notes): the
latent row is [c (512 dims) | k_rope (64 dims)], the split of DeepSeek's
published MLA; the score of query head h against token j uses the whole row,
s = scale * <q_h, row_j> (q_h is the absorbed 576-dim query), and the value
is the compressed part c_j (the first 512 dims), so the output is the
512-dim latent o_h = sum_j softmax(s)_j c_j (its up-projection belongs to
the model, not to attention).  lse is natural-log and includes the scale.

Cache layout: [num_blocks][block_size][576] bf16 (uint16 bit patterns);
token t of a request is in block table[t // bs] at offset t % bs.
All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np

from . import bf16
from .attention import attend

LATENT_DIMS = 576     # cache row (the page's figure)
VALUE_DIMS = 512      # compressed KV part used as the value (reading)


def gather_latent(cache_bits, table_row, length: int, block_size: int):
    """The first `length` latent rows of one request, float64 [L, 576]."""
    t = np.arange(length, dtype=np.int64)
    blk = np.asarray(table_row, dtype=np.int64)[t // block_size]
    return bf16.to_f64(cache_bits[blk, t % block_size])


def mla_decode(q, cache_bits, block_tables, seq_lens, scale, block_size=16,
               value_dims=VALUE_DIMS):
    """q [B, H, 576] float64 (absorbed queries); cache_bits [nb, bs, 576]
    bf16 bits.  Returns out [B, H, value_dims], lse [B, H]; a request of
    length 0 gets out = 0, lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    B, H, _ = q.shape
    out = np.zeros((B, H, value_dims))
    lse = np.zeros((B, H))
    for b in range(B):
        R = gather_latent(cache_bits, block_tables[b], int(seq_lens[b]), block_size)
        o, l = attend(q[b], R, R[:, :value_dims], scale)
        out[b], lse[b] = o, l
    return out, lse
