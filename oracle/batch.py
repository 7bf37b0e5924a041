"""Request classification and batch reorder -- oracle side.
TEST INFRASTRUCTURE ONLY.

"Beyond just running: native inference optimisation in vLLM on AMD ROCm":
* section "Every batch handles a mixed workload": prefill = a fresh prompt,
  extend = more prompt tokens on top of an already partly built KV cache,
  decode = one generated token at a time;
* section "ROCM_AITER_FA", batch reorder: the model runner reorders the
  requests to [decode:extend:prefill] before the three-way routing;
  reorder_batch_threshold = 1, i.e. a request with at most one query token is a
  decode;
* the iteration table of section "Interactive animation" walks requests
  through prefill -> extend -> decode under a token budget.

Reading: path = decode if query_len <= threshold, else extend if the request
already has cached context (ctx_len > 0), else prefill.  The reorder is stable
within each class (the page does not order requests inside a class).
"""
from __future__ import annotations

DECODE, EXTEND, PREFILL = 0, 1, 2
NAMES = {DECODE: "decode", EXTEND: "extend", PREFILL: "prefill"}


def classify(query_len: int, ctx_len: int, threshold: int = 1) -> int:
    if query_len <= threshold:
        return DECODE
    return EXTEND if ctx_len > 0 else PREFILL


def reorder(query_lens, ctx_lens, threshold: int = 1):
    """-> (perm, (n_decode, n_extend, n_prefill)); perm[i] is the original
    index of the request placed at position i."""
    cls = [classify(int(q), int(c), threshold) for q, c in zip(query_lens, ctx_lens)]
    perm = [i for k in (DECODE, EXTEND, PREFILL) for i, c in enumerate(cls) if c == k]
    counts = tuple(sum(1 for c in cls if c == k) for k in (DECODE, EXTEND, PREFILL))
    return perm, counts
