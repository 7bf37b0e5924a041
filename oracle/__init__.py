"""CPU oracle for paged KV-cache attention over mixed serving batches.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import, call or link anything under ``oracle/``; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
do.  The oracle shares no code with the HIP path: no kernels, no headers, no
table or constant generators, no pre- or post-processing.

Everything here is plain numpy in float64 (fp32 only where the method itself
fixes an fp32 decision: the fp8 quantisation step of the cache write).  Every
function cites the passage it follows, by page and section:

* "Beyond just running: native inference optimisation in vLLM on AMD ROCm"
  (vLLM blog, 2026-02-27; ROCm attention backends) -- sections "Every batch
  handles a mixed workload", "Unified attention backends" (two-stage forward),
  "ROCM_AITER_FA" (batch reorder, chunked context, preshuffled layout) and
  "Processing details of the three paths" (extend stages, LSE merge).
* "From LLM performance optimisation to DeepSeek deployment" (aif.amtbbs.org,
  2025-02-20) -- section 3 "Paged Attention" (block table) and section 5
  "Chunked Prefill".
* "Advanced inference: why your single-node vLLM setup needs prefill/decode
  disaggregation" (vLLM blog, 2026-04-07; MORI-IO KV connector) -- section
  "Architecture", write mode (layer-wise KV push into preallocated blocks).
* "vLLM disaggregated serving guide" (agentlenshq) -- section "Disaggregated
  architecture technical details" (KV bytes per token).

Modules
-------
fp8        OCP FP8 E4M3 (e4m3fn) codec from the format definition.
bf16       bfloat16 bit patterns -> float64.
cache      paged cache model: gather through the block table (both layouts),
           slot-mapped write, layer pack/unpack.
attention  exact softmax attention for the decode, prefill and extend paths.
merge      log-sum-exp merge of partial attention states.
batch      request classification and [decode:extend:prefill] reorder.
mla        absorbed multi-head latent attention decode over a paged 576-dim
           latent cache ("Beyond just running ...", section "AITER MLA
           backend: optimised for DeepSeek").

Parity status: every function above is pinned by ``tests/test_oracle_*.py``
(closed forms, invariants, library routines, brute force and the pages'
worked examples under ``tests/golden/``); none is "parity unpinned".
"""
