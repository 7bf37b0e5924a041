#!/usr/bin/env python3
"""Benchmark of the paged KV-cache attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  A step is one pass of the workload's whole hot path
over one batch of seeded synthetic input that is already resident in HBM:

  llama70b_decode_layer (default, the headline): Llama-3.1-70B-shaped decode
      layer -- batch 64, 64 query : 8 KV heads, head_dim 128, bf16 NHD cache,
      block 16, context lengths uniform in [2048, 8192], fully fragmented
      tables.  Step = kv_write of the 64 new tokens + paged_decode + packing
      all 5000 blocks of 8 requests x 10000 tokens (kv_pack_layer) + unpacking
      them into a receiving cache (kv_unpack_layer).
      value = algorithmic HBM bytes of the step / step time (GB/s).
  qwen3_mixed_batch: Qwen3-235B-A22B-shaped mixed batch reordered
      [decode:extend:prefill] -- 64:4 heads, 48 decodes (context [2000, 3000]),
      4 extends (512 new on 2000 cached), 2 prefills of 2000, all causal.
      Step = kv_write of all 6096 rows + paged_decode + extend_attn +
      prefill_attn.  value = query tokens / step time (tokens/s).
  fp8_preshuffled_decode: batch 128, 64:4 heads, fp8 e4m3 KV with per-tensor
      scales in the preshuffled layout (x = 16), context lengths uniform in
      [1000, 16000].  Step = kv_write (quantising) + paged_decode.
      value = algorithmic HBM bytes / step time (GB/s).
  long_context_extend: 2 x (100000 cached + 8192 new) tokens, 64:8 heads,
      32768-token chunk budget.  Step = kv_write + extend_attn.
      value = new tokens / step time (tokens/s).
  tiny_decode: batch 4, 8:2 heads, context [100, 512].  Step = kv_write +
      paged_decode (launch-bound; reported in us).
  decode_layout_compare: the Llama-3.1-70B decode layer's requests decoded
      from the NHD cache and from the same values in the bf16 preshuffled
      layout (x = 8).  Step = both decodes.
  heavy_tailed_mixed_batch: 64:4 heads, lognormal lengths (64 decodes, 12
      extends with many short and a few long new-token runs, 2 prefills).
      Step = kv_write + paged_decode + extend_attn + prefill_attn (three-way
      routing); the same batch as ONE extend_attn call over every request is
      timed beside it.
  deepseek_mla_decode: one GPU's share of DeepSeek-R1 MLA decode under TP8 --
      batch 128, 16 query heads, 576-dim bf16 latent rows, block 16, context
      [10000, 11000].  Step = mla_decode.
The default run measures the headline and then every other workload as a
"secondary" entry, each with its roofline and its CPU-oracle baseline.

Before the W warm-up steps of each workload, the step runs untimed for
SETTLE_S of wall time ("settle": steps and ms in the line): coming out of idle
the GPU needs some tens of milliseconds of sustained work to reach its steady
clocks, and W steps of a sub-millisecond step would time the ramp instead.

Per call, after the timed region: the average device time from HIP events
around the call alone ("ms"), and for decode calls also with the L2 and MALL
flushed before each call by a 512 MB read outside the event pair ("ms_cold",
HBM rather than cache).  device_ms_per_step is the sum of the calls' device
times, beside the host wall clock ms_per_step (their difference is launch and
host overhead between calls).

Roofline: the dominant call's algorithmic bytes (or flops) per launch divided
by its average duration, from HIP events recorded around it in every timed
step on the stream the library launches on.  traffic: HBM bytes per
call from rocprofv3 FETCH_SIZE / WRITE_SIZE counters, scaled by what the same
counters read for the pack kernel (a plain copy of known size), read from the
committed profile when it was taken on the current kernel sources, else null.
cpu_baseline: the CPU oracle timed on a bounded sample of the same workload
(for the decode layer and the tiny decode also with its BLAS on one thread,
"one_thread").
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
SETTLE_S = 0.25                # untimed sustained work before each workload's warm-up
ONE_THREAD_BASELINE = ("llama70b_decode_layer", "tiny_decode")   # oracle also timed on one thread
SETTLE_MAX_STEPS = 2000

METRIC = "paged decode HBM GB/s (% of 8 TB/s); mixed-batch attention tokens/s"


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


# Sources each roofline kernel is compiled from; a counter profile counts only
# while their hash matches the one recorded when the counters were taken.
KERNEL_SOURCES = {
    "paged_decode": ["paged_decode.hip", "common.h"],
    "prefill_attn": ["flash_attn.hip", "common.h"],
    "extend_attn": ["flash_attn.hip", "common.h"],
    "mla_decode": ["mla_decode.hip", "common.h"],
}


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "paged_kv_cache_mapped_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(kernel, workload):
    """HBM bytes per call of `kernel` from the committed counter profile, or
    None when there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- `"):
            k, v = line[3:].split("`", 1)
            fields[k] = v.split(":", 1)[1].strip().strip("`")
    try:
        if fields["source_sha256"] != source_hash(kernel):
            return None
        return float(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def cpu_info():
    """Host CPU model, logical CPU count and the BLAS thread count the oracle
    runs with (numpy's matmul is its only multi-threaded part)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return {"cpu_model": model, "os_cpu_count": os.cpu_count() or 1, "blas_threads": int(blas)}


class HipEvents:
    """Timing events recorded straight through the HIP runtime that torch has
    loaded, created with hipEventDisableSystemFence: a default event record
    ends with a system-scope release (a writeback and invalidate of the GPU
    caches), which costs several microseconds per marker and stalls the next
    kernel.  The timestamps are taken the same way."""

    FLAG = 0x20000000                     # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.events = []

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def new(self):
        ev = self.ct.c_void_p()
        self._ok(self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.ct.c_uint(self.FLAG)),
                 "hipEventCreateWithFlags")
        self.events.append(ev)
        return ev

    def record(self, ev, stream):
        self._ok(self.hip.hipEventRecord(ev, self.ct.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def ms(self, a, b):
        out = self.ct.c_float()
        self._ok(self.hip.hipEventElapsedTime(self.ct.byref(out), a, b), "hipEventElapsedTime")
        return float(out.value)

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


# ----------------------------------------------------------------------------- workloads
class Call:
    """One library call of the step with its algorithmic cost per launch."""

    def __init__(self, name, fn, bytes_=0.0, flops=0.0):
        self.name, self.fn, self.bytes, self.flops = name, fn, float(bytes_), float(flops)


def build_llama70b_decode_layer(torch, pk, w, dev):
    st = w.llama70b_decode_layer()
    job = w.pack_job(2, st.cache.spec.num_blocks)
    sp = st.cache.spec
    dc = pk.PagedKVCache(dev(st.cache.k), dev(st.cache.v), sp.block_size, sp.num_kv_heads,
                         sp.head_dim)
    recv = pk.PagedKVCache(torch.zeros_like(dc.k), torch.zeros_like(dc.v), sp.block_size,
                           sp.num_kv_heads, sp.head_dim)
    q, kn, vn = dev(st.q), dev(st.k_new), dev(st.v_new)
    slots, tables, lens = dev(st.slot_mapping), dev(st.block_tables), dev(st.seq_lens)
    msl = int(st.seq_lens.max())
    B, Hq, D, Hkv = st.batch, st.num_q_heads, sp.head_dim, sp.num_kv_heads
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(pk.paged_decode_workspace_bytes(dc, B, Hq, msl), 16), dtype=torch.uint8,
                     device=q.device)
    src_ids, dst_ids = dev(job.src_ids), dev(job.dst_ids)
    n = int(job.src_ids.size)
    buf = torch.empty(pk.kv_layer_packed_bytes(dc, n), dtype=torch.uint8, device=q.device)

    row = Hkv * D * 2
    write_bytes = B * (2 * row * 2 + 8)
    kv_bytes = float(st.seq_lens.astype(np.int64).sum()) * row * 2
    blocks = float(((st.seq_lens + 15) // 16).sum())
    decode_bytes = kv_bytes + 2 * B * Hq * D * 2 + B * Hq * 4 + blocks * 4 + B * 4
    decode_flops = float(st.seq_lens.astype(np.int64).sum()) * Hq * 4 * D
    pack_bytes = 2.0 * buf.numel() + n * 4

    calls = [
        Call("kv_write", lambda: pk.kv_write(dc, kn, vn, slots), write_bytes),
        Call("paged_decode", lambda: pk.paged_decode(dc, q, tables, lens, msl, st.scale, out=out,
                                                     lse=lse, workspace=ws),
             decode_bytes, decode_flops),
        Call("kv_pack_layer", lambda: pk.kv_pack_layer(dc, src_ids, buf), pack_bytes),
        Call("kv_unpack_layer", lambda: pk.kv_unpack_layer(recv, dst_ids, buf), pack_bytes),
    ]
    config = {
        "workload": "llama-3.1-70b decode layer: batch 64, 64:8 heads, head_dim 128, bf16 NHD "
                    "cache, block 16, ctx U[2048,8192]; + pack/unpack of 5000 blocks "
                    "(8 req x 10000 tokens, 327.68 MB)",
        "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": 16,
        "kv_tokens": int(st.seq_lens.sum()), "pack_blocks": n,
    }

    def cpu_sample(budget_s):
        from oracle import attention as oa, bf16 as ob, cache as oc
        ocache = oc.Cache(st.cache.k, st.cache.v, "nhd", "bf16", 16, Hkv, D)
        qf = ob.to_f64(st.q)
        done_bytes, t0, nreq = 0.0, time.perf_counter(), 0
        while time.perf_counter() - t0 < budget_s * 0.8:      # cycles over the batch
            b = nreq % B
            oa.paged_decode(qf[b:b + 1], ocache, st.block_tables[b:b + 1], st.seq_lens[b:b + 1],
                            st.scale)
            done_bytes += float(st.seq_lens[b]) * row * 2 + 2 * Hq * D * 2
            nreq += 1
        m, npk = 500, 0
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < budget_s * 0.2:
            buf_h = oc.pack_layer(ocache, job.src_ids[:m])
            oc.unpack_layer(ocache, job.dst_ids[:m], buf_h)
            done_bytes += 4.0 * buf_h.size
            npk += 1
        t2 = time.perf_counter()
        return done_bytes / (t2 - t0) / 1e9, (
            f"oracle decode of {nreq} requests of this batch (all 64 heads) + {npk} pack/unpack "
            f"round trips of {m} of the {n} blocks; {t2 - t0:.1f} s")

    return calls, "paged_decode", "hbm", config, cpu_sample, ("GB/s", None)


def build_qwen3_mixed_batch(torch, pk, w, dev):
    mb = w.qwen3_mixed_batch()
    sp = mb.cache.spec
    dc = pk.PagedKVCache(dev(mb.cache.k), dev(mb.cache.v), sp.block_size, sp.num_kv_heads,
                         sp.head_dim)
    q, kn, vn, slots = dev(mb.q), dev(mb.k_new), dev(mb.v_new), dev(mb.slot_mapping)
    d0, d1 = mb.rows_decode
    e0, e1 = mb.rows_extend
    p0, p1 = mb.rows_prefill
    Hq, Hkv, D = mb.num_q_heads, sp.num_kv_heads, sp.head_dim
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], Hq), dtype=torch.float32, device=q.device)
    dtab, dlen = dev(mb.dec_tables), dev(mb.dec_seq_lens)
    dmsl = int(mb.dec_seq_lens.max())
    dws = torch.empty(max(pk.paged_decode_workspace_bytes(dc, d1 - d0, Hq, dmsl), 16),
                      dtype=torch.uint8, device=q.device)
    ecu, ectx, etab = dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables)
    E = int(mb.ext_ctx.size)
    emq = int(np.diff(mb.ext_cu_q).max())
    emc = int(mb.ext_ctx.max())
    ews = torch.empty(max(pk.extend_attn_workspace_bytes(dc, E, e1 - e0, Hq, emc, 32768), 16),
                      dtype=torch.uint8, device=q.device)
    pcu = dev(mb.pre_cu)
    pmax = int(np.diff(mb.pre_cu).max())
    T = int(q.shape[0])

    row = Hkv * D * 2
    dec_bytes = float(mb.dec_seq_lens.astype(np.int64).sum()) * row * 2
    ext_pairs = sum(int(n) * int(c) + int(n) * (int(n) + 1) // 2
                    for n, c in zip(np.diff(mb.ext_cu_q), mb.ext_ctx))
    pre_pairs = sum(int(n) * (int(n) + 1) // 2 for n in np.diff(mb.pre_cu))

    calls = [
        Call("kv_write", lambda: pk.kv_write(dc, kn, vn, slots), T * (4 * row + 8)),
        Call("paged_decode", lambda: pk.paged_decode(dc, q[d0:d1], dtab, dlen, dmsl, mb.scale,
                                                     out=out[d0:d1], lse=lse[d0:d1], workspace=dws),
             dec_bytes),
        Call("extend_attn", lambda: pk.extend_attn(dc, q[e0:e1], kn[e0:e1], vn[e0:e1], ecu, ectx,
                                                   etab, emq, emc, mb.scale, 32768, out=out[e0:e1],
                                                   lse=lse[e0:e1], workspace=ews),
             0.0, float(ext_pairs) * Hq * 4 * D),
        Call("prefill_attn", lambda: pk.prefill_attn(q[p0:p1], kn[p0:p1], vn[p0:p1], pcu, pmax,
                                                     mb.scale, True, out=out[p0:p1], lse=lse[p0:p1]),
             0.0, float(pre_pairs) * Hq * 4 * D),
    ]
    config = {
        "workload": "qwen3-235b-a22b mixed batch [decode:extend:prefill]: 64:4 heads, head_dim 128, "
                    "bf16 NHD, block 16; 48 decodes ctx U[2000,3000], 4 extends 512 new on 2000 "
                    "cached, 2 prefills of 2000; 6096 query tokens",
        "query_tokens": T, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
    }

    def cpu_sample(budget_s):
        from oracle import attention as oa, bf16 as ob, cache as oc
        ocache = oc.write(oc.Cache(mb.cache.k, mb.cache.v, "nhd", "bf16", 16, Hkv, D),
                          mb.k_new, mb.v_new, mb.slot_mapping)
        qf = ob.to_f64(mb.q)
        kf, vf = ob.to_f64(mb.k_new), ob.to_f64(mb.v_new)
        t0 = time.perf_counter()
        nd = npf = 0
        while time.perf_counter() - t0 < budget_s:     # decode rows and prefill rows alternately
            b = nd % (d1 - d0)
            oa.paged_decode(qf[b:b + 1], ocache, mb.dec_tables[b:b + 1], mb.dec_seq_lens[b:b + 1],
                            mb.scale)
            nd += 1
            r = (npf * 97) % (p1 - p0)
            oa.prefill(qf[p0:p1], kf[p0:p1], vf[p0:p1], mb.pre_cu, mb.scale, rows=[r])
            npf += 1
        t2 = time.perf_counter()
        return (nd + npf) / (t2 - t0), (f"oracle decode of {nd} decode rows + {npf} prefill rows "
                                        f"of this batch (all 64 heads); {t2 - t0:.1f} s")

    return calls, "prefill_attn", "mfma", config, cpu_sample, ("tokens/s", T)


def build_long_context_extend(torch, pk, w, dev):
    mb = w.long_context_extend()
    sp = mb.cache.spec
    dc = pk.PagedKVCache(dev(mb.cache.k), dev(mb.cache.v), sp.block_size, sp.num_kv_heads,
                         sp.head_dim)
    q, kn, vn, slots = dev(mb.q), dev(mb.k_new), dev(mb.v_new), dev(mb.slot_mapping)
    Hq, Hkv, D = mb.num_q_heads, sp.num_kv_heads, sp.head_dim
    T = int(q.shape[0])
    E = int(mb.ext_ctx.size)
    emq, emc = int(np.diff(mb.ext_cu_q).max()), int(mb.ext_ctx.max())
    ws = torch.empty(max(pk.extend_attn_workspace_bytes(dc, E, T, Hq, emc, 32768), 16),
                     dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    ecu, ectx, etab = dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables)
    pairs = sum(int(n) * int(c) + int(n) * (int(n) + 1) // 2
                for n, c in zip(np.diff(mb.ext_cu_q), mb.ext_ctx))
    calls = [
        Call("kv_write", lambda: pk.kv_write(dc, kn, vn, slots), T * (4 * Hkv * D * 2 + 8)),
        Call("extend_attn", lambda: pk.extend_attn(dc, q, kn, vn, ecu, ectx, etab, emq, emc,
                                                   mb.scale, 32768, out=out, lse=lse, workspace=ws),
             0.0, float(pairs) * Hq * 4 * D),
    ]
    config = {"workload": "long-context extend: 2 requests x (100000 cached + 8192 new), 64:8 heads, "
                          "head_dim 128, bf16 NHD, block 16, 32768-token chunk budget",
              "query_tokens": T}

    def cpu_sample(budget_s):
        from oracle import attention as oa, bf16 as ob, cache as oc
        ocache = oc.Cache(mb.cache.k, mb.cache.v, "nhd", "bf16", 16, Hkv, D)
        qf, kf, vf = ob.to_f64(mb.q), ob.to_f64(mb.k_new), ob.to_f64(mb.v_new)
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < budget_s:
            oa.extend(qf, kf, vf, mb.ext_cu_q, mb.ext_ctx, ocache, mb.ext_tables, mb.scale,
                      rows=[(n * 997) % T])
            n += 1
        return n / (time.perf_counter() - t0), f"oracle extend of {n} rows (all 64 heads)"

    return calls, "extend_attn", "mfma", config, cpu_sample, ("tokens/s", T)


def build_fp8_preshuffled_decode(torch, pk, w, dev):
    st = w.fp8_preshuffled_decode()
    sp = st.cache.spec
    dc = pk.PagedKVCache(dev(st.cache.k), dev(st.cache.v), sp.block_size, sp.num_kv_heads,
                         sp.head_dim, sp.layout, sp.dtype, st.cache.k_scale, st.cache.v_scale)
    q, kn, vn = dev(st.q), dev(st.k_new), dev(st.v_new)
    slots, tables, lens = dev(st.slot_mapping), dev(st.block_tables), dev(st.seq_lens)
    msl = int(st.seq_lens.max())
    B, Hq, D, Hkv = st.batch, st.num_q_heads, sp.head_dim, sp.num_kv_heads
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(pk.paged_decode_workspace_bytes(dc, B, Hq, msl), 16), dtype=torch.uint8,
                     device=q.device)
    row = Hkv * D                                         # fp8: one byte per element
    write_bytes = B * (2 * Hkv * D * 2 + 2 * row + 8)
    kv_bytes = float(st.seq_lens.astype(np.int64).sum()) * row * 2
    blocks = float(((st.seq_lens + 15) // 16).sum())
    decode_bytes = kv_bytes + 2 * B * Hq * D * 2 + B * Hq * 4 + blocks * 4 + B * 4
    decode_flops = float(st.seq_lens.astype(np.int64).sum()) * Hq * 4 * D
    calls = [
        Call("kv_write", lambda: pk.kv_write(dc, kn, vn, slots), write_bytes),
        Call("paged_decode", lambda: pk.paged_decode(dc, q, tables, lens, msl, st.scale, out=out,
                                                     lse=lse, workspace=ws),
             decode_bytes, decode_flops),
    ]
    config = {
        "workload": "fp8 e4m3 preshuffled decode: batch 128, 64:4 heads, head_dim 128, block 16, "
                    "x 16, ctx U[1000,16000], per-tensor scales, q/out bf16",
        "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": 16,
        "kv_tokens": int(st.seq_lens.sum()),
    }

    def cpu_sample(budget_s):
        from oracle import attention as oa, bf16 as ob, cache as oc
        ocache = oc.Cache(st.cache.k, st.cache.v, "preshuffled", "fp8", 16, Hkv, D, 16,
                          st.cache.k_scale, st.cache.v_scale)
        qf = ob.to_f64(st.q)
        done, t0, nreq = 0.0, time.perf_counter(), 0
        while time.perf_counter() - t0 < budget_s:
            b = nreq % B
            oa.paged_decode(qf[b:b + 1], ocache, st.block_tables[b:b + 1], st.seq_lens[b:b + 1],
                            st.scale)
            done += float(st.seq_lens[b]) * row * 2 + 2 * Hq * D * 2
            nreq += 1
        t1 = time.perf_counter()
        return done / (t1 - t0) / 1e9, f"oracle decode of {nreq} requests of this batch; {t1 - t0:.1f} s"

    return calls, "paged_decode", "hbm", config, cpu_sample, ("GB/s", None)


def build_tiny_decode(torch, pk, w, dev):
    st = w.tiny_decode()
    sp = st.cache.spec
    dc = pk.PagedKVCache(dev(st.cache.k), dev(st.cache.v), sp.block_size, sp.num_kv_heads,
                         sp.head_dim)
    q, kn, vn = dev(st.q), dev(st.k_new), dev(st.v_new)
    slots, tables, lens = dev(st.slot_mapping), dev(st.block_tables), dev(st.seq_lens)
    msl = int(st.seq_lens.max())
    B, Hq, D, Hkv = st.batch, st.num_q_heads, sp.head_dim, sp.num_kv_heads
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(pk.paged_decode_workspace_bytes(dc, B, Hq, msl), 16), dtype=torch.uint8,
                     device=q.device)
    row = Hkv * D * 2
    kv_bytes = float(st.seq_lens.astype(np.int64).sum()) * row * 2
    blocks = float(((st.seq_lens + 15) // 16).sum())
    decode_bytes = kv_bytes + 2 * B * Hq * D * 2 + B * Hq * 4 + blocks * 4 + B * 4
    calls = [
        Call("kv_write", lambda: pk.kv_write(dc, kn, vn, slots), B * (2 * row * 2 + 8)),
        Call("paged_decode", lambda: pk.paged_decode(dc, q, tables, lens, msl, st.scale, out=out,
                                                     lse=lse, workspace=ws), decode_bytes),
    ]
    config = {"workload": "tiny decode: batch 4, 8:2 heads, head_dim 128, bf16 NHD, block 16, "
                          "256 blocks, ctx U[100,512]; one write + decode step (launch-bound)",
              "batch": B, "kv_tokens": int(st.seq_lens.sum())}

    def cpu_sample(budget_s):
        from oracle import attention as oa, bf16 as ob, cache as oc
        ocache = oc.Cache(st.cache.k, st.cache.v, "nhd", "bf16", 16, Hkv, D)
        qf = ob.to_f64(st.q)
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < budget_s:
            oc.write(ocache, st.k_new, st.v_new, st.slot_mapping)
            oa.paged_decode(qf, ocache, st.block_tables, st.seq_lens, st.scale)
            n += 1
        dt = time.perf_counter() - t0
        return n * kv_bytes / dt / 1e9, f"{n} oracle write + decode steps of the whole batch; {dt:.1f} s"

    return calls, "paged_decode", "hbm", config, cpu_sample, ("GB/s", None)


def build_decode_layout_compare(torch, pk, w, dev):
    """The decode layer's requests from two caches holding the same values:
    NHD, and the bf16 preshuffled layout (x = 8) made from it by a permute."""
    st = w.llama70b_decode_layer()
    sp = st.cache.spec
    nb, bs, Hkv, D = sp.num_blocks, sp.block_size, sp.num_kv_heads, sp.head_dim
    k_nhd, v_nhd = dev(st.cache.k), dev(st.cache.v)
    X = 8
    # k[b, h, d // X, t, d % X] = K[b, t, h, d];  v[b, h, t // X, d, t % X] = V[b, t, h, d]
    k_pre = k_nhd.view(nb, bs, Hkv, D // X, X).permute(0, 2, 3, 1, 4).contiguous()
    v_pre = v_nhd.view(nb, bs // X, X, Hkv, D).permute(0, 3, 1, 4, 2).contiguous()
    nhd = pk.PagedKVCache(k_nhd, v_nhd, bs, Hkv, D)
    pre = pk.PagedKVCache(k_pre, v_pre, bs, Hkv, D, "preshuffled", "bf16")
    q, tables, lens = dev(st.q), dev(st.block_tables), dev(st.seq_lens)
    msl = int(st.seq_lens.max())
    B, Hq = st.batch, st.num_q_heads
    out_n, out_p = torch.empty_like(q), torch.empty_like(q)
    lse_n = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    lse_p = torch.empty_like(lse_n)
    wsn = torch.empty(max(pk.paged_decode_workspace_bytes(nhd, B, Hq, msl), 16), dtype=torch.uint8,
                      device=q.device)
    wsp = torch.empty_like(wsn)
    row = Hkv * D * 2
    kv_bytes = float(st.seq_lens.astype(np.int64).sum()) * row * 2
    blocks = float(((st.seq_lens + 15) // 16).sum())
    decode_bytes = kv_bytes + 2 * B * Hq * D * 2 + B * Hq * 4 + blocks * 4 + B * 4
    calls = [
        Call("paged_decode_nhd", lambda: pk.paged_decode(nhd, q, tables, lens, msl, st.scale,
                                                         out=out_n, lse=lse_n, workspace=wsn),
             decode_bytes),
        Call("paged_decode_preshuffled", lambda: pk.paged_decode(pre, q, tables, lens, msl,
                                                                 st.scale, out=out_p, lse=lse_p,
                                                                 workspace=wsp),
             decode_bytes),
    ]
    config = {"workload": "llama-3.1-70b decode layer (batch 64, 64:8, ctx U[2048,8192], block 16) "
                          "decoded from the bf16 NHD cache and from the same values in the bf16 "
                          "preshuffled layout (x 8)",
              "batch": B, "kv_tokens": int(st.seq_lens.sum())}

    def cpu_sample(budget_s):
        from oracle import attention as oa, bf16 as ob, cache as oc
        ocache = oc.Cache(st.cache.k, st.cache.v, "nhd", "bf16", 16, Hkv, D)
        qf = ob.to_f64(st.q)
        t0, done, n = time.perf_counter(), 0.0, 0
        while time.perf_counter() - t0 < budget_s:
            b = n % B
            oa.paged_decode(qf[b:b + 1], ocache, st.block_tables[b:b + 1], st.seq_lens[b:b + 1],
                            st.scale)
            done += float(st.seq_lens[b]) * row * 2
            n += 1
        dt = time.perf_counter() - t0
        return done / dt / 1e9, f"oracle decode of {n} requests of this batch (NHD); {dt:.1f} s"

    return calls, "paged_decode_preshuffled", "hbm", config, cpu_sample, ("GB/s", None)


def unified_batch_args(mb):
    """The whole reordered batch as ONE extend call (the single-kernel
    alternative to three-way routing): a decode is an extend of 1 new token on
    L - 1 cached tokens, a prefill an extend with no cached context."""
    nd = mb.n_decode
    qlens = np.concatenate([np.ones(nd, np.int64), np.diff(mb.ext_cu_q), np.diff(mb.pre_cu)])
    ctx = np.concatenate([mb.dec_seq_lens - 1, mb.ext_ctx,
                          np.zeros(len(mb.pre_cu) - 1, np.int64)]).astype(np.int32)
    width = max(mb.dec_tables.shape[1] if nd else 1, mb.ext_tables.shape[1])
    tables = np.full((len(qlens), width), mb.cache.poison_block, np.int32)
    if nd:
        tables[:nd, :mb.dec_tables.shape[1]] = mb.dec_tables
    ne = len(mb.ext_ctx)
    tables[nd:nd + ne, :mb.ext_tables.shape[1]] = mb.ext_tables
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return cu, ctx, tables, int(qlens.max()), int(ctx.max())


def build_heavy_tailed_mixed_batch(torch, pk, w, dev):
    mb = w.heavy_tailed_mixed_batch()
    sp = mb.cache.spec
    dc = pk.PagedKVCache(dev(mb.cache.k), dev(mb.cache.v), sp.block_size, sp.num_kv_heads,
                         sp.head_dim)
    q, kn, vn, slots = dev(mb.q), dev(mb.k_new), dev(mb.v_new), dev(mb.slot_mapping)
    d0, d1 = mb.rows_decode
    e0, e1 = mb.rows_extend
    p0, p1 = mb.rows_prefill
    Hq, Hkv, D = mb.num_q_heads, sp.num_kv_heads, sp.head_dim
    T = int(q.shape[0])
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    dtab, dlen = dev(mb.dec_tables), dev(mb.dec_seq_lens)
    dmsl = int(mb.dec_seq_lens.max())
    dws = torch.empty(max(pk.paged_decode_workspace_bytes(dc, d1 - d0, Hq, dmsl), 16),
                      dtype=torch.uint8, device=q.device)
    ecu, ectx, etab = dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables)
    E = int(mb.ext_ctx.size)
    emq, emc = int(np.diff(mb.ext_cu_q).max()), int(mb.ext_ctx.max())
    ews = torch.empty(max(pk.extend_attn_workspace_bytes(dc, E, e1 - e0, Hq, emc, 32768), 16),
                      dtype=torch.uint8, device=q.device)
    pcu = dev(mb.pre_cu)
    pmax = int(np.diff(mb.pre_cu).max())
    ucu, uctx, utab, umq, umc = unified_batch_args(mb)
    ucu_d, uctx_d, utab_d = dev(ucu), dev(uctx), dev(utab)
    uout = torch.empty_like(q)
    ulse = torch.empty_like(lse)
    uws = torch.empty(max(pk.extend_attn_workspace_bytes(dc, len(uctx), T, Hq, umc, 32768), 16),
                      dtype=torch.uint8, device=q.device)

    row = Hkv * D * 2
    dec_bytes = float(mb.dec_seq_lens.astype(np.int64).sum()) * row * 2
    ext_pairs = sum(int(n) * int(c) + int(n) * (int(n) + 1) // 2
                    for n, c in zip(np.diff(mb.ext_cu_q), mb.ext_ctx))
    pre_pairs = sum(int(n) * (int(n) + 1) // 2 for n in np.diff(mb.pre_cu))
    dec_pairs = int(mb.dec_seq_lens.astype(np.int64).sum())
    calls = [
        Call("kv_write", lambda: pk.kv_write(dc, kn, vn, slots), T * (4 * row + 8)),
        Call("paged_decode", lambda: pk.paged_decode(dc, q[d0:d1], dtab, dlen, dmsl, mb.scale,
                                                     out=out[d0:d1], lse=lse[d0:d1], workspace=dws),
             dec_bytes),
        Call("extend_attn", lambda: pk.extend_attn(dc, q[e0:e1], kn[e0:e1], vn[e0:e1], ecu, ectx,
                                                   etab, emq, emc, mb.scale, 32768, out=out[e0:e1],
                                                   lse=lse[e0:e1], workspace=ews),
             0.0, float(ext_pairs) * Hq * 4 * D),
        Call("prefill_attn", lambda: pk.prefill_attn(q[p0:p1], kn[p0:p1], vn[p0:p1], pcu, pmax,
                                                     mb.scale, True, out=out[p0:p1], lse=lse[p0:p1]),
             0.0, float(pre_pairs) * Hq * 4 * D),
    ]
    # the same batch through one extend call over every request (not part of
    # the step; timed per call for the comparison)
    unified = Call("unified_extend_attn", lambda: pk.extend_attn(
        dc, q, kn, vn, ucu_d, uctx_d, utab_d, umq, umc, mb.scale, 32768, out=uout, lse=ulse,
        workspace=uws), 0.0, float(ext_pairs + pre_pairs + dec_pairs) * Hq * 4 * D)
    config = {
        "workload": "heavy-tailed mixed batch [decode:extend:prefill]: 64:4 heads, head_dim 128, "
                    "bf16 NHD, block 16; lognormal lengths: 64 decodes (ctx median 2000), "
                    "12 extends (new median 96, ctx median 3000), 2 prefills (median 1500)",
        "query_tokens": T, "decode_ctx": mb.dec_seq_lens.tolist(),
        "extend_new": np.diff(mb.ext_cu_q).tolist(), "extend_ctx": mb.ext_ctx.tolist(),
        "prefill_len": np.diff(mb.pre_cu).tolist(),
    }

    def cpu_sample(budget_s):
        from oracle import attention as oa, bf16 as ob, cache as oc
        ocache = oc.write(oc.Cache(mb.cache.k, mb.cache.v, "nhd", "bf16", 16, Hkv, D),
                          mb.k_new, mb.v_new, mb.slot_mapping)
        qf, kf, vf = ob.to_f64(mb.q), ob.to_f64(mb.k_new), ob.to_f64(mb.v_new)
        t0, n = time.perf_counter(), 0
        rng = np.random.default_rng(0)
        while time.perf_counter() - t0 < budget_s:     # random rows of the batch
            r = int(rng.integers(0, T))
            if r < d1:
                oa.paged_decode(qf[r:r + 1], ocache, mb.dec_tables[r:r + 1],
                                mb.dec_seq_lens[r:r + 1], mb.scale)
            elif r < e1:
                oa.extend(qf[e0:e1], kf[e0:e1], vf[e0:e1], mb.ext_cu_q, mb.ext_ctx, ocache,
                          mb.ext_tables, mb.scale, rows=[r - e0])
            else:
                oa.prefill(qf[p0:p1], kf[p0:p1], vf[p0:p1], mb.pre_cu, mb.scale, rows=[r - p0])
            n += 1
        dt = time.perf_counter() - t0
        return n / dt, f"oracle rows of {n} random query tokens of this batch (all 64 heads); {dt:.1f} s"

    return calls, "extend_attn", "mfma", config, cpu_sample, ("tokens/s", T), [unified]


def build_deepseek_mla_decode(torch, pk, w, dev):
    st = w.deepseek_mla_decode()
    cache, q = dev(st.cache), dev(st.q)
    tables, lens = dev(st.block_tables), dev(st.seq_lens)
    msl = int(st.seq_lens.max())
    B, H = st.batch, st.num_heads
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(int(pk.lib().mla_decode_workspace_bytes(B, H, msl)), 16),
                     dtype=torch.uint8, device=q.device)
    tok = float(st.seq_lens.astype(np.int64).sum())
    blocks = float(((st.seq_lens + 15) // 16).sum())
    mla_bytes = tok * 576 * 2 + B * H * (576 + 512) * 2 + B * H * 4 + blocks * 4 + B * 4
    mla_flops = tok * H * 2 * (576 + 512)
    calls = [Call("mla_decode", lambda: pk.mla_decode(cache, q, tables, lens, msl, st.scale,
                                                      out=out, lse=lse, workspace=ws),
                  mla_bytes, mla_flops)]
    config = {"workload": "deepseek-r1 MLA absorbed decode, one GPU's share under TP8: batch 128, "
                          "16 query heads, 576-dim bf16 latent rows (value = first 512), block 16, "
                          "ctx U[10000,11000]",
              "batch": B, "num_heads": H, "kv_tokens": int(tok)}

    def cpu_sample(budget_s):
        from oracle import bf16 as ob, mla
        qf = ob.to_f64(st.q)
        t0, done, n = time.perf_counter(), 0.0, 0
        while time.perf_counter() - t0 < budget_s:
            b = n % B
            mla.mla_decode(qf[b:b + 1], st.cache, st.block_tables[b:b + 1], st.seq_lens[b:b + 1],
                           st.scale, 16)
            done += float(st.seq_lens[b]) * 576 * 2
            n += 1
        dt = time.perf_counter() - t0
        return done / dt / 1e9, f"oracle MLA decode of {n} requests of this batch; {dt:.1f} s"

    return calls, "mla_decode", "hbm", config, cpu_sample, ("GB/s", None)


WORKLOADS = {
    "llama70b_decode_layer": build_llama70b_decode_layer,
    "qwen3_mixed_batch": build_qwen3_mixed_batch,
    "fp8_preshuffled_decode": build_fp8_preshuffled_decode,
    "long_context_extend": build_long_context_extend,
    "tiny_decode": build_tiny_decode,
    "decode_layout_compare": build_decode_layout_compare,
    "heavy_tailed_mixed_batch": build_heavy_tailed_mixed_batch,
    "deepseek_mla_decode": build_deepseek_mla_decode,
}
SECONDARY_METRIC = {
    "qwen3_mixed_batch": "mixed-batch attention tokens/s",
    "fp8_preshuffled_decode": "paged decode HBM GB/s (fp8 preshuffled cache)",
    "long_context_extend": "long-context extend tokens/s (chunked context, LSE merge)",
    "tiny_decode": "paged decode HBM GB/s (tiny, launch-bound)",
    "decode_layout_compare": "paged decode HBM GB/s, bf16 preshuffled vs NHD layout",
    "heavy_tailed_mixed_batch": "mixed-batch attention tokens/s, heavy-tailed lengths, "
                                "three-way routed vs one unified extend call",
    "deepseek_mla_decode": "MLA absorbed decode HBM GB/s (576-dim latent cache)",
}


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama70b_decode_layer", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work per workload for cpu_baseline")
    ap.add_argument("--no-secondary", action="store_true",
                    help="measure only the chosen workload")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build runs its whole hot path on a single "
              "MI355X (no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_mapped_amd as pk
    from synth import workloads as w

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pk.lib()
    # 512 MB read before each "cold" call: it replaces the L2 and MALL contents
    # with clean lines (a fill would leave dirty lines whose write-back then
    # lands inside the timed call)
    flush_buf = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    flush_sink = torch.zeros(1, dtype=torch.float32, device="cuda")

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def measure(name, with_cpu):
        _log(f"building workload {name}")
        built = WORKLOADS[name](torch, pk, w, dev)
        calls, dominant, bound, config, cpu_sample, (unit, tokens) = built[:6]
        extra = built[6] if len(built) > 6 else []     # timed per call only, not in the step
        torch.cuda.synchronize()

        def step():
            for c in calls:
                c.fn()

        # Clock settle: the GPU comes to each workload out of idle (the batch
        # was just built on the host) at reduced clocks, and its step time
        # keeps falling over the first tens of milliseconds of sustained work
        # (3-13 % on these workloads).  The step is repeated, untimed, for
        # SETTLE_S of wall time (at most SETTLE_MAX_STEPS), then the W
        # warm-up steps run as asked.
        settle_steps, t_settle = 0, time.perf_counter()
        while (time.perf_counter() - t_settle < SETTLE_S and settle_steps < SETTLE_MAX_STEPS):
            for _ in range(4):
                step()
            settle_steps += 4
            torch.cuda.synchronize()
        settle_ms = (time.perf_counter() - t_settle) * 1e3
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        _log(f"timing {args.steps} steps of {name} (after {settle_steps} settle steps, "
             f"{settle_ms:.0f} ms)")
        # HIP events on the stream the library launches on, around the dominant
        # call of every timed step (events between every pair of calls would add
        # a marker packet each to the step)
        stream = torch.cuda.current_stream()
        hev = HipEvents()
        ev = [(hev.new(), hev.new()) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            for c in calls:
                if c.name == dominant:
                    hev.record(ev[s][0], stream)
                    c.fn()
                    hev.record(ev[s][1], stream)
                else:
                    c.fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / max(args.steps, 1)
        dom_ms = sum(hev.ms(a, b) for a, b in ev) / max(len(ev), 1)

        def timed(c, cold):
            evs = [(hev.new(), hev.new()) for _ in range(args.steps)]
            for a, b in evs:
                if cold:
                    torch.sum(flush_buf, dim=0, keepdim=True, out=flush_sink)   # outside the events
                hev.record(a, stream)
                c.fn()
                hev.record(b, stream)
            torch.cuda.synchronize()
            return sum(hev.ms(a, b) for a, b in evs) / max(len(evs), 1)

        # every call's own duration, from events around it, after the timed region
        per = {}
        for c in calls:
            avg = dom_ms if c.name == dominant else timed(c, False)
            d = {"ms": round(avg, 5)}
            if c.bytes:
                d["GB/s"] = round(c.bytes / (avg * 1e-3) / 1e9, 1)
                d["hbm_frac"] = round(d["GB/s"] / HBM_PEAK_GBS, 4)
            if c.flops:
                d["TFLOP/s"] = round(c.flops / (avg * 1e-3) / 1e12, 1)
                d["mfma_frac"] = round(d["TFLOP/s"] / BF16_PEAK_TFLOPS, 4)
            if c.name.startswith("paged_decode") or c.name == "mla_decode":
                cold = timed(c, True)
                d["ms_cold"] = round(cold, 5)
                d["GB/s_cold"] = round(c.bytes / (cold * 1e-3) / 1e9, 1)
                d["hbm_frac_cold"] = round(d["GB/s_cold"] / HBM_PEAK_GBS, 4)
            per[c.name] = d
        device_ms = sum(per[c.name]["ms"] for c in calls)
        for c in extra:
            c.fn()
            torch.cuda.synchronize()
            avg = timed(c, False)
            d = {"ms": round(avg, 5), "not_in_step": True}
            if c.flops:
                d["TFLOP/s"] = round(c.flops / (avg * 1e-3) / 1e12, 1)
                d["mfma_frac"] = round(d["TFLOP/s"] / BF16_PEAK_TFLOPS, 4)
            per[c.name] = d

        dom = next(c for c in calls if c.name == dominant)
        dms = dom_ms
        if bound == "hbm":
            ach = dom.bytes / (dms * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": dominant, "achieved": round(ach, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": counter_traffic(dominant.split("_nhd")[0].split("_preshuffled")[0],
                                               name)}
        else:
            ach = dom.flops / (dms * 1e-3) / 1e12
            roof = {"bound": "mfma", "kernel": dominant, "achieved": round(ach, 1),
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                    "traffic": counter_traffic(dominant, name)}
        if unit == "GB/s":
            value = sum(c.bytes for c in calls) / (ms * 1e-3) / 1e9
        else:
            value = tokens / (ms * 1e-3)
        cpu = None
        if with_cpu:
            _log(f"timing the CPU oracle on a sample of {name}")
            info = cpu_info()
            v, sample = cpu_sample(args.cpu_budget)
            cpu = {"value": round(v, 4), "unit": unit, "cores": info["blas_threads"],
                   "kind": "oracle", "sample": sample, "precision": "float64",
                   "cpu_model": info["cpu_model"], "os_cpu_count": info["os_cpu_count"]}
            if name in ONE_THREAD_BASELINE:
                # the same oracle with its BLAS limited to one thread
                try:
                    from threadpoolctl import threadpool_limits
                    with threadpool_limits(limits=1):
                        v1, sample1 = cpu_sample(args.cpu_budget * 0.3)
                    cpu["one_thread"] = {"value": round(v1, 4), "cores": 1, "sample": sample1}
                except ImportError:
                    cpu["one_thread"] = None
        hev.close()
        # free this workload's device memory before the next one
        del calls, extra, built
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return {"value": value, "unit": unit, "ms": ms, "device_ms": device_ms, "config": config,
                "roofline": roof, "calls": per, "cpu": cpu,
                "settle": {"steps": settle_steps, "ms": round(settle_ms, 1)}}

    with_cpu = not args.no_cpu_baseline
    main_r = measure(args.workload, with_cpu)
    secondary = {}
    if args.workload == "llama70b_decode_layer" and not args.no_secondary:
        for name in SECONDARY_METRIC:
            r = measure(name, with_cpu)
            e = {"metric": SECONDARY_METRIC[name], "value": round(r["value"], 1),
                 "unit": r["unit"], "ms_per_step": round(r["ms"], 4),
                 "device_ms_per_step": round(r["device_ms"], 4), "settle": r["settle"],
                 "config": r["config"],
                 "roofline": r["roofline"], "cpu_baseline": r["cpu"], "calls": r["calls"]}
            if name == "heavy_tailed_mixed_batch":
                c = r["calls"]
                routed = sum(c[k]["ms"] for k in ("paged_decode", "extend_attn", "prefill_attn"))
                e["three_way_attention_ms"] = round(routed, 5)
                e["unified_attention_ms"] = c["unified_extend_attn"]["ms"]
                e["unified_vs_three_way_time"] = round(c["unified_extend_attn"]["ms"] / routed, 3)
            if name == "decode_layout_compare":
                c = r["calls"]
                e["preshuffled_vs_nhd"] = round(c["paged_decode_preshuffled"]["GB/s"] /
                                                c["paged_decode_nhd"]["GB/s"], 4)
            secondary[name] = e
    value, unit, ms, config = main_r["value"], main_r["unit"], main_r["ms"], main_r["config"]
    roof, per, cpu = main_r["roofline"], main_r["calls"], main_r["cpu"]

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": main_r["settle"],
        "ms_per_step": round(ms, 4),
        "device_ms_per_step": round(main_r["device_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded numpy PCG64; no datasets or weights)",
        "config": config, "roofline": roof, "cpu_baseline": cpu, "calls": per,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
