"""GPU parity of the two extend executions (split: per-chunk partials and a
log-sum-exp merge pass; fused: one running softmax state), forced through
extend_attn_ex at the workloads' sizes, plus needle tests that make a
mis-addressed context block visible.

The pages' extend ("Beyond just running: native inference optimisation in vLLM
on AMD ROCm", section "Processing details of the three paths"): new tokens
among themselves, then each context chunk under the per-iteration budget
(section "ROCM_AITER_FA", about 32K tokens split across the extends), then a
log-sum-exp merge.  Split mode runs exactly those stages; both modes must
match the oracle (bf16 outputs within 1.5e-2, lse within 1e-3)."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import attention as oa, bf16 as ob
from synth import workloads as w

from .gpu_util import (BF16_TOL, LSE_TOL, bf16_to_f64, dev, device_cache, max_err, oracle_cache,
                       say, torch)

pytestmark = pytest.mark.gpu


def _run(mb, dc, budget, mode):
    e0, e1 = mb.rows_extend
    q, kn, vn = dev(mb.q[e0:e1]), dev(mb.k_new[e0:e1]), dev(mb.v_new[e0:e1])
    out, lse = pk.extend_attn(dc, q, kn, vn, dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables),
                              int(np.diff(mb.ext_cu_q).max()), int(mb.ext_ctx.max()), mb.scale,
                              budget, mode=mode)
    torch().cuda.synchronize()
    return bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(mb, rows=None, ocache=None):
    e0, e1 = mb.rows_extend
    return oa.extend(ob.to_f64(mb.q[e0:e1]), ob.to_f64(mb.k_new[e0:e1]), ob.to_f64(mb.v_new[e0:e1]),
                     mb.ext_cu_q, mb.ext_ctx, ocache or oracle_cache(mb.cache), mb.ext_tables,
                     mb.scale, rows=rows)


def _cmp(out, lse, ro, rl, rows, tol=BF16_TOL):
    rows = np.asarray(rows)
    e = max_err(out[rows], ro[rows])
    el = max_err(lse[rows], rl[rows])
    say(f"  max|err| out {e:.3e} lse {el:.3e} over {len(rows)} rows")
    assert e <= tol, e
    assert el <= LSE_TOL, el


def _cmp_modes(a, b):
    """Split and fused compute the same softmax in different fp32 orders:
    every row of both must agree within the output and lse bounds."""
    e = max_err(a[0], b[0])
    el = max_err(a[1], b[1])
    say(f"  split vs fused: max|diff| out {e:.3e} lse {el:.3e} over every row")
    assert e <= BF16_TOL and el <= LSE_TOL


@pytest.mark.parametrize("budget", [32768, 2048])
def test_extend_split_qwen3_every_row(budget):
    """The mixed batch's 4 extends (2000 cached + 512 new, 64:4) run split:
    budget 32768 -> one 8192-token chunk per request (2 parts), budget 2048 ->
    512-token chunks (4 context chunks + the new tokens = 5 parts, merged).
    Every row against the oracle, and against the fused run."""
    mb = w.qwen3_mixed_batch()
    say(f"extend split 4x(2000+512) 64:4 budget={budget}")
    dc = device_cache(mb.cache)
    split = _run(mb, dc, budget, "split")
    again = _run(mb, dc, budget, "split")
    assert np.array_equal(split[0], again[0]) and np.array_equal(split[1], again[1])
    ro, rl = _oracle(mb)
    _cmp(*split, ro, rl, np.arange(ro.shape[0]))
    _cmp_modes(split, _run(mb, dc, budget, "fused"))


def _long_8to1(seed, n_seq=2, ctx=100000, new=512):
    # 8 query heads : 1 KV head, the per-GPU share of a 64:8 model under TP8
    return w.mixed_batch(seed, 8, 1, 128, 16, n_seq * ((ctx + new) // 16 + 2) + 8, [],
                         [ctx] * n_seq, [new] * n_seq, [])


def test_extend_split_long_context_seven_chunks():
    """2 x (100000 cached + 512 new), 8:1 heads, budget 32768: each request
    gets 16384-token chunks -> 7 chunks (the last 1696 tokens) + the new
    tokens, merged by log-sum-exp.  Sampled rows against the oracle, every row
    against the fused execution."""
    mb = _long_8to1(41)
    say("extend split 2x(100000+512) 8:1 budget 32768 (7 chunks + merge)")
    dc = device_cache(mb.cache)
    split = _run(mb, dc, 32768, "split")
    rng = np.random.default_rng(41)
    rows = sorted(set([0, 1, 255, 511, 512, 513, 1023] + list(rng.integers(0, 1024, 25))))
    ro, rl = _oracle(mb, rows)
    _cmp(*split, ro, rl, rows)
    _cmp_modes(split, _run(mb, dc, 32768, "fused"))


def test_extend_split_long_context_full_size_sampled():
    """The long-context workload (2 x (100000 cached + 8192 new), 64:8,
    budget 32768 -> 7 chunks per request + the new tokens) in split mode:
    sampled rows against the oracle, and every row of every head against the
    fused execution."""
    mb = w.long_context_extend()
    say("extend split long context 2x(100000+8192) 64:8")
    dc = device_cache(mb.cache)
    split = _run(mb, dc, 32768, "split")
    rng = np.random.default_rng(44)
    rows = sorted(set([0, 8191, 8192, 16383] + list(rng.integers(0, 16384, 8))))
    ro, rl = _oracle(mb, rows)
    _cmp(*split, ro, rl, rows)
    fused = _run(mb, dc, 32768, "fused")
    _cmp_modes(split, fused)


@pytest.mark.parametrize("mode", ["auto", "fused", "split"])
def test_extend_odd_query_group(mode):
    """24 query heads : 8 KV heads (group of 3): a work item is one query head
    over 256 tokens (an odd group has no power-of-two head split).  5600 new
    tokens give 24 * 44 = 1056 query tiles of 128, enough for the automatic
    plan to fuse on 256 compute units.  Every row against the oracle."""
    mb = w.mixed_batch(45, 24, 8, 128, 16, 700, [], [1000, 77], [2900, 2700], [])
    w.poison_cache(mb.cache, mb.ext_tables, mb.ext_ctx)
    say(f"extend 24:8 mode={mode} new [2900, 2700] ctx [1000, 77]")
    dc = device_cache(mb.cache)
    out, lse = _run(mb, dc, 32768, mode)
    ro, rl = _oracle(mb)
    _cmp(out, lse, ro, rl, np.arange(ro.shape[0]))


def _plant(rng, q, k, v, rows, heads, kv_head, scale_dims=128):
    """A needle: the query rows `rows` of `heads` point along a random unit
    direction u (|q| ~ sqrt(D)), and key k_slot = 30 u.  Their scaled score
    with the needle is ~30 while every other key scores ~N(0, 1), so the
    exact output of those rows is the needle's value row to ~1e-8."""
    D = q.shape[-1]
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    for r in rows:
        for h in heads:
            qv = np.sqrt(scale_dims) * u + 0.1 * rng.standard_normal(D)
            q[r, h] = w.f32_to_bf16_bits(qv.astype(np.float32))
    k[:] = w.f32_to_bf16_bits((30.0 * u).astype(np.float32))
    v[:] = w.f32_to_bf16_bits((3.0 * rng.standard_normal(D)).astype(np.float32))
    return v.copy()


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_extend_needle_deep_in_long_context(mode):
    """2 x (100000 cached + 256 new), 8:1 heads: one needle key in a random
    block deep in each request's context (a different block per request).
    64 query rows per request look for it; their output must be its value
    row.  A context block read from the wrong place moves those rows by O(1)."""
    mb = _long_8to1(46, ctx=100000, new=256)
    rng = np.random.default_rng(46)
    e0, _ = mb.rows_extend
    needles = []
    for e in range(2):
        t = int(rng.integers(50000, 100000))
        blk, off = int(mb.ext_tables[e, t // 16]), t % 16
        rows = e0 + int(mb.ext_cu_q[e]) + rng.choice(256, 64, replace=False)
        vrow = _plant(rng, mb.q, mb.cache.k[blk, off], mb.cache.v[blk, off], rows, range(8), 0)
        needles.append((rows - e0, vrow))
        say(f"  needle of request {e} at context token {t} (block {blk}, offset {off})")
    say(f"extend needle 2x(100000+256) 8:1 mode={mode}")
    out, lse = _run(mb, device_cache(mb.cache), 32768, mode)
    for rows, vrow in needles:
        ro, rl = _oracle(mb, list(rows))
        _cmp(out, lse, ro, rl, rows)
        want = ob.to_f64(vrow[0])
        assert max_err(out[rows], np.broadcast_to(want, out[rows].shape)) <= 0.05


def test_prefill_needle_early_in_long_prompt():
    """A 16000-token causal prefill (8:1 heads) with one needle key at token
    37: 64 later rows spread over the prompt (several hundred query tiles
    past it) must return its value row; 4 rows before it must not see it."""
    rng = np.random.default_rng(47)
    T, Hq, Hkv, D = 16000, 8, 1, 128
    q = w.normal_bf16(rng, (T, Hq, D))
    k = w.normal_bf16(rng, (T, Hkv, D))
    v = w.normal_bf16(rng, (T, Hkv, D))
    rows = np.sort(rng.choice(np.arange(100, T), 64, replace=False))
    vrow = _plant(rng, q, k[37], v[37], rows, range(Hq), 0)
    cu = np.array([0, T], np.int32)
    say("prefill needle 16000 tokens 8:1, needle at token 37")
    out, lse = pk.prefill_attn(dev(q), dev(k), dev(v), dev(cu), T, 1 / np.sqrt(D))
    torch().cuda.synchronize()
    out, lse = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
    check = list(rows) + [0, 5, 36]
    ro, rl = oa.prefill(ob.to_f64(q), ob.to_f64(k), ob.to_f64(v), cu, 1 / np.sqrt(D), rows=check)
    _cmp(out, lse, ro, rl, check)
    want = ob.to_f64(vrow[0])
    assert max_err(out[rows], np.broadcast_to(want, out[rows].shape)) <= 0.05
    assert np.abs(out[[0, 5, 36]] - want).max() > 0.5       # rows before it do not see it
