"""GPU parity: prefill and extend attention, and the whole mixed batch, against
the oracle (bf16 outputs within 1.5e-2, lse within 1e-3)."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import attention as oa, bf16 as ob, cache as oc
from synth import workloads as w

from .gpu_util import (BF16_TOL, LSE_TOL, bf16_to_f64, dev, device_cache, max_err, oracle_cache,
                       say, torch)

pytestmark = pytest.mark.gpu


def _prefill_case(seed, lens, Hq, Hkv, D=128):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = w.normal_bf16(rng, (T, Hq, D))
    k = w.normal_bf16(rng, (T, Hkv, D))
    v = w.normal_bf16(rng, (T, Hkv, D))
    return cu, q, k, v


def _cmp_rows(out, lse, ro, rl, rows, tol=BF16_TOL):
    e = max_err(out[rows], ro[rows])
    el = max_err(lse[rows], rl[rows])
    say(f"  max|err| out {e:.3e} lse {el:.3e} over {len(rows)} rows")
    assert e <= tol, e
    assert el <= LSE_TOL, el


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (16, 1)])
def test_prefill_varlen_small(causal, Hq, Hkv):
    lens = [1, 13, 64, 127, 128, 129, 300]
    cu, q, k, v = _prefill_case(21, lens, Hq, Hkv)
    say(f"prefill varlen causal={causal} {Hq}:{Hkv} lens={lens}")
    out, lse = pk.prefill_attn(dev(q), dev(k), dev(v), dev(cu), max(lens), 1 / np.sqrt(128), causal)
    torch().cuda.synchronize()
    ro, rl = oa.prefill(ob.to_f64(q), ob.to_f64(k), ob.to_f64(v), cu, 1 / np.sqrt(128), causal)
    rows = np.arange(cu[-1])
    _cmp_rows(bf16_to_f64(out), lse.cpu().numpy(), ro, rl, rows)


def test_prefill_qwen3_shape_sampled():
    """2 prefills of 2000 tokens, 64:4 heads; 96 sampled rows checked."""
    cu, q, k, v = _prefill_case(22, [2000, 2000], 64, 4)
    say("prefill 2x2000 64:4")
    out, lse = pk.prefill_attn(dev(q), dev(k), dev(v), dev(cu), 2000, 1 / np.sqrt(128))
    torch().cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 1, 127, 128, 1999, 2000, 2001, 3999] + list(rng.integers(0, 4000, 88))))
    ro, rl = oa.prefill(ob.to_f64(q), ob.to_f64(k), ob.to_f64(v), cu, 1 / np.sqrt(128), rows=rows)
    _cmp_rows(bf16_to_f64(out), lse.cpu().numpy(), ro, rl, rows)


def _extend_inputs(mb):
    e0, e1 = mb.rows_extend
    dc = device_cache(mb.cache)
    return dc, e0, e1


def _run_extend(mb, dc, budget, e0, e1):
    q, kn, vn = dev(mb.q[e0:e1]), dev(mb.k_new[e0:e1]), dev(mb.v_new[e0:e1])
    out, lse = pk.extend_attn(dc, q, kn, vn, dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables),
                              int(np.diff(mb.ext_cu_q).max()), int(mb.ext_ctx.max()), mb.scale,
                              budget)
    torch().cuda.synchronize()
    return bf16_to_f64(out), lse.cpu().numpy()


def _oracle_extend(mb, e0, e1, rows=None):
    return oa.extend(ob.to_f64(mb.q[e0:e1]), ob.to_f64(mb.k_new[e0:e1]), ob.to_f64(mb.v_new[e0:e1]),
                     mb.ext_cu_q, mb.ext_ctx, oracle_cache(mb.cache), mb.ext_tables, mb.scale,
                     rows=rows)


@pytest.mark.parametrize("budget", [32768, 640, 64])
def test_extend_small_chunked(budget):
    mb = w.mixed_batch(31, 8, 2, 128, 16, 200, [], [0, 5, 64, 100, 333, 700], [1, 7, 128, 129, 64, 200], [])
    w.poison_cache(mb.cache, mb.ext_tables, mb.ext_ctx)   # nothing past the context may be read
    say(f"extend small budget={budget}")
    dc, e0, e1 = _extend_inputs(mb)
    out, lse = _run_extend(mb, dc, budget, e0, e1)
    ro, rl = _oracle_extend(mb, e0, e1)
    _cmp_rows(out, lse, ro, rl, np.arange(e1 - e0))


def test_extend_qwen3_shape_full():
    """4 extends of 512 new tokens on 2000 cached, 64:4 heads, automatic
    execution: every row (the split execution at several budgets is tested in
    test_gpu_extend_modes)."""
    mb = w.qwen3_mixed_batch()
    e0, e1 = mb.rows_extend
    say("extend 4x(2000+512) 64:4")
    dc = device_cache(mb.cache)
    out, lse = _run_extend(mb, dc, 32768, e0, e1)
    out2, lse2 = _run_extend(mb, dc, 32768, e0, e1)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)        # deterministic
    ro, rl = _oracle_extend(mb, e0, e1)
    _cmp_rows(out, lse, ro, rl, np.arange(e1 - e0))


def test_extend_long_context_full_size_sampled():
    """2 requests with 100000 cached and 8192 new tokens, 64:8 heads, budget
    32768 (16384-token chunks); sampled rows against the oracle."""
    mb = w.long_context_extend()
    e0, e1 = mb.rows_extend
    say("extend long context 2x(100000+8192) 64:8")
    dc = device_cache(mb.cache)
    out, lse = _run_extend(mb, dc, 32768, e0, e1)
    rng = np.random.default_rng(4)
    rows = sorted(set([0, 1, 8191, 8192, 8193, 16383] + list(rng.integers(0, 16384, 10))))
    ro, rl = _oracle_extend(mb, e0, e1, rows=rows)
    _cmp_rows(out, lse, ro, rl, rows)


def test_mixed_batch_end_to_end():
    """The Qwen3-shaped batch through the whole path: reorder from arrival
    order, write every row's K/V, then decode / extend / prefill into slices of
    one output."""
    mb = w.qwen3_mixed_batch()
    perm, counts = pk.reorder_batch(mb.raw_query_lens, mb.raw_ctx_lens)
    assert counts == (48, 4, 2)
    qsorted = np.asarray(mb.raw_query_lens)[perm]
    assert (qsorted[:48] == 1).all() and (qsorted[48:52] == 512).all() and (qsorted[52:] == 2000).all()
    say("mixed batch end to end")
    dc = device_cache(mb.cache)
    t = torch()
    q, kn, vn = dev(mb.q), dev(mb.k_new), dev(mb.v_new)
    pk.kv_write(dc, kn, vn, dev(mb.slot_mapping))
    out = t.empty_like(q)
    lse = t.empty((q.shape[0], mb.num_q_heads), dtype=t.float32, device=q.device)
    d0, d1 = mb.rows_decode
    e0, e1 = mb.rows_extend
    p0, p1 = mb.rows_prefill
    pk.paged_decode(dc, q[d0:d1], dev(mb.dec_tables), dev(mb.dec_seq_lens),
                    int(mb.dec_seq_lens.max()), mb.scale, out=out[d0:d1], lse=lse[d0:d1])
    pk.extend_attn(dc, q[e0:e1], kn[e0:e1], vn[e0:e1], dev(mb.ext_cu_q), dev(mb.ext_ctx),
                   dev(mb.ext_tables), 512, 2000, mb.scale, 32768, out=out[e0:e1], lse=lse[e0:e1])
    pk.prefill_attn(q[p0:p1], kn[p0:p1], vn[p0:p1], dev(mb.pre_cu), 2000, mb.scale,
                    out=out[p0:p1], lse=lse[p0:p1])
    t.cuda.synchronize()
    o = bf16_to_f64(out)
    l = lse.cpu().numpy()
    ocache = oc.write(oracle_cache(mb.cache), mb.k_new, mb.v_new, mb.slot_mapping)
    qf = ob.to_f64(mb.q)
    ro, rl = oa.paged_decode(qf[d0:d1], ocache, mb.dec_tables, mb.dec_seq_lens, mb.scale)
    _cmp_rows(o[d0:d1], l[d0:d1], ro, rl, np.arange(d1 - d0))
    rows = list(range(0, e1 - e0, 37))
    ro, rl = _oracle_extend(mb, e0, e1, rows=rows)
    _cmp_rows(o[e0:e1], l[e0:e1], ro, rl, rows)
    rows = list(range(0, p1 - p0, 53))
    ro, rl = oa.prefill(qf[p0:p1], ob.to_f64(mb.k_new[p0:p1]), ob.to_f64(mb.v_new[p0:p1]),
                        mb.pre_cu, mb.scale, rows=rows)
    _cmp_rows(o[p0:p1], l[p0:p1], ro, rl, rows)
