"""GPU parity on a heavy-tailed mixed batch (lognormal lengths: many short
extends beside a few long ones, decodes from 16 to 15000 tokens), run both
ways the pages contrast ("Beyond just running: native inference optimisation
in vLLM on AMD ROCm", section "Why route three ways explicitly"): three-way
routing (paged_decode + extend_attn + prefill_attn on the reordered batch)
and ONE extend call over every request (decode = 1 new token on L - 1 cached
tokens, prefill = no cached context).  Both against the oracle."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import attention as oa, bf16 as ob, cache as oc
from synth import workloads as w

from .gpu_util import (BF16_TOL, LSE_TOL, bf16_to_f64, dev, device_cache, max_err, oracle_cache,
                       say, torch)

pytestmark = pytest.mark.gpu


def _unified_args(mb):
    nd = mb.n_decode
    qlens = np.concatenate([np.ones(nd, np.int64), np.diff(mb.ext_cu_q), np.diff(mb.pre_cu)])
    ctx = np.concatenate([mb.dec_seq_lens - 1, mb.ext_ctx,
                          np.zeros(len(mb.pre_cu) - 1, np.int64)]).astype(np.int32)
    width = max(mb.dec_tables.shape[1], mb.ext_tables.shape[1])
    tables = np.full((len(qlens), width), mb.cache.poison_block, np.int32)
    tables[:nd, :mb.dec_tables.shape[1]] = mb.dec_tables
    tables[nd:nd + len(mb.ext_ctx), :mb.ext_tables.shape[1]] = mb.ext_tables
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return cu, ctx, tables


def _cmp(out, lse, ro, rl, rows, what):
    e = max_err(out[rows], ro[rows])
    el = max_err(lse[rows], rl[rows])
    say(f"  {what}: max|err| out {e:.3e} lse {el:.3e} over {len(rows)} rows")
    assert e <= BF16_TOL and el <= LSE_TOL, (e, el)


def test_heavy_tailed_batch_three_way_and_unified():
    mb = w.heavy_tailed_mixed_batch()
    t = torch()
    say(f"heavy-tailed batch: {mb.n_decode} decodes, extends new {np.diff(mb.ext_cu_q).tolist()} "
        f"ctx {mb.ext_ctx.tolist()}, prefills {np.diff(mb.pre_cu).tolist()}")
    dc = device_cache(mb.cache)
    q, kn, vn = dev(mb.q), dev(mb.k_new), dev(mb.v_new)
    pk.kv_write(dc, kn, vn, dev(mb.slot_mapping))
    d0, d1 = mb.rows_decode
    e0, e1 = mb.rows_extend
    p0, p1 = mb.rows_prefill
    T, Hq = q.shape[0], mb.num_q_heads
    out = t.empty_like(q)
    lse = t.empty((T, Hq), dtype=t.float32, device="cuda")
    pk.paged_decode(dc, q[d0:d1], dev(mb.dec_tables), dev(mb.dec_seq_lens),
                    int(mb.dec_seq_lens.max()), mb.scale, out=out[d0:d1], lse=lse[d0:d1])
    pk.extend_attn(dc, q[e0:e1], kn[e0:e1], vn[e0:e1], dev(mb.ext_cu_q), dev(mb.ext_ctx),
                   dev(mb.ext_tables), int(np.diff(mb.ext_cu_q).max()), int(mb.ext_ctx.max()),
                   mb.scale, 32768, out=out[e0:e1], lse=lse[e0:e1])
    pk.prefill_attn(q[p0:p1], kn[p0:p1], vn[p0:p1], dev(mb.pre_cu), int(np.diff(mb.pre_cu).max()),
                    mb.scale, out=out[p0:p1], lse=lse[p0:p1])
    cu, ctx, tables = _unified_args(mb)
    uout, ulse = pk.extend_attn(dc, q, kn, vn, dev(cu), dev(ctx), dev(tables),
                                int(np.diff(cu).max()), int(ctx.max()), mb.scale, 32768)
    t.cuda.synchronize()
    o, l = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
    uo, ul = bf16_to_f64(uout), ulse.cpu().numpy().astype(np.float64)

    ocache = oc.write(oracle_cache(mb.cache), mb.k_new, mb.v_new, mb.slot_mapping)
    qf, kf, vf = ob.to_f64(mb.q), ob.to_f64(mb.k_new), ob.to_f64(mb.v_new)
    rng = np.random.default_rng(6)
    # decode rows: all of them
    rd, rld = oa.paged_decode(qf[d0:d1], ocache, mb.dec_tables, mb.dec_seq_lens, mb.scale)
    _cmp(o[d0:d1], l[d0:d1], rd, rld, np.arange(d1 - d0), "three-way decode")
    _cmp(uo[d0:d1], ul[d0:d1], rd, rld, np.arange(d1 - d0), "unified decode rows")
    # extend rows: the first and last row of every request plus random ones
    ends = np.concatenate([mb.ext_cu_q[:-1], mb.ext_cu_q[1:] - 1])
    rows = sorted(set(ends.tolist() + rng.integers(0, e1 - e0, 40).tolist()))
    re_, rle = oa.extend(qf[e0:e1], kf[e0:e1], vf[e0:e1], mb.ext_cu_q, mb.ext_ctx, ocache,
                         mb.ext_tables, mb.scale, rows=rows)
    _cmp(o[e0:e1], l[e0:e1], re_, rle, rows, "three-way extend")
    _cmp(uo[e0:e1], ul[e0:e1], re_, rle, rows, "unified extend rows")
    # prefill rows
    rows = sorted(set([0, 1, 2890, 2891, 5542] + rng.integers(0, p1 - p0, 30).tolist()))
    rows = [r for r in rows if r < p1 - p0]
    rp, rlp = oa.prefill(qf[p0:p1], kf[p0:p1], vf[p0:p1], mb.pre_cu, mb.scale, rows=rows)
    _cmp(o[p0:p1], l[p0:p1], rp, rlp, rows, "three-way prefill")
    _cmp(uo[p0:p1], ul[p0:p1], rp, rlp, rows, "unified prefill rows")
