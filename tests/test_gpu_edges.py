"""GPU parity at the degenerate edges of the method: empty sequences inside a
varlen prefill, an all-empty call, one-token decode contexts, extends with no
cached context (which are prefills) and one-token extends (which are decodes of
the context plus that token), and a long single prefill that spans many tiles
with a ragged tail.  Each is compared with the oracle (bf16 outputs within
1.5e-2, lse within 1e-3) and, where two paths must agree, with each other."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import attention as oa, bf16 as ob
from synth import workloads as w

from .gpu_util import (BF16_TOL, LSE_TOL, bf16_to_f64, dev, device_cache, max_err, oracle_cache,
                       say, torch)

pytestmark = pytest.mark.gpu

SCALE = 1 / np.sqrt(128)


def _prefill(lens, Hq, Hkv, causal, seed):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = w.normal_bf16(rng, (T, Hq, 128))
    k = w.normal_bf16(rng, (T, Hkv, 128))
    v = w.normal_bf16(rng, (T, Hkv, 128))
    out, lse = pk.prefill_attn(dev(q), dev(k), dev(v), dev(cu), max(max(lens), 1), SCALE, causal)
    torch().cuda.synchronize()
    return cu, q, k, v, bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_with_empty_sequences(causal):
    """Zero-length requests between and around real ones own no rows and
    change nothing for their neighbours."""
    lens = [0, 5, 0, 0, 200, 129, 0]
    say(f"prefill with empty sequences causal={causal} lens={lens}")
    cu, q, k, v, out, lse = _prefill(lens, 8, 2, causal, 41)
    ro, rl = oa.prefill(ob.to_f64(q), ob.to_f64(k), ob.to_f64(v), cu, SCALE, causal)
    assert max_err(out, ro) <= BF16_TOL
    assert max_err(lse, rl) <= LSE_TOL


def test_prefill_all_empty_is_noop():
    say("prefill with only empty sequences")
    t = torch()
    cu = dev(np.zeros(4, dtype=np.int32))
    q = t.zeros((0, 8, 128), dtype=t.bfloat16, device="cuda")
    kv = t.zeros((0, 2, 128), dtype=t.bfloat16, device="cuda")
    out, lse = pk.prefill_attn(q, kv, kv, cu, 0, SCALE)
    t.cuda.synchronize()
    assert out.shape == (0, 8, 128) and lse.shape == (0, 8)


def test_prefill_long_single_sequence_sampled():
    """One 16000-token sequence (125 query tiles, a ragged last one), causal
    and not, 8:1 heads; sampled rows including the first and last ones."""
    n = 16000
    for causal in (True, False):
        say(f"prefill 1x{n} 8:1 causal={causal}")
        cu, q, k, v, out, lse = _prefill([n], 8, 1, causal, 42)
        rng = np.random.default_rng(7)
        rows = sorted(set([0, 1, 63, 64, 127, 128, n - 129, n - 2, n - 1]
                          + list(rng.integers(0, n, 24))))
        ro, rl = oa.prefill(ob.to_f64(q), ob.to_f64(k), ob.to_f64(v), cu, SCALE, causal,
                            rows=rows)
        e = max_err(out[rows], ro[rows])
        el = max_err(lse[rows], rl[rows])
        say(f"  max|err| out {e:.3e} lse {el:.3e}")
        assert e <= BF16_TOL and el <= LSE_TOL


def test_decode_one_token_contexts():
    """Every request has a single cached token: o = v_0 and lse = s_0."""
    st = w.decode_workload(43, 6, 16, 2, 128, 16, 64, 1, 1)
    assert (st.seq_lens == 1).all()
    say("decode with one-token contexts")
    dc = device_cache(st.cache)
    out, lse = pk.paged_decode(dc, dev(st.q), dev(st.block_tables), dev(st.seq_lens), 1, st.scale)
    torch().cuda.synchronize()
    ro, rl = oa.paged_decode(ob.to_f64(st.q), oracle_cache(st.cache), st.block_tables,
                             st.seq_lens, st.scale)
    assert max_err(bf16_to_f64(out), ro) <= BF16_TOL
    assert max_err(lse.cpu().numpy().astype(np.float64), rl) <= LSE_TOL


def _extend(mb, budget=32768):
    e0, e1 = mb.rows_extend
    dc = device_cache(mb.cache)
    q, kn, vn = dev(mb.q[e0:e1]), dev(mb.k_new[e0:e1]), dev(mb.v_new[e0:e1])
    out, lse = pk.extend_attn(dc, q, kn, vn, dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables),
                              int(np.diff(mb.ext_cu_q).max()), max(int(mb.ext_ctx.max()), 0),
                              mb.scale, budget)
    torch().cuda.synchronize()
    ro, rl = oa.extend(ob.to_f64(mb.q[e0:e1]), ob.to_f64(mb.k_new[e0:e1]),
                       ob.to_f64(mb.v_new[e0:e1]), mb.ext_cu_q, mb.ext_ctx, oracle_cache(mb.cache),
                       mb.ext_tables, mb.scale)
    return bf16_to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl


def test_extend_without_context_equals_prefill():
    """Extends whose cached context is empty are causal prefills of their new
    tokens: against the oracle, and against prefill_attn on the same rows."""
    new = [1, 64, 130, 300]
    mb = w.mixed_batch(44, 16, 2, 128, 16, 64, [], [0, 0, 0, 0], new, [])
    say(f"extend with empty contexts new={new}")
    out, lse, ro, rl = _extend(mb)
    assert max_err(out, ro) <= BF16_TOL and max_err(lse, rl) <= LSE_TOL
    e0, e1 = mb.rows_extend
    po, pl = pk.prefill_attn(dev(mb.q[e0:e1]), dev(mb.k_new[e0:e1]), dev(mb.v_new[e0:e1]),
                             dev(mb.ext_cu_q), max(new), mb.scale, True)
    torch().cuda.synchronize()
    assert max_err(bf16_to_f64(po), out) <= 2 * BF16_TOL
    assert max_err(pl.cpu().numpy().astype(np.float64), lse) <= LSE_TOL


def test_extend_one_new_token_equals_decode():
    """An extend of one token on C cached tokens attends to exactly what a
    decode of C + 1 tokens does once that token is in the cache."""
    ctx = [1, 15, 16, 17, 500, 1000]
    mb = w.mixed_batch(45, 8, 2, 128, 16, 256, [], ctx, [1] * len(ctx), [])
    say(f"extend one token ctx={ctx}")
    out, lse, ro, rl = _extend(mb, budget=64)
    assert max_err(out, ro) <= BF16_TOL and max_err(lse, rl) <= LSE_TOL
    # the same rows through paged_decode after writing the new token
    e0, e1 = mb.rows_extend
    dc = device_cache(mb.cache)
    pk.kv_write(dc, dev(mb.k_new[e0:e1]), dev(mb.v_new[e0:e1]), dev(mb.slot_mapping[e0:e1]))
    lens = (np.asarray(ctx) + 1).astype(np.int32)
    do, dl = pk.paged_decode(dc, dev(mb.q[e0:e1]), dev(mb.ext_tables), dev(lens), int(lens.max()),
                             mb.scale)
    torch().cuda.synchronize()
    assert max_err(bf16_to_f64(do), out) <= 2 * BF16_TOL
    assert max_err(dl.cpu().numpy().astype(np.float64), lse) <= LSE_TOL


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (6, 2)])
def test_prefill_persistent_walk(causal, Hq, Hkv):
    """Many more work items than CUs, so every persistent workgroup runs a
    series of them, with odd and even key-tile counts (an item then starts in
    either LDS buffer) and many skipped items (query tiles past a short
    sequence); head groups of 8 (two heads per item) and of 3 (two query tiles
    per item).  Sampled rows of every sequence against the oracle."""
    rng = np.random.default_rng(46)
    lens = [int(x) for x in rng.integers(1, 320, 300)] + [130, 129, 65, 64, 63, 1]
    say(f"prefill persistent walk causal={causal} {Hq}:{Hkv} seqs={len(lens)}")
    cu, q, k, v, out, lse = _prefill(lens, Hq, Hkv, causal, 47)
    rows = []
    for n in range(len(lens)):
        s0, L = int(cu[n]), lens[n]
        rows += sorted({s0, s0 + L - 1, s0 + int(rng.integers(0, L))})
    ro, rl = oa.prefill(ob.to_f64(q), ob.to_f64(k), ob.to_f64(v), cu, SCALE, causal, rows=rows)
    e = max_err(out[rows], ro[rows])
    el = max_err(lse[rows], rl[rows])
    say(f"  max|err| out {e:.3e} lse {el:.3e} over {len(rows)} rows")
    assert e <= BF16_TOL and el <= LSE_TOL
    assert not np.isnan(out).any()


def test_prefill_walk_mostly_empty_rounds():
    """299 one-token prompts beside one of 131072 tokens, 8:2 heads: every
    request gets as many query items as the longest (1024), so a persistent
    workgroup walks ~4800 rounds, nearly all of them empty and skipped.  Every
    short row and sampled rows of the long prompt against the oracle."""
    lens = [1] * 299 + [131072]
    say("prefill 299 x 1 + 1 x 131072 tokens, 8:2, causal")
    cu, q, k, v, out, lse = _prefill(lens, 8, 2, True, 48)
    n = lens[-1]
    s0 = int(cu[-2])
    rng = np.random.default_rng(8)
    rows = list(range(299)) + sorted({s0, s0 + 1, s0 + 127, s0 + 128, s0 + n - 1}
                                     | {s0 + int(x) for x in rng.integers(0, n, 12)})
    ro, rl = oa.prefill(ob.to_f64(q), ob.to_f64(k), ob.to_f64(v), cu, SCALE, True, rows=rows)
    e = max_err(out[rows], ro[rows])
    el = max_err(lse[rows], rl[rows])
    say(f"  max|err| out {e:.3e} lse {el:.3e} over {len(rows)} rows")
    assert e <= BF16_TOL and el <= LSE_TOL


@pytest.mark.parametrize("bs", [1, 16, 32])
def test_extend_fused_ragged_contexts(bs):
    """Enough query tiles for the fused extend (64 heads x 17 query tiles),
    with cached contexts of 1, 63, 64, 65 and 1000 tokens (partial first and
    last key tiles) and block sizes whose tiles are not whole blocks (1, 32)
    as well as 16; the cache past every context is poisoned.  Sampled rows
    of every request against the oracle."""
    ctx, new = [1, 63, 64, 65, 1000], [600, 500, 400, 300, 300]
    nb = sum((c + n + bs - 1) // bs for c, n in zip(ctx, new)) + 64
    mb = w.mixed_batch(48, 64, 4, 128, bs, nb, [], ctx, new, [])
    w.poison_cache(mb.cache, mb.ext_tables, mb.ext_ctx)
    say(f"extend fused ragged contexts bs={bs} ctx={ctx} new={new}")
    e0, e1 = mb.rows_extend
    dc = device_cache(mb.cache)
    q, kn, vn = dev(mb.q[e0:e1]), dev(mb.k_new[e0:e1]), dev(mb.v_new[e0:e1])
    out, lse = pk.extend_attn(dc, q, kn, vn, dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables),
                              max(new), max(ctx), mb.scale, 32768)
    torch().cuda.synchronize()
    out, lse = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(49)
    rows = []
    for i in range(len(new)):
        s0 = int(mb.ext_cu_q[i])
        rows += sorted({s0, s0 + 1, s0 + 127, s0 + 128, s0 + new[i] - 1}
                       | {s0 + int(x) for x in rng.integers(0, new[i], 6)})
    ro, rl = oa.extend(ob.to_f64(mb.q[e0:e1]), ob.to_f64(mb.k_new[e0:e1]),
                       ob.to_f64(mb.v_new[e0:e1]), mb.ext_cu_q, mb.ext_ctx,
                       oracle_cache(mb.cache), mb.ext_tables, mb.scale, rows=rows)
    e = max_err(out[rows], ro[rows])
    el = max_err(lse[rows], rl[rows])
    say(f"  max|err| out {e:.3e} lse {el:.3e} over {len(rows)} rows")
    assert e <= BF16_TOL and el <= LSE_TOL
    assert not np.isnan(out).any()
