"""Randomised parity sweep: seeded random prefill, extend and decode shapes
(head groups 1-16, ragged lengths including empty sequences, block sizes 1-64,
NHD and preshuffled layouts, bf16 and fp8 caches, chunk budgets, split sizes),
each against the oracle on sampled rows (bf16 outputs within 1.5e-2, fp8-KV
outputs within 5e-2, lse within 1e-3).  Every case is named before it runs."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import attention as oa, bf16 as ob
from synth import workloads as w

from .gpu_util import (BF16_TOL, FP8_TOL, LSE_TOL, bf16_to_f64, dev, device_cache, max_err,
                       oracle_cache, say, torch)

pytestmark = pytest.mark.gpu

N_CASES = 60
HEADS = [(8, 8), (8, 1), (16, 2), (12, 4), (6, 2), (64, 4), (64, 8), (5, 1), (32, 4)]
# group sizes 2, 4, 6, 12, 24 and 64: a workgroup takes 2, 4, 2, 4, 8 and 8
# query heads (gcd(G, 8)) over 128, 64, 128, 64, 32 and 32 tokens
MORE_GROUPS = [(8, 4), (16, 4), (12, 2), (24, 2), (48, 2), (64, 1)]


def test_random_shapes_against_oracle():
    _sweep(2024, N_CASES, HEADS)


def test_random_shapes_more_head_groups():
    _sweep(2025, 30, MORE_GROUPS)


def _sweep(seed0, n_cases, HEADS):
    t = torch()
    rng = np.random.default_rng(seed0)
    worst = {}
    fails = []
    for n in range(1, n_cases + 1):
        kind = rng.choice(['prefill', 'extend', 'decode'])
        Hq, Hkv = HEADS[rng.integers(len(HEADS))]
        seed = int(rng.integers(1 << 30))
        if kind == 'prefill':
            ns = int(rng.integers(1, 40))
            lens = [int(x) for x in rng.integers(0, 700, ns)]
            if max(lens) == 0:
                lens[0] = 1
            causal = bool(rng.integers(2))
            say(f"[{n}] prefill {Hq}:{Hkv} causal={causal} lens={lens}")
            r2 = np.random.default_rng(seed)
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            T = int(cu[-1])
            q = w.normal_bf16(r2, (T, Hq, 128))
            k = w.normal_bf16(r2, (T, Hkv, 128))
            v = w.normal_bf16(r2, (T, Hkv, 128))
            out, lse = pk.prefill_attn(dev(q), dev(k), dev(v), dev(cu), max(lens), 1 / np.sqrt(128), causal)
            t.cuda.synchronize()
            out, lse = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
            rows = sorted(set(int(x) for x in r2.integers(0, T, min(T, 120))) | {0, T - 1})
            ro, rl = oa.prefill(ob.to_f64(q), ob.to_f64(k), ob.to_f64(v), cu, 1 / np.sqrt(128), causal, rows=rows)
            e, el, tol = max_err(out[rows], ro[rows]), max_err(lse[rows], rl[rows]), BF16_TOL
        elif kind == 'extend':
            ne = int(rng.integers(1, 12))
            bs = int(rng.choice([1, 4, 16, 32, 64]))
            ctx = [int(x) for x in rng.integers(0, 1500, ne)]
            new = [int(x) for x in rng.integers(1, 600, ne)]
            budget = int(rng.choice([64, 256, 2048, 32768]))
            nb = sum((c + m + bs - 1) // bs for c, m in zip(ctx, new)) + 64
            say(f"[{n}] extend {Hq}:{Hkv} bs={bs} budget={budget} ctx={ctx} new={new}")
            mb = w.mixed_batch(seed, Hq, Hkv, 128, bs, nb, [], ctx, new, [])
            w.poison_cache(mb.cache, mb.ext_tables, mb.ext_ctx)
            e0, e1 = mb.rows_extend
            dc = device_cache(mb.cache)
            out, lse = pk.extend_attn(dc, dev(mb.q[e0:e1]), dev(mb.k_new[e0:e1]), dev(mb.v_new[e0:e1]),
                                      dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables), max(new),
                                      max(ctx), mb.scale, budget)
            t.cuda.synchronize()
            out, lse = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
            T = e1 - e0
            r2 = np.random.default_rng(seed + 1)
            rows = sorted(set(int(x) for x in r2.integers(0, T, min(T, 80))) | {0, T - 1})
            ro, rl = oa.extend(ob.to_f64(mb.q[e0:e1]), ob.to_f64(mb.k_new[e0:e1]), ob.to_f64(mb.v_new[e0:e1]),
                               mb.ext_cu_q, mb.ext_ctx, oracle_cache(mb.cache), mb.ext_tables, mb.scale, rows=rows)
            e, el, tol = max_err(out[rows], ro[rows]), max_err(lse[rows], rl[rows]), BF16_TOL
        else:
            B = int(rng.integers(1, 80))
            bs = int(rng.choice([1, 8, 16, 32]))
            layout = str(rng.choice(['nhd', 'preshuffled'])) if bs >= 16 else 'nhd'
            dtype = str(rng.choice(['bf16', 'fp8']))
            hi = int(rng.integers(2, 5000))
            lo = int(rng.integers(1, hi))
            nb = B * ((hi + bs - 1) // bs) + 64
            split = int(rng.choice([0, 0, 64, 256, 1024]))
            say(f"[{n}] decode {Hq}:{Hkv} B={B} bs={bs} {layout} {dtype} lens[{lo},{hi}] split={split}")
            st = w.decode_workload(seed, B, Hq, Hkv, 128, bs, nb, lo, hi, layout=layout, dtype=dtype)
            w.poison_cache(st.cache, st.block_tables, st.seq_lens)
            dc = device_cache(st.cache)
            out, lse = pk.paged_decode(dc, dev(st.q), dev(st.block_tables), dev(st.seq_lens), int(st.seq_lens.max()),
                                       st.scale, split_tokens=split)
            t.cuda.synchronize()
            out, lse = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
            rows = sorted(set(int(x) for x in np.random.default_rng(seed).integers(0, B, min(B, 10))))
            ro, rl = oa.paged_decode(ob.to_f64(st.q[rows]), oracle_cache(st.cache), st.block_tables[rows],
                                     st.seq_lens[rows], st.scale)
            e, el = max_err(out[rows], ro), max_err(lse[rows], rl)
            tol = BF16_TOL if dtype == 'bf16' else FP8_TOL
        ok = e <= tol and el <= LSE_TOL
        worst[kind] = max(worst.get(kind, 0.0), e / tol)
        print(f"    err {e:.3e} lse {el:.3e} {'ok' if ok else 'FAIL'}", flush=True)
        if not ok:
            fails.append(n)

    say(f"worst err/tol {worst}")
    assert not fails, f"cases {fails} out of tolerance"
