"""GPU parity of the hybrid extend ("Beyond just running: native inference
optimisation in vLLM on AMD ROCm", section "Processing details of the three
paths", extend path: (1) the new tokens among themselves, (2) all new tokens
against each chunk of the cached context, (3) the log-sum-exp merge; section
"Why route three ways explicitly": extend batches mix long and short
requests).  In automatic mode, when the fused execution is chosen and the
context spans two or more chunks, a device-side plan lists every query item
of the batch (requests heaviest first) and runs the requests whose walk would
hold their workgroups far beyond the batch's mean load split -- their chunks
in parallel, partials merged -- beside the fused requests in the same launch.

Checks: the plan (white box: the first two words of the workspace are the
number of split requests and the compact rows they use) splits the expected
requests; the rows of split requests equal the forced split execution bit for
bit and the others the forced fused one (the same work items, the same merge
order); the oracle agrees within 1.5e-2 (bf16 caches) / 5e-2 (fp8), lse 1e-3;
a workspace too small for the plan falls back to plain fused."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import attention as oa, bf16 as ob
from synth import workloads as w

from .gpu_util import (BF16_TOL, FP8_TOL, LSE_TOL, bf16_to_f64, dev, device_cache, max_err,
                       oracle_cache, say, torch)

pytestmark = pytest.mark.gpu

ONE_LONG_CTX = [20000, 500, 1200, 64, 3000, 0, 900]
ONE_LONG_NEW = [29, 700, 900, 1000, 512, 800, 1024]

# (name, Hq, Hkv, contexts, new tokens, budget, layout, dtype, split requests)
CASES = [
    ("64:4 one long request", 64, 4, ONE_LONG_CTX, ONE_LONG_NEW, 32768, "nhd", "bf16", [0]),
    ("24:8 odd group", 24, 8, ONE_LONG_CTX, [29, 1500, 1500, 1000, 512, 800, 1024], 32768,
     "nhd", "bf16", [0]),
    ("64:8 two long requests", 64, 8, [9000, 300, 7000, 100, 50], [40, 1600, 3, 1500, 1000],
     8192, "nhd", "bf16", [0, 2]),
    ("64:4 fp8 nhd", 64, 4, ONE_LONG_CTX, ONE_LONG_NEW, 32768, "nhd", "fp8", [0]),
    ("64:4 fp8 preshuffled", 64, 4, ONE_LONG_CTX, ONE_LONG_NEW, 32768, "preshuffled", "fp8", [0]),
    ("64:4 bf16 preshuffled", 64, 4, ONE_LONG_CTX, ONE_LONG_NEW, 32768, "preshuffled", "bf16", [0]),
    # four lanes only (fewer than the XCDs): one long request beside a
    # 16000-token extend that alone fills the GPU
    ("8:2 few lanes", 8, 2, [30000, 100, 200], [20, 16000, 500], 8192, "nhd", "bf16", [0]),
]


def _batch(seed, Hq, Hkv, ctx, new, layout, dtype):
    nb = sum(-(-(c + n) // 16) for c, n in zip(ctx, new)) + 64
    mb = w.mixed_batch(seed, Hq, Hkv, 128, 16, nb, [], ctx, new, [], layout=layout, dtype=dtype)
    w.poison_cache(mb.cache, mb.ext_tables, mb.ext_ctx)
    return mb


def _run(mb, dc, budget, mode, workspace=None):
    e0, e1 = mb.rows_extend
    q, kn, vn = dev(mb.q[e0:e1]), dev(mb.k_new[e0:e1]), dev(mb.v_new[e0:e1])
    out, lse = pk.extend_attn(dc, q, kn, vn, dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables),
                              int(np.diff(mb.ext_cu_q).max()), int(mb.ext_ctx.max()), mb.scale,
                              budget, mode=mode, workspace=workspace)
    torch().cuda.synchronize()
    return bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)


def _same(a, b, rows, what):
    assert np.array_equal(a[0][rows], b[0][rows]), f"{what}: outputs differ"
    assert np.array_equal(a[1][rows], b[1][rows]), f"{what}: lse differ"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_hybrid_extend(case):
    name, Hq, Hkv, ctx, new, budget, layout, dtype, expect = case
    t = torch()
    mb = _batch(71, Hq, Hkv, ctx, new, layout, dtype)
    dc = device_cache(mb.cache)
    E, T = len(ctx), int(sum(new))
    say(f"hybrid extend {name}: ctx {ctx} new {new} budget {budget}")
    need = pk.extend_attn_workspace_bytes(dc, E, T, Hq, max(ctx), budget)
    assert need > 0
    ws = t.full((need,), 0x7F, dtype=t.uint8, device="cuda")     # stale contents
    hyb = _run(mb, dc, budget, "auto", ws)
    n_split, used = ws[:8].view(t.int32).cpu().tolist()
    assert n_split == len(expect) and used == sum(new[b] for b in expect), (n_split, used)
    fused = _run(mb, dc, budget, "fused")
    split = _run(mb, dc, budget, "split")
    cu = mb.ext_cu_q
    srows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in expect])
    frows = np.setdiff1d(np.arange(T), srows)
    _same(hyb, split, srows, "split requests vs forced split")
    _same(hyb, fused, frows, "fused requests vs forced fused")
    # the oracle: every row of the split requests, the ends of the others and
    # random rows
    rng = np.random.default_rng(71)
    ends = np.concatenate([cu[:-1], cu[1:] - 1])
    ends = ends[(ends >= 0) & (ends < T) & np.isin(ends, frows)]
    rows = np.unique(np.concatenate([srows, ends, rng.choice(frows, 48, replace=False)]))
    e0, e1 = mb.rows_extend
    ro, rl = oa.extend(ob.to_f64(mb.q[e0:e1]), ob.to_f64(mb.k_new[e0:e1]),
                       ob.to_f64(mb.v_new[e0:e1]), cu, mb.ext_ctx, oracle_cache(mb.cache),
                       mb.ext_tables, mb.scale, rows=rows)
    tol = FP8_TOL if dtype == "fp8" else BF16_TOL
    e = max_err(hyb[0][rows], ro[rows])
    el = max_err(hyb[1][rows], rl[rows])
    say(f"  max|err| out {e:.3e} lse {el:.3e} over {len(rows)} rows (bound {tol})")
    assert e <= tol and el <= LSE_TOL, (e, el)


def test_hybrid_falls_back_to_fused_without_room():
    """A workspace smaller than the plan needs: the call runs plain fused (no
    error), bit for bit."""
    t = torch()
    mb = _batch(72, 64, 4, ONE_LONG_CTX, ONE_LONG_NEW, "nhd", "bf16")
    dc = device_cache(mb.cache)
    say("hybrid extend with a 16-byte workspace")
    small = _run(mb, dc, 32768, "auto", t.zeros(16, dtype=t.uint8, device="cuda"))
    fused = _run(mb, dc, 32768, "fused")
    rows = np.arange(int(sum(ONE_LONG_NEW)))
    _same(small, fused, rows, "fallback vs forced fused")


def test_hybrid_nothing_to_split_is_fused():
    """Requests of equal length: no walk stands out, the plan splits none and
    every row is the fused execution's."""
    t = torch()
    mb = _batch(73, 64, 4, [6000] * 4, [1024] * 4, "nhd", "bf16")
    dc = device_cache(mb.cache)
    need = pk.extend_attn_workspace_bytes(dc, 4, 4096, 64, 6000, 8192)
    ws = t.full((need,), 0x7F, dtype=t.uint8, device="cuda")
    say("hybrid extend, four equal requests")
    hyb = _run(mb, dc, 8192, "auto", ws)
    assert ws[:8].view(t.int32).cpu().tolist() == [0, 0]
    _same(hyb, _run(mb, dc, 8192, "fused"), np.arange(4096), "no split vs forced fused")
