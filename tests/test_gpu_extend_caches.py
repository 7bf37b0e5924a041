"""GPU parity of extend_attn on the other caches ("Beyond just running: native
inference optimisation in vLLM on AMD ROCm", section "ROCM_AITER_FA": the
preshuffled layout k [block][head][D/x][block_size][x], v [block][head]
[block_size/x][D][x], and fp8 e4m3 KV with per-tensor scales; section
"Processing details of the three paths": the extend path reads the cached
context chunk by chunk).  The context is read in place through the block
table and decoded while it is staged (no gather copy); both executions
(split and fused) against the oracle: bf16 caches within 1.5e-2, fp8 caches
within 5e-2, lse within 1e-3."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import attention as oa, bf16 as ob
from synth import workloads as w

from .gpu_util import (BF16_TOL, FP8_TOL, LSE_TOL, bf16_to_f64, dev, device_cache, max_err,
                       oracle_cache, say, torch)

pytestmark = pytest.mark.gpu

KINDS = [("nhd", "fp8"), ("preshuffled", "bf16"), ("preshuffled", "fp8")]


def _run(mb, budget, mode, dc=None):
    e0, e1 = mb.rows_extend
    dc = dc or device_cache(mb.cache)
    q, kn, vn = dev(mb.q[e0:e1]), dev(mb.k_new[e0:e1]), dev(mb.v_new[e0:e1])
    out, lse = pk.extend_attn(dc, q, kn, vn, dev(mb.ext_cu_q), dev(mb.ext_ctx), dev(mb.ext_tables),
                              int(np.diff(mb.ext_cu_q).max()), int(mb.ext_ctx.max()), mb.scale,
                              budget, mode=mode)
    torch().cuda.synchronize()
    return bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(mb, rows=None):
    e0, e1 = mb.rows_extend
    return oa.extend(ob.to_f64(mb.q[e0:e1]), ob.to_f64(mb.k_new[e0:e1]), ob.to_f64(mb.v_new[e0:e1]),
                     mb.ext_cu_q, mb.ext_ctx, oracle_cache(mb.cache), mb.ext_tables, mb.scale,
                     rows=rows)


def _cmp(out, lse, ro, rl, rows, tol):
    rows = np.asarray(rows)
    e = max_err(out[rows], ro[rows])
    el = max_err(lse[rows], rl[rows])
    say(f"  max|err| out {e:.3e} lse {el:.3e} over {len(rows)} rows (bound {tol})")
    assert e <= tol, e
    assert el <= LSE_TOL, el


@pytest.mark.parametrize("layout,dtype", KINDS)
@pytest.mark.parametrize("mode,budget", [("fused", 32768), ("split", 32768), ("split", 64)])
def test_extend_ragged_contexts(layout, dtype, mode, budget):
    """Contexts of 0 .. 700 tokens (partial first and last key tiles, blocks
    wholly past a context inside its last tile), new tokens 1 .. 300, 8:2
    heads; every slot past a context is NaN, so any over-read shows."""
    mb = w.mixed_batch(51, 8, 2, 128, 16, 400, [], [0, 5, 16, 63, 64, 65, 100, 333, 700],
                       [1, 7, 128, 129, 64, 200, 3, 50, 300], [], layout=layout, dtype=dtype)
    w.poison_cache(mb.cache, mb.ext_tables, mb.ext_ctx)
    say(f"extend {layout} {dtype} mode={mode} budget={budget} ragged contexts")
    out, lse = _run(mb, budget, mode)
    ro, rl = _oracle(mb)
    _cmp(out, lse, ro, rl, np.arange(ro.shape[0]), BF16_TOL if dtype == "bf16" else FP8_TOL)


@pytest.mark.parametrize("bs", [1, 32])
def test_extend_nhd_fp8_block_sizes(bs):
    mb = w.mixed_batch(52, 16, 2, 128, bs, 12 * 800 // bs + 64, [], [1, 31, 32, 33, 500, 777],
                       [5, 64, 65, 1, 130, 20], [], dtype="fp8")
    w.poison_cache(mb.cache, mb.ext_tables, mb.ext_ctx)
    say(f"extend nhd fp8 bs={bs}")
    for mode in ("fused", "split"):
        out, lse = _run(mb, 256, mode)
        ro, rl = _oracle(mb)
        _cmp(out, lse, ro, rl, np.arange(ro.shape[0]), FP8_TOL)


@pytest.mark.parametrize("layout,dtype", KINDS)
def test_extend_qwen3_shape_other_caches(layout, dtype):
    """The mixed batch's 4 extends (2000 cached + 512 new, 64:4) on the other
    caches: every row, split (512-token chunks: 4 chunks + the new tokens,
    merged) and fused."""
    mb = w.mixed_batch(3, 64, 4, 128, 16, 12288, [], [2000] * 4, [512] * 4, [], layout=layout,
                       dtype=dtype)
    dc = device_cache(mb.cache)
    ro, rl = _oracle(mb)
    tol = BF16_TOL if dtype == "bf16" else FP8_TOL
    for mode, budget in (("split", 2048), ("fused", 32768)):
        say(f"extend 4x(2000+512) 64:4 {layout} {dtype} mode={mode}")
        out, lse = _run(mb, budget, mode, dc)
        _cmp(out, lse, ro, rl, np.arange(ro.shape[0]), tol)


def _set_token(cache, blk, off, h, kvec_codes, vvec_codes):
    """Write one token's K and V (already in the cache's element type) at
    (block, offset, head) by the layout formulas."""
    sp = cache.spec
    if sp.layout == "nhd":
        cache.k[blk, off, h] = kvec_codes
        cache.v[blk, off, h] = vvec_codes
    else:
        x = sp.x
        d = np.arange(sp.head_dim)
        cache.k[blk, h, d // x, off, d % x] = kvec_codes
        cache.v[blk, h, off // x, d, off % x] = vvec_codes


def _codes(cache, vals, scale):
    if cache.spec.dtype == "bf16":
        return w.f32_to_bf16_bits(vals.astype(np.float32))
    import torch as t
    return t.from_numpy((vals / scale).astype(np.float32)).to(t.float8_e4m3fn).view(t.uint8).numpy()


@pytest.mark.parametrize("layout,dtype", KINDS)
def test_extend_needle_long_context_other_caches(layout, dtype):
    """2 x (100000 cached + 256 new), 8:1 heads, the context on the other
    caches: one needle key in a random block deep in each request's context;
    64 query rows per request point at it (score ~48 against ~N(0, 9) for the
    rest), so their exact output is the needle's value row -- a block read
    from the wrong place moves them by O(1).  Both executions against the
    oracle on those rows."""
    ctx, new = 100000, 256
    mb = w.mixed_batch(53, 8, 1, 128, 16, 2 * ((ctx + new) // 16 + 2) + 8, [], [ctx] * 2,
                       [new] * 2, [], layout=layout, dtype=dtype)
    rng = np.random.default_rng(53)
    D = 128
    needles = []
    for e in range(2):
        tok = int(rng.integers(50000, ctx))
        blk, off = int(mb.ext_tables[e, tok // 16]), tok % 16
        u = rng.standard_normal(D)
        u /= np.linalg.norm(u)
        kvals = 4.5 * u / np.abs(u).max()                 # representable in every cache
        vvals = 3.0 * np.tanh(rng.standard_normal(D))
        _set_token(mb.cache, blk, off, 0, _codes(mb.cache, kvals, mb.cache.k_scale),
                   _codes(mb.cache, vvals, mb.cache.v_scale))
        rows = int(mb.ext_cu_q[e]) + rng.choice(new, 64, replace=False)
        for r in rows:
            for h in range(8):
                qv = 3.0 * np.sqrt(D) * u + 0.1 * rng.standard_normal(D)
                mb.q[r, h] = w.f32_to_bf16_bits(qv.astype(np.float32))
        needles.append(rows)
        say(f"  needle of request {e} at token {tok} (block {blk}, offset {off})")
    tol = BF16_TOL if dtype == "bf16" else FP8_TOL
    dc = device_cache(mb.cache)
    rows = np.concatenate(needles)
    ro, rl = _oracle(mb, list(rows))
    for mode in ("split", "fused"):
        say(f"extend needle 2x(100000+256) 8:1 {layout} {dtype} mode={mode}")
        out, lse = _run(mb, 32768, mode, dc)
        _cmp(out, lse, ro, rl, rows, tol)
    # the test is sensitive: the exact output of those rows is the needle's V
    for e, rs in enumerate(needles):
        assert np.std(ro[rs].reshape(-1, D), axis=0).max() < 0.05
