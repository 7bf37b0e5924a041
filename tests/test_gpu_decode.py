"""GPU parity: paged decode against the oracle (bf16 outputs within 1.5e-2,
fp8-KV outputs within 5e-2, lse within 1e-3), plus poison, needle,
split-invariance and determinism checks."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import attention as oa, bf16 as ob, cache as oc, fp8 as of8
from synth import workloads as w

from .gpu_util import (BF16_TOL, FP8_TOL, LSE_TOL, bf16_to_f64, dev, device_cache, max_err,
                       oracle_cache, say, torch)

pytestmark = pytest.mark.gpu


def _run(dc, st, split=0, max_seq_len=None):
    msl = int(st.seq_lens.max()) if max_seq_len is None else max_seq_len
    out, lse = pk.paged_decode(dc, dev(st.q), dev(st.block_tables), dev(st.seq_lens), msl,
                               st.scale, split_tokens=split)
    torch().cuda.synchronize()
    return bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)


def _check(st, ocache, out, lse, tol, rows=None):
    rows = range(st.batch) if rows is None else rows
    q = ob.to_f64(st.q)
    worst = [0.0, 0.0]
    for b in rows:
        ro, rl = oa.paged_decode(q[b:b + 1], ocache, st.block_tables[b:b + 1], st.seq_lens[b:b + 1],
                                 st.scale)
        e = max_err(out[b], ro[0])
        el = max_err(lse[b], rl[0])
        assert e <= tol, (b, e)
        assert el <= LSE_TOL, (b, el)
        worst = [max(worst[0], e), max(worst[1], el)]
    say(f"  max|err| out {worst[0]:.3e} lse {worst[1]:.3e} over {len(list(rows))} requests")


def test_tiny_decode_eight_steps():
    """Batch 4, 8:2 heads, lengths in [100, 512]: eight steps of write-then-decode."""
    st = w.tiny_decode()
    rng = np.random.default_rng(101)
    dc = device_cache(st.cache)
    ocache = oracle_cache(st.cache)
    for step in range(8):
        say(f"tiny decode step {step} lens={st.seq_lens.tolist()}")
        pk.kv_write(dc, dev(st.k_new), dev(st.v_new), dev(st.slot_mapping))
        ocache = oc.write(ocache, st.k_new, st.v_new, st.slot_mapping)
        out, lse = _run(dc, st)
        _check(st, ocache, out, lse, BF16_TOL)
        st = w.next_decode_step(rng, st)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 1), (32, 2), (40, 2), (12, 4)])
@pytest.mark.parametrize("layout,dtype", [("nhd", "bf16"), ("nhd", "fp8"),
                                          ("preshuffled", "bf16"), ("preshuffled", "fp8")])
def test_decode_shapes_and_layouts(Hq, Hkv, layout, dtype):
    st = w.decode_workload(5, 6, Hq, Hkv, 128, 16, 400, 1, 700, layout=layout, dtype=dtype,
                           fixed_lens=[1, 15, 16, 33])  # edge lengths
    w.poison_cache(st.cache, st.block_tables, st.seq_lens)
    say(f"decode {layout} {dtype} {Hq}:{Hkv} lens={st.seq_lens.tolist()}")
    dc = device_cache(st.cache)
    tol = BF16_TOL if dtype == "bf16" else FP8_TOL
    out, lse = _run(dc, st)
    _check(st, oracle_cache(st.cache), out, lse, tol)


@pytest.mark.parametrize("bs", [1, 4, 32, 64])
def test_decode_block_sizes(bs):
    st = w.decode_workload(6, 5, 16, 2, 128, bs, 5 * 900 // bs + 64, 1, 900)
    w.poison_cache(st.cache, st.block_tables, st.seq_lens)
    say(f"decode bs={bs}")
    out, lse = _run(device_cache(st.cache), st)
    _check(st, oracle_cache(st.cache), out, lse, BF16_TOL)


@pytest.mark.parametrize("layout,dtype,bs", [("preshuffled", "bf16", 8), ("preshuffled", "bf16", 16),
                                             ("preshuffled", "bf16", 64), ("preshuffled", "fp8", 16),
                                             ("preshuffled", "fp8", 32), ("preshuffled", "fp8", 64),
                                             ("nhd", "fp8", 1), ("nhd", "fp8", 8), ("nhd", "fp8", 64)])
def test_decode_block_sizes_by_layout(layout, dtype, bs):
    """Tiles of 32 tokens over blocks of 8 to 64 tokens in every cache kind:
    the K rows of a tile come from one or several blocks, and lengths end
    inside a block, inside a tile half and on tile boundaries."""
    lens = [1, 7, 8, 15, 16, 17, 31, 32, 33, 47, 63, 64, 65, 200, 513]
    nb = sum(-(-n // bs) for n in lens) + 64
    st = w.decode_workload(12, len(lens), 16, 2, 128, bs, nb, 1, 600, layout=layout, dtype=dtype,
                           fixed_lens=lens)
    w.poison_cache(st.cache, st.block_tables, st.seq_lens)
    say(f"decode {layout} {dtype} bs={bs} lens={st.seq_lens.tolist()}")
    out, lse = _run(device_cache(st.cache), st)
    _check(st, oracle_cache(st.cache), out, lse, BF16_TOL if dtype == "bf16" else FP8_TOL)


def test_decode_split_invariance_and_determinism():
    st = w.decode_workload(8, 4, 32, 4, 128, 16, 600, 1500, 2200)
    dc = device_cache(st.cache)
    ocache = oracle_cache(st.cache)
    ref = None
    for split in (0, 128, 256, 1024, 4096):
        say(f"decode split={split}")
        out, lse = _run(dc, st, split)
        _check(st, ocache, out, lse, BF16_TOL)
        out2, lse2 = _run(dc, st, split)
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2)   # deterministic
        if ref is not None:
            assert max_err(out, ref[0]) <= 2 * BF16_TOL and max_err(lse, ref[1]) <= LSE_TOL
        ref = (out, lse)


@pytest.mark.parametrize("batch", [2048, 2300])
def test_decode_large_batch_plans(batch):
    """Batches of up to 2048 requests are planned by every workgroup in its own
    LDS, larger ones by the separate planning kernel; both agree with the
    oracle (short, skewed lengths: many requests per piece)."""
    st = w.decode_workload(12, batch, 8, 2, 128, 16, batch * 9 + 64, 1, 120,
                           fixed_lens=[1, 2, 120, 31, 32, 33])
    w.poison_cache(st.cache, st.block_tables, st.seq_lens)
    say(f"decode batch={batch}")
    dc = device_cache(st.cache)
    out, lse = _run(dc, st)
    rows = list(range(8)) + list(np.random.default_rng(3).choice(batch, 200, replace=False))
    rows += [batch - 1]
    _check(st, oracle_cache(st.cache), out, lse, BF16_TOL, rows)
    out_s, lse_s = _run(dc, st, split=64)     # many pieces per request
    _check(st, oracle_cache(st.cache), out_s, lse_s, BF16_TOL, rows)


def test_decode_workspace_reuse_with_stale_contents():
    """The plan and the partial slots live in the caller's workspace: calls of
    different shapes on one workspace that starts out as random bytes must each
    produce the oracle's result, and repeated calls bit-identical ones."""
    t = torch()
    big = w.decode_workload(13, 24, 32, 4, 128, 16, 24 * 260 + 64, 500, 4000)
    small = w.decode_workload(14, 5, 16, 2, 128, 16, 5 * 80 + 64, 300, 1200)
    dcb, dcs = device_cache(big.cache), device_cache(small.cache)
    need = max(pk.paged_decode_workspace_bytes(dcb, 24, 32, int(big.seq_lens.max()), 128),
               pk.paged_decode_workspace_bytes(dcs, 5, 16, int(small.seq_lens.max()), 128))
    ws = t.randint(0, 256, (need,), dtype=t.uint8, device="cuda")
    say("decode workspace reuse")

    def run(dc, st, split):
        out, lse = pk.paged_decode(dc, dev(st.q), dev(st.block_tables), dev(st.seq_lens),
                                   int(st.seq_lens.max()), st.scale, workspace=ws,
                                   split_tokens=split)
        t.cuda.synchronize()
        return bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)

    ob_, os_ = oracle_cache(big.cache), oracle_cache(small.cache)
    first = run(dcb, big, 128)
    _check(big, ob_, *first, BF16_TOL)
    for split in (128, 0, 256):
        o, l = run(dcs, small, split)
        _check(small, os_, o, l, BF16_TOL)
    again = run(dcb, big, 128)
    assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


def test_decode_needle():
    """One planted key with a dominant score: the output must be its value row
    (catches a mis-gathered block, which random data would hide)."""
    st = w.decode_workload(9, 4, 8, 2, 128, 16, 700, 1000, 2500)
    rng = np.random.default_rng(9)
    k = st.cache.k
    for b in range(st.batch):
        L = int(st.seq_lens[b])
        t = int(rng.integers(0, L))
        blk, off = st.block_tables[b, t // 16], t % 16
        for g in range(2):
            qsum = ob.to_f64(st.q[b, 4 * g:4 * g + 4]).sum(0)
            needle = 3.0 * qsum / np.linalg.norm(qsum) * np.sqrt(128)
            k[blk, off, g] = w.f32_to_bf16_bits(needle.astype(np.float32))
    say("decode needle")
    out, lse = _run(device_cache(st.cache), st)
    _check(st, oracle_cache(st.cache), out, lse, BF16_TOL)


def test_decode_llama70b_full_size():
    """Batch 64, 64:8 heads, lengths in [2048, 8192], 32768 blocks: every
    request checked against the oracle."""
    st = w.llama70b_decode_layer()
    say("decode llama70b full size")
    dc = device_cache(st.cache)
    pk.kv_write(dc, dev(st.k_new), dev(st.v_new), dev(st.slot_mapping))
    ocache = oc.write(oracle_cache(st.cache), st.k_new, st.v_new, st.slot_mapping)
    out, lse = _run(dc, st)
    assert not np.isnan(out).any()
    _check(st, ocache, out, lse, BF16_TOL)


def test_decode_fp8_preshuffled_full_size():
    """Batch 128, 64:4 heads, lengths in [1000, 16000], fp8 e4m3 preshuffled
    (x = 16), 131072 blocks: every request checked against the oracle."""
    st = w.fp8_preshuffled_decode()
    say("decode fp8 preshuffled full size")
    dc = device_cache(st.cache)
    pk.kv_write(dc, dev(st.k_new), dev(st.v_new), dev(st.slot_mapping))
    ocache = oc.write(oracle_cache(st.cache), st.k_new, st.v_new, st.slot_mapping)
    out, lse = _run(dc, st)
    assert not np.isnan(out).any()
    _check(st, ocache, out, lse, FP8_TOL)


@pytest.mark.parametrize("split", [0, 64])
def test_decode_empty_requests(split):
    """Requests of length 0 see no key: out = 0 and lse = -inf (the output
    buffer starts as NaN, so an unwritten row shows).  Their neighbours, in
    the same pieces, are unaffected."""
    t = torch()
    st = w.decode_workload(15, 9, 16, 2, 128, 16, 9 * 40 + 64, 100, 600)
    lens = st.seq_lens.copy()
    lens[[0, 4, 5, 8]] = 0
    st.seq_lens = lens
    say(f"decode with empty requests split={split} lens={lens.tolist()}")
    dc = device_cache(st.cache)
    out = t.full((st.batch, 16, 128), float("nan"), dtype=t.bfloat16, device="cuda")
    lse = t.full((st.batch, 16), float("nan"), dtype=t.float32, device="cuda")
    pk.paged_decode(dc, dev(st.q), dev(st.block_tables), dev(st.seq_lens), int(lens.max()), st.scale,
                    out=out, lse=lse, split_tokens=split)
    t.cuda.synchronize()
    o, l = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
    empty = lens == 0
    assert (o[empty] == 0).all() and np.isneginf(l[empty]).all()
    _check(st, oracle_cache(st.cache), o, l, BF16_TOL, rows=list(np.flatnonzero(~empty)))
    ro, rl = oa.paged_decode(ob.to_f64(st.q[empty]), oracle_cache(st.cache),
                             st.block_tables[empty], lens[empty], st.scale)
    assert (ro == 0).all() and np.isneginf(rl).all()        # the oracle's reading agrees


@pytest.mark.parametrize("layout", ["nhd", "preshuffled"])
def test_decode_fp8_every_code(layout):
    """Every e4m3fn code through the decode's fp8 read: two requests of one
    token each, whose V rows carry codes 0..127 and 128..255 (the two NaN
    codes replaced by 0).  With one key the softmax weight is exactly 1, so
    with unit scales the output is each code's value, bit for bit (every
    e4m3fn value is a bf16 value).  The cache is placed by the oracle's
    write of those values, which round-trips them to the same codes."""
    st = w.decode_workload(16, 2, 4, 2, 128, 16, 64, 1, 1, layout=layout, dtype="fp8",
                           fixed_lens=[1, 1])
    codes = np.arange(256).astype(np.uint8).reshape(2, 128)
    codes[(codes & 0x7F) == 0x7F] = 0
    vals = of8.decode(codes)
    vbits = w.f32_to_bf16_bits(vals.astype(np.float32))
    v_new = np.ascontiguousarray(np.broadcast_to(vbits[:, None, :], (2, 2, 128)))
    sp = st.cache.spec
    base = oc.Cache(st.cache.k, st.cache.v, sp.layout, sp.dtype, sp.block_size, sp.num_kv_heads,
                    sp.head_dim, sp.x, 1.0, 1.0)
    ocache = oc.write(base, st.k_new, v_new, st.slot_mapping)
    dc = pk.PagedKVCache(dev(ocache.k), dev(ocache.v), sp.block_size, sp.num_kv_heads,
                         sp.head_dim, sp.layout, sp.dtype, 1.0, 1.0)
    say(f"decode fp8 every code {layout}")
    out, lse = _run(dc, st)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], vals[b]), (b, h)
    ro, rl = oa.paged_decode(ob.to_f64(st.q), ocache, st.block_tables, st.seq_lens, st.scale)
    assert np.array_equal(ro, np.broadcast_to(vals[:, None, :], ro.shape))   # the oracle agrees
    assert max_err(lse, rl) <= LSE_TOL
