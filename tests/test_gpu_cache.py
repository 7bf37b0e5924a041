"""GPU parity: slot-mapped cache write and layer pack/unpack against the oracle,
bit-exact."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import cache as oc, fp8 as ofp8
from synth import workloads as w

from .gpu_util import dev, device_cache, host_bits, oracle_cache, say, torch

pytestmark = pytest.mark.gpu


def _write_case(seed, spec, T, pad_every=0):
    rng = np.random.default_rng(seed)
    cd = w.random_cache(rng, spec)
    nslots = spec.num_blocks * spec.block_size
    slots = rng.permutation(nslots)[:T].astype(np.int64)
    if pad_every:
        slots[::pad_every] = -1
    k = w.normal_bf16(rng, (T, spec.num_kv_heads, spec.head_dim))
    v = w.normal_bf16(rng, (T, spec.num_kv_heads, spec.head_dim))
    return cd, k, v, slots


@pytest.mark.parametrize("layout,dtype", [("nhd", "bf16"), ("nhd", "fp8"),
                                          ("preshuffled", "bf16"), ("preshuffled", "fp8")])
@pytest.mark.parametrize("bs", [16, 32])
def test_kv_write_bit_exact(layout, dtype, bs):
    spec = w.CacheSpec(96, bs, 4, 128, layout, dtype)
    cd, k, v, slots = _write_case(7, spec, 300, pad_every=7)
    say(f"kv_write {layout} {dtype} bs={bs} T=300")
    dc = device_cache(cd)
    pk.kv_write(dc, dev(k), dev(v), dev(slots))
    torch().cuda.synchronize()
    ref = oc.write(oracle_cache(cd), k, v, slots)
    assert np.array_equal(host_bits(dc.k), ref.k)
    assert np.array_equal(host_bits(dc.v), ref.v)


def test_kv_write_mixed_batch_rows():
    """All 6096 new rows of the Qwen3-shaped mixed batch (64:4 heads)."""
    mb = w.qwen3_mixed_batch()
    say("kv_write qwen3 mixed batch T=6096")
    dc = device_cache(mb.cache)
    pk.kv_write(dc, dev(mb.k_new), dev(mb.v_new), dev(mb.slot_mapping))
    torch().cuda.synchronize()
    ref = oc.write(oracle_cache(mb.cache), mb.k_new, mb.v_new, mb.slot_mapping)
    assert np.array_equal(host_bits(dc.k), ref.k) and np.array_equal(host_bits(dc.v), ref.v)


def test_kv_write_zero_tokens_is_noop():
    spec = w.CacheSpec(8, 16, 2, 128)
    cd, k, v, slots = _write_case(1, spec, 4)
    dc = device_cache(cd)
    t = torch()
    pk.kv_write(dc, dev(k)[:0], dev(v)[:0], dev(slots)[:0])
    t.cuda.synchronize()
    assert np.array_equal(host_bits(dc.k), cd.k)


@pytest.mark.parametrize("scale", [1.0, 0.0136, 0.37, 3.0])
def test_fp8_store_exhaustive_over_bf16(scale):
    """Every finite bf16 value through the quantising store, NHD and
    preshuffled, against the oracle's nearest-value encoder."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    bits = np.where(np.isnan(f), 0, bits).astype(np.uint16)        # finite inputs + inf
    H, D = 4, 128
    T = bits.size // (H * D)
    k = bits.reshape(T, H, D)
    v = k[::-1].copy()
    for layout in ("nhd", "preshuffled"):
        spec = w.CacheSpec(T // 16, 16, H, D, layout, "fp8")
        kc = np.zeros(spec.shapes()[0], np.uint8)
        vc = np.zeros(spec.shapes()[1], np.uint8)
        cd = w.CacheData(spec, kc, vc, scale, scale * 0.5)
        slots = np.arange(T, dtype=np.int64)
        say(f"fp8 exhaustive {layout} scale={scale}")
        dc = device_cache(cd)
        pk.kv_write(dc, dev(k), dev(v), dev(slots))
        torch().cuda.synchronize()
        ref = oc.write(oracle_cache(cd), k, v, slots)
        assert np.array_equal(host_bits(dc.k), ref.k), layout
        assert np.array_equal(host_bits(dc.v), ref.v), layout
    # sanity: the oracle path really is the codec under test
    assert ofp8.quantize(np.float32(1.0), 1.0) == 0x38


def _pack_roundtrip(cd, job):
    dc = device_cache(cd)
    src = dev(job.src_ids)
    buf = pk.kv_pack_layer(dc, src)
    torch().cuda.synchronize()
    ocache = oracle_cache(cd)
    want = oc.pack_layer(ocache, job.src_ids)
    got = host_bits(buf)
    assert got.size == want.size and np.array_equal(got, want)
    # unpack into a second (zeroed) cache at other ids
    t = torch()
    dst = pk.PagedKVCache(t.zeros_like(dc.k), t.zeros_like(dc.v), dc.block_size, dc.num_kv_heads,
                          dc.head_dim, dc.layout, dc.dtype, dc.k_scale, dc.v_scale)
    pk.kv_unpack_layer(dst, dev(job.dst_ids), buf)
    t.cuda.synchronize()
    empty = oc.Cache(np.zeros_like(cd.k), np.zeros_like(cd.v), ocache.layout, ocache.dtype,
                     ocache.block_size, ocache.num_kv_heads, ocache.head_dim, ocache.x)
    ref = oc.unpack_layer(empty, job.dst_ids, want)
    assert np.array_equal(host_bits(dst.k), ref.k) and np.array_equal(host_bits(dst.v), ref.v)


@pytest.mark.parametrize("layout,dtype", [("nhd", "bf16"), ("preshuffled", "fp8"), ("nhd", "fp8")])
def test_pack_unpack_small(layout, dtype):
    rng = np.random.default_rng(3)
    spec = w.CacheSpec(300, 16, 4, 128, layout, dtype)
    cd = w.random_cache(rng, spec)
    job = w.pack_job(3, 300, num_seqs=3, tokens_per_seq=1000)
    say(f"pack/unpack {layout} {dtype} n={job.src_ids.size}")
    _pack_roundtrip(cd, job)


def test_pack_unpack_llama70b_layer_full():
    """8 requests x 10000 tokens = 5000 blocks of a 32768-block Llama-3.1-70B
    layer (327,680,000 packed bytes)."""
    rng = np.random.default_rng(2)
    spec = w.CacheSpec(32768, 16, 8, 128)
    cd = w.random_cache(rng, spec)
    job = w.pack_job(2, 32768)
    assert job.src_ids.size == 5000
    say("pack/unpack llama70b layer 5000 blocks")
    _pack_roundtrip(cd, job)
