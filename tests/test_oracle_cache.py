"""Pins for the oracle's cache write, pack/unpack and the layout fixtures
(CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import bf16, cache as oc, fp8
from synth import workloads as w

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cache(rng, nb, bs, H, D, layout="nhd", dtype="bf16"):
    spec = w.CacheSpec(nb, bs, H, D, layout, dtype)
    cd = w.random_cache(rng, spec)
    return oc.Cache(cd.k, cd.v, layout, dtype, bs, H, D, spec.x, cd.k_scale, cd.v_scale)


def test_kv_bytes_per_token_golden():
    g = json.load(open(os.path.join(GOLD, "kv_bytes_per_token.json")))
    s = g["shape_reading"]
    rng = np.random.default_rng(0)
    c = _cache(rng, 4, s["block_size"], s["num_kv_heads"], s["head_dim"])
    n_blocks = 3
    per_layer_per_token = oc.packed_bytes(c, n_blocks) / (n_blocks * s["block_size"])
    per_token = per_layer_per_token * s["layers"]
    assert per_token == g["printed"]["kib_per_token"] * 1024
    total = per_token * g["printed"]["prompt_tokens"]
    assert abs(total / 1e9 - g["printed"]["approx_transfer_gb"]) / g["printed"]["approx_transfer_gb"] < 0.1
    # the full-size layer pack of 8 requests x 10000 tokens: 5000 blocks
    assert oc.packed_bytes(c, 8 * 10000 // 16) == 327_680_000


def test_preshuffled_layout_golden():
    g = json.load(open(os.path.join(GOLD, "preshuffled_layout.json")))
    nb, H, D, bs = 3, 4, 128, 16
    for dtype, x in (("fp8", 16), ("bf16", 8)):
        spec = w.CacheSpec(nb, bs, H, D, "preshuffled", dtype)
        env = {"num_blocks": nb, "num_heads": H, "head_dim": D, "block_size": bs, "x": x}
        want_k = tuple(eval(e, {}, env) for e in g["k_cache"])
        want_v = tuple(eval(e, {}, env) for e in g["v_cache"])
        assert spec.x == x and spec.shapes() == (want_k, want_v)


@pytest.mark.parametrize("layout,dtype", [("nhd", "bf16"), ("preshuffled", "bf16"),
                                          ("preshuffled", "fp8"), ("nhd", "fp8")])
def test_write_then_gather_returns_written_tokens(layout, dtype):
    rng = np.random.default_rng(4)
    H, D, bs, nb = 2, 32, 16, 12
    c = _cache(rng, nb, bs, H, D, layout, dtype)
    table = rng.permutation(nb)[:5]
    T = 7
    pos = np.array([0, 15, 16, 33, 40, 63, 79])
    slots = table[pos // bs] * bs + pos % bs
    slots_pad = np.concatenate([slots[:3], [-1], slots[3:]])
    kb = w.normal_bf16(rng, (T + 1, H, D))
    vb = w.normal_bf16(rng, (T + 1, H, D))
    c2 = oc.write(c, kb, vb, slots_pad)
    kb = np.delete(kb, 3, axis=0)
    vb = np.delete(vb, 3, axis=0)
    K, V = oc.gather(c2, table, 80)
    if dtype == "bf16":
        assert np.array_equal(K[pos], bf16.to_f64(kb)) and np.array_equal(V[pos], bf16.to_f64(vb))
    else:
        # dequantised codes are within half an fp8 step of the written values
        # (the exact bytes are pinned by test_fp8_write_bytes_exact)
        kx = bf16.to_f64(kb)
        rel = np.abs(K[pos] - kx) / np.maximum(np.abs(kx), 2.0 ** -6 * c.k_scale)
        assert rel.max() <= 2.0 ** -4 + 1e-12
    # untouched tokens are unchanged
    K0, V0 = oc.gather(c, table, 80)
    other = np.setdiff1d(np.arange(80), pos)
    assert np.array_equal(K0[other], K[other]) and np.array_equal(V0[other], V[other])


def test_negative_slots_write_nothing():
    rng = np.random.default_rng(5)
    c = _cache(rng, 4, 16, 2, 32)
    kb = w.normal_bf16(rng, (3, 2, 32))
    c2 = oc.write(c, kb, kb, [-1, -5, -1])
    assert np.array_equal(c.k, c2.k) and np.array_equal(c.v, c2.v)


@pytest.mark.parametrize("layout,dtype", [("nhd", "bf16"), ("preshuffled", "fp8")])
def test_pack_unpack(layout, dtype):
    rng = np.random.default_rng(6)
    H, D, bs, nb = 2, 32, 16, 20
    c = _cache(rng, nb, bs, H, D, layout, dtype)
    ids = rng.permutation(nb)[:7]
    buf = oc.pack_layer(c, ids)
    assert buf.size == oc.packed_bytes(c, 7)
    # built independently: append each block's K bytes, then each block's V
    parts = [c.k[i].tobytes() for i in ids] + [c.v[i].tobytes() for i in ids]
    assert buf.tobytes() == b"".join(parts)
    # unpack into other blocks of an empty cache: those blocks now equal the
    # source blocks, nothing else changed
    dst = oc.Cache(np.zeros_like(c.k), np.zeros_like(c.v), layout, dtype, bs, H, D,
                   c.x, c.k_scale, c.v_scale)
    dst_ids = rng.permutation(nb)[:7]
    d2 = oc.unpack_layer(dst, dst_ids, buf)
    assert np.array_equal(d2.k[dst_ids], c.k[ids]) and np.array_equal(d2.v[dst_ids], c.v[ids])
    rest = np.setdiff1d(np.arange(nb), dst_ids)
    assert not d2.k[rest].any() and not d2.v[rest].any()
    # round trip in place
    c3 = oc.unpack_layer(c, ids, buf)
    assert np.array_equal(c3.k, c.k) and np.array_equal(c3.v, c.v)


@pytest.mark.parametrize("layout", ["nhd", "preshuffled"])
def test_fp8_write_bytes_exact(layout):
    """The quantising write, byte for byte, against a cache image built
    independently: each code is torch's float8_e4m3fn cast of the fp32 product
    fl32(x) * fl32(1/scale) (a library conversion the oracle does not call),
    and each code is placed by the layout formulas element by element:
    NHD k[blk, off, h, d]; preshuffled k[blk, h, d // 16, off, d % 16] and
    v[blk, h, off // 16, d, off % 16].  K and V use different scales (a factor
    of 37 apart), so swapping them, or misplacing an element, changes bytes."""
    import torch
    rng = np.random.default_rng(17)
    H, D, bs, nb, x = 2, 32, 16, 6, 16
    k_scale, v_scale = 0.37, 0.01
    if layout == "nhd":
        kshape = vshape = (nb, bs, H, D)
    else:
        kshape, vshape = (nb, H, D // x, bs, x), (nb, H, bs // x, D, x)
    k0 = rng.integers(0, 256, size=kshape, dtype=np.uint8) & 0x77      # finite codes
    v0 = rng.integers(0, 256, size=vshape, dtype=np.uint8) & 0x77
    c = oc.Cache(k0, v0, layout, "fp8", bs, H, D, x if layout != "nhd" else 0, k_scale, v_scale)
    T = 9
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[4] = -1                                                     # padding token
    # values spread over the whole code range, kept below 448 * scale
    kb = w.f32_to_bf16_bits((rng.standard_normal((T, H, D)) * 40.0 * k_scale).astype(np.float32))
    vb = w.f32_to_bf16_bits((rng.standard_normal((T, H, D)) * 40.0 * v_scale).astype(np.float32))

    def codes(bits, scale):
        f = (bits.astype(np.uint32) << 16).view(np.float32)
        y = f * (np.float32(1.0) / np.float32(scale))                  # fp32 product
        assert np.all(np.abs(y) < 448)
        return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn) \
            .view(torch.uint8).numpy()

    kc, vc = codes(kb, k_scale), codes(vb, v_scale)
    want_k, want_v = k0.copy(), v0.copy()
    for i in range(T):
        s_ = int(slots[i])
        if s_ < 0:
            continue
        blk, off = s_ // bs, s_ % bs
        for h in range(H):
            for d in range(D):
                if layout == "nhd":
                    want_k[blk, off, h, d] = kc[i, h, d]
                    want_v[blk, off, h, d] = vc[i, h, d]
                else:
                    want_k[blk, h, d // x, off, d % x] = kc[i, h, d]
                    want_v[blk, h, off // x, d, off % x] = vc[i, h, d]
    got = oc.write(c, kb, vb, slots)
    assert got.k.tobytes() == want_k.tobytes()
    assert got.v.tobytes() == want_v.tobytes()
    # the planted mistakes this pin exists for change bytes
    swapped = oc.write(oc.Cache(k0, v0, layout, "fp8", bs, H, D, c.x, v_scale, k_scale),
                       kb, vb, slots)
    assert swapped.k.tobytes() != want_k.tobytes()
