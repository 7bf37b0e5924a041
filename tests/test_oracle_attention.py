"""Pins for the oracle's attention, gather and merge (CPU only).

Each check is fixed by something other than the oracle's own formula:
* torch's scaled_dot_product_attention (a library routine the oracle does not
  call), float64 on the CPU, with KV heads repeated per query group and an
  explicit boolean mask for the causal / bottom-right extend cases;
* closed forms: one key, zero query, identical keys, a planted needle;
* invariants: relabelling physical blocks (block-table permutation) leaves the
  output bitwise unchanged; a two-chunk LSE merge equals the full softmax;
  extend with no cached context equals causal prefill; extend of one new
  token equals decode over C + 1 tokens;
* the gather is checked against a cache built by copying a known logical
  sequence into its blocks one block at a time.
"""
import math

import numpy as np
import pytest

from oracle import attention, bf16, cache as oc, merge
from synth import workloads as w


def _rand_cache(rng, nb, bs, H, D, layout="nhd", dtype="bf16"):
    spec = w.CacheSpec(nb, bs, H, D, layout, dtype)
    cd = w.random_cache(rng, spec)
    return oc.Cache(cd.k, cd.v, layout, dtype, bs, H, D, spec.x, cd.k_scale, cd.v_scale)


def _sdpa(q, k, v, scale, mask=None):
    """torch SDPA in float64; q [n, Hq, D], k/v [m, Hkv, D]."""
    torch = pytest.importorskip("torch")
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(np.repeat(k, G, axis=1).transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(np.repeat(v, G, axis=1).transpose(1, 0, 2)))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.numpy().transpose(1, 0, 2)


# ---------------------------------------------------------------- gather
@pytest.mark.parametrize("layout,dtype,bs", [("nhd", "bf16", 16), ("nhd", "bf16", 1),
                                             ("nhd", "bf16", 4), ("preshuffled", "bf16", 16),
                                             ("preshuffled", "fp8", 16), ("preshuffled", "fp8", 32)])
def test_gather_recovers_scattered_sequence(layout, dtype, bs):
    rng = np.random.default_rng(11)
    H, D, L = 2, 32, 53
    nb = (L + bs - 1) // bs + 4
    c = _rand_cache(rng, nb, bs, H, D, layout, dtype)
    x = 16 // (1 if dtype == "fp8" else 2)
    nblk = (L + bs - 1) // bs
    table = rng.permutation(nb)[:nblk]
    # a known logical sequence of raw element codes
    if dtype == "bf16":
        seqk = w.normal_bf16(rng, (L, H, D))
        seqv = w.normal_bf16(rng, (L, H, D))
    else:
        seqk = rng.integers(0, 0x7E, size=(L, H, D)).astype(np.uint8)
        seqv = rng.integers(0, 0x7E, size=(L, H, D)).astype(np.uint8)
    # copy it in block by block, element by element, straight from the layout
    # formulas of the page
    for i in range(nblk):
        blk = table[i]
        for off in range(bs):
            t = i * bs + off
            if t >= L:
                break
            for h in range(H):
                for d in range(D):
                    if layout == "nhd":
                        c.k[blk, off, h, d] = seqk[t, h, d]
                        c.v[blk, off, h, d] = seqv[t, h, d]
                    else:
                        c.k[blk, h, d // x, off, d % x] = seqk[t, h, d]
                        c.v[blk, h, off // x, d, off % x] = seqv[t, h, d]
    K, V = oc.gather(c, table, L)
    if dtype == "bf16":
        assert np.array_equal(K, bf16.to_f64(seqk)) and np.array_equal(V, bf16.to_f64(seqv))
    else:
        from oracle import fp8
        assert np.array_equal(K, fp8.decode(seqk) * np.float32(c.k_scale))
        assert np.array_equal(V, fp8.decode(seqv) * np.float32(c.v_scale))


def test_preshuffled_index_map_is_a_bijection():
    nb, H, D, bs, x = 1, 2, 32, 16, 16
    kc = np.full((nb, H, D // x, bs, x), -1, dtype=np.int64)
    vc = np.full((nb, H, bs // x, D, x), -1, dtype=np.int64)
    n = 0
    for t in range(bs):
        for h in range(H):
            for d in range(D):
                assert kc[0, h, d // x, t, d % x] == -1
                assert vc[0, h, t // x, d, t % x] == -1
                kc[0, h, d // x, t, d % x] = n
                vc[0, h, t // x, d, t % x] = n
                n += 1
    assert (kc >= 0).all() and (vc >= 0).all()


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (16, 1)])
@pytest.mark.parametrize("layout,dtype", [("nhd", "bf16"), ("preshuffled", "fp8")])
def test_decode_matches_sdpa(Hq, Hkv, layout, dtype):
    rng = np.random.default_rng(3)
    D, bs, nb, B = 32, 16, 40, 3
    c = _rand_cache(rng, nb, bs, Hkv, D, layout, dtype)
    lens = np.array([1, 17, 100])
    tables = np.full((B, 8), nb - 1)
    perm = rng.permutation(nb - 1)
    s = 0
    for b, L in enumerate(lens):
        n = (L + bs - 1) // bs
        tables[b, :n] = perm[s:s + n]
        s += n
    q = bf16.to_f64(w.normal_bf16(rng, (B, Hq, D)))
    scale = 1 / math.sqrt(D)
    out, lse = attention.paged_decode(q, c, tables, lens, scale)
    for b in range(B):
        K, V = oc.gather(c, tables[b], lens[b])
        ref = _sdpa(q[b][None], K, V, scale)[0]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(5)
    D = 16
    K = rng.standard_normal((9, D))
    V = rng.standard_normal((9, D))
    q = rng.standard_normal((1, D))
    sc = 0.3
    # one key: o = v0, lse = s0
    o, l = attention.attend(q, K[:1], V[:1], sc)
    assert np.allclose(o[0], V[0], atol=1e-15) and abs(l[0] - sc * q[0] @ K[0]) < 1e-14
    # zero query: uniform weights, o = mean(V), lse = ln L
    o, l = attention.attend(np.zeros((1, D)), K, V, sc)
    assert np.allclose(o[0], V.mean(0), atol=1e-14) and abs(l[0] - math.log(9)) < 1e-14
    # identical keys: lse = s + ln L, o = mean(V)
    Ks = np.repeat(K[:1], 9, axis=0)
    o, l = attention.attend(q, Ks, V, sc)
    assert abs(l[0] - (sc * q[0] @ K[0] + math.log(9))) < 1e-13
    assert np.allclose(o[0], V.mean(0), atol=1e-14)
    # needle: one key with a dominant score
    Kn = K.copy()
    Kn[6] = 60.0 * q[0] / np.linalg.norm(q[0])
    o, l = attention.attend(q, Kn, V, 1.0)
    assert np.allclose(o[0], V[6], atol=1e-12)


def test_block_relabelling_is_bitwise_invariant():
    rng = np.random.default_rng(9)
    Hq, Hkv, D, bs, nb, B = 8, 2, 32, 4, 64, 3
    c = _rand_cache(rng, nb, bs, Hkv, D)
    lens = np.array([5, 33, 60])
    tables = np.zeros((B, 16), dtype=np.int64)
    perm = rng.permutation(nb)
    s = 0
    for b, L in enumerate(lens):
        n = (L + bs - 1) // bs
        tables[b, :n] = perm[s:s + n]
        s += n
    q = bf16.to_f64(w.normal_bf16(rng, (B, Hq, D)))
    out1, lse1 = attention.paged_decode(q, c, tables, lens, 0.2)
    pi = rng.permutation(nb)                 # physical block b moves to pi[b]
    c2 = c.copy()
    c2.k[pi] = c.k
    c2.v[pi] = c.v
    out2, lse2 = attention.paged_decode(q, c2, pi[tables], lens, 0.2)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


# ---------------------------------------------------------------- merge
@pytest.mark.parametrize("split", [1, 7, 20, 39])
def test_two_chunk_merge_equals_full_softmax(split):
    rng = np.random.default_rng(split)
    D, m = 16, 40
    q = rng.standard_normal((5, D))
    K = rng.standard_normal((m, D)) * 2
    V = rng.standard_normal((m, D))
    o, l = attention.attend(q, K, V, 0.5)
    o1, l1 = attention.attend(q, K[:split], V[:split], 0.5)
    o2, l2 = attention.attend(q, K[split:], V[split:], 0.5)
    om, lm = merge.merge(o1, l1, o2, l2)
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, l, atol=1e-13)
    # many chunks, any order of folding gives the same result
    parts = [attention.attend(q, K[i:i + 6], V[i:i + 6], 0.5) for i in range(0, m, 6)]
    om2, lm2 = merge.merge_all(parts[::-1])
    np.testing.assert_allclose(om2, o, atol=1e-13)
    np.testing.assert_allclose(lm2, l, atol=1e-13)


def test_merge_with_empty_state():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((3, 8))
    l = rng.standard_normal(3)
    empty_o = np.zeros((3, 8))
    empty_l = np.full(3, -np.inf)
    om, lm = merge.merge(o, l, empty_o, empty_l)
    assert np.array_equal(om, o) and np.array_equal(lm, l)
    om, lm = merge.merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(om == 0) and np.all(lm == -np.inf)


# ---------------------------------------------------------------- prefill / extend
def test_prefill_matches_sdpa_causal_varlen():
    rng = np.random.default_rng(21)
    Hq, Hkv, D = 8, 2, 32
    lens = [1, 13, 40]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    q = bf16.to_f64(w.normal_bf16(rng, (T, Hq, D)))
    k = bf16.to_f64(w.normal_bf16(rng, (T, Hkv, D)))
    v = bf16.to_f64(w.normal_bf16(rng, (T, Hkv, D)))
    out, lse = attention.prefill(q, k, v, cu, 0.25)
    for n in range(len(lens)):
        s0, s1 = cu[n], cu[n + 1]
        L = s1 - s0
        mask = np.tril(np.ones((L, L), bool))
        ref = _sdpa(q[s0:s1], k[s0:s1], v[s0:s1], 0.25, mask)
        np.testing.assert_allclose(out[s0:s1], ref, atol=1e-12)
    # non-causal too
    out_nc, _ = attention.prefill(q, k, v, cu, 0.25, causal=False)
    ref = _sdpa(q[cu[2]:], k[cu[2]:], v[cu[2]:], 0.25)
    np.testing.assert_allclose(out_nc[cu[2]:], ref, atol=1e-12)


def test_prefill_rows_subset_matches_full():
    rng = np.random.default_rng(22)
    q = rng.standard_normal((30, 4, 16))
    k = rng.standard_normal((30, 2, 16))
    v = rng.standard_normal((30, 2, 16))
    cu = np.array([0, 10, 30])
    full, lf = attention.prefill(q, k, v, cu, 0.3)
    rows = [0, 9, 10, 29]
    sub, ls = attention.prefill(q, k, v, cu, 0.3, rows=rows)
    assert np.array_equal(sub[rows], full[rows]) and np.array_equal(ls[rows], lf[rows])
    assert np.isnan(sub[5]).all()


def _extend_case(rng, ctx, new, Hq=8, Hkv=2, D=32, bs=16, nb=64):
    c = _rand_cache(rng, nb, bs, Hkv, D)
    E = len(ctx)
    tables = np.zeros((E, 16), dtype=np.int64)
    perm = rng.permutation(nb)
    s = 0
    for e in range(E):
        n = (ctx[e] + bs - 1) // bs
        tables[e, :n] = perm[s:s + n]
        s += n
    cu = np.concatenate([[0], np.cumsum(new)])
    T = cu[-1]
    q = bf16.to_f64(w.normal_bf16(rng, (T, Hq, D)))
    kn = bf16.to_f64(w.normal_bf16(rng, (T, Hkv, D)))
    vn = bf16.to_f64(w.normal_bf16(rng, (T, Hkv, D)))
    return c, tables, cu, q, kn, vn


def test_extend_matches_sdpa_bottom_right_mask():
    rng = np.random.default_rng(31)
    ctx, new = [35, 70], [9, 20]
    c, tables, cu, q, kn, vn = _extend_case(rng, ctx, new)
    out, lse = attention.extend(q, kn, vn, cu, ctx, c, tables, 0.2)
    for e in range(2):
        C, n = ctx[e], new[e]
        Kc, Vc = oc.gather(c, tables[e], C)
        K = np.concatenate([Kc, kn[cu[e]:cu[e + 1]]])
        V = np.concatenate([Vc, vn[cu[e]:cu[e + 1]]])
        mask = np.ones((n, C + n), bool)
        mask[:, C:] = np.tril(np.ones((n, n), bool))
        ref = _sdpa(q[cu[e]:cu[e + 1]], K, V, 0.2, mask)
        np.testing.assert_allclose(out[cu[e]:cu[e + 1]], ref, atol=1e-12)


def test_extend_without_context_is_prefill():
    rng = np.random.default_rng(32)
    c, tables, cu, q, kn, vn = _extend_case(rng, [0, 0], [7, 12])
    out, lse = attention.extend(q, kn, vn, cu, [0, 0], c, tables, 0.2)
    ref, lref = attention.prefill(q, kn, vn, cu, 0.2)
    np.testing.assert_allclose(out, ref, atol=1e-13)
    np.testing.assert_allclose(lse, lref, atol=1e-13)


def test_extend_of_one_token_is_decode():
    rng = np.random.default_rng(33)
    C, Hq, Hkv, D, bs = 45, 8, 2, 32, 16
    c, tables, cu, q, kn, vn = _extend_case(rng, [C], [1])
    out, lse = attention.extend(q, kn, vn, cu, [C], c, tables, 0.2)
    # the same token written into the cache at position C, then decoded
    c2 = c.copy()
    blk, off = tables[0][C // bs], C % bs
    kbits = w.f32_to_bf16_bits(kn[0].astype(np.float32))
    vbits = w.f32_to_bf16_bits(vn[0].astype(np.float32))
    c2.k[blk, off] = kbits
    c2.v[blk, off] = vbits
    od, ld = attention.paged_decode(q, c2, tables, [C + 1], 0.2)
    np.testing.assert_allclose(out, od, atol=1e-13)
    np.testing.assert_allclose(lse, ld, atol=1e-13)


def test_extend_chunk_decomposition_is_exact():
    """The page's extend method (new-token causal part, then each context
    chunk, LSE-merged) reproduces the plain definition."""
    rng = np.random.default_rng(34)
    C, n, scale = 50, 6, 0.2
    c, tables, cu, q, kn, vn = _extend_case(rng, [C], [n], Hq=2, Hkv=1)
    out, lse = attention.extend(q, kn, vn, cu, [C], c, tables, scale)
    Kc, Vc = oc.gather(c, tables[0], C)
    h = 1
    causal = np.tril(np.ones((n, n), bool))
    state = attention.attend(q[:, h], kn[:, 0], vn[:, 0], scale, causal)
    for s in range(0, C, 16):
        part = attention.attend(q[:, h], Kc[s:s + 16, 0], Vc[s:s + 16, 0], scale)
        state = merge.merge(*state, *part)
    np.testing.assert_allclose(state[0], out[:, h], atol=1e-13)
    np.testing.assert_allclose(state[1], lse[:, h], atol=1e-13)
