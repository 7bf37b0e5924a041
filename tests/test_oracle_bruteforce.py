"""Brute-force pins for the oracle's three attention paths (CPU only).

An independent pure-Python float implementation, written from the
definitions alone: every key/value element is read from the physical cache
arrays one at a time with the layout formulas (NHD [block][slot][head][dim];
preshuffled K [block][head][dim/x][slot][x], V [block][head][slot/x][dim][x]),
bf16 bit patterns and OCP e4m3fn codes are decoded from their bit fields, and
softmax attention is a loop over keys with math.exp.  Nothing here calls the
oracle's gather, codec or attention code; the oracle must agree to float64
rounding on tiny decode, causal prefill and bottom-right extend cases, for
both layouts, bf16 and fp8, and GQA ratios 1, 2 and 4.

Reference: "Beyond just running: native inference optimisation in vLLM on AMD
ROCm", sections "Processing details of the three paths" and "ROCM_AITER_FA"
(preshuffled layout); "From LLM performance optimisation to DeepSeek
deployment", section 3 "Paged Attention" (block table).
"""
import math
import struct

import numpy as np
import pytest

from oracle import attention, bf16, cache as oc
from synth import workloads as w


def _bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _e4m3fn_value(code):
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _element(cd, which, blk, slot, h, d):
    """Element (slot, head, dim) of block blk, straight from the raw arrays."""
    sp = cd.spec
    raw = cd.k if which == "k" else cd.v
    if sp.layout == "nhd":
        code = raw[blk, slot, h, d]
    else:
        x = sp.x
        code = raw[blk, h, d // x, slot, d % x] if which == "k" else raw[blk, h, slot // x, d, slot % x]
    if sp.dtype == "bf16":
        return _bf16_value(code)
    return _e4m3fn_value(code) * (cd.k_scale if which == "k" else cd.v_scale)


def _key_row(cd, table, t, h):
    bs = cd.spec.block_size
    blk, slot = int(table[t // bs]), t % bs
    D = cd.spec.head_dim
    return ([_element(cd, "k", blk, slot, h, d) for d in range(D)],
            [_element(cd, "v", blk, slot, h, d) for d in range(D)])


def _softmax_attend(qrow, keys, vals, scale):
    s = [scale * sum(a * b for a, b in zip(qrow, k)) for k in keys]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    l = sum(e)
    o = [sum(e[j] * vals[j][d] for j in range(len(keys))) / l for d in range(len(qrow))]
    return o, m + math.log(l)


def _tiny_cache(seed, layout, dtype, nb=7, bs=16, H=2, D=16):
    rng = np.random.default_rng(seed)
    cd = w.random_cache(rng, w.CacheSpec(nb, bs, H, D, layout, dtype))
    ocache = oc.Cache(cd.k, cd.v, layout, dtype, bs, H, D, cd.spec.x, cd.k_scale, cd.v_scale)
    return rng, cd, ocache


CASES = [("nhd", "bf16", 2, 2), ("nhd", "bf16", 4, 1), ("nhd", "fp8", 4, 2),
         ("preshuffled", "bf16", 2, 1), ("preshuffled", "fp8", 8, 2)]


@pytest.mark.parametrize("layout,dtype,Hq,Hkv", CASES)
def test_decode_brute_force(layout, dtype, Hq, Hkv):
    rng, cd, ocache = _tiny_cache(41, layout, dtype, H=Hkv)
    D, bs, nb = 16, 16, 7
    lens = [1, 17, 40]
    tables = np.stack([rng.permutation(nb)[:3] for _ in lens]).astype(np.int32)
    q = bf16.to_f64(w.normal_bf16(rng, (len(lens), Hq, D)))
    scale = 1 / math.sqrt(D)
    o_or, l_or = attention.paged_decode(q, ocache, tables, np.asarray(lens), scale)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        for h in range(Hq):
            rows = [_key_row(cd, tables[b], t, h // G) for t in range(L)]
            o, l = _softmax_attend(list(q[b, h]), [r[0] for r in rows], [r[1] for r in rows], scale)
            np.testing.assert_allclose(o_or[b, h], o, rtol=0, atol=1e-12)
            assert abs(l_or[b, h] - l) < 1e-12


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1), (4, 2)])
def test_prefill_causal_brute_force(Hq, Hkv):
    rng = np.random.default_rng(42)
    D = 16
    lens = [1, 5, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    q = bf16.to_f64(w.normal_bf16(rng, (T, Hq, D)))
    k = bf16.to_f64(w.normal_bf16(rng, (T, Hkv, D)))
    v = bf16.to_f64(w.normal_bf16(rng, (T, Hkv, D)))
    scale = 0.3
    o_or, l_or = attention.prefill(q, k, v, cu, scale, causal=True)
    G = Hq // Hkv
    for n in range(len(lens)):
        s0 = int(cu[n])
        for i in range(lens[n]):
            for h in range(Hq):
                keys = [list(k[s0 + j, h // G]) for j in range(i + 1)]
                vals = [list(v[s0 + j, h // G]) for j in range(i + 1)]
                o, l = _softmax_attend(list(q[s0 + i, h]), keys, vals, scale)
                np.testing.assert_allclose(o_or[s0 + i, h], o, rtol=0, atol=1e-12)
                assert abs(l_or[s0 + i, h] - l) < 1e-12


@pytest.mark.parametrize("layout,dtype,Hq,Hkv", CASES[:3] + CASES[4:])
def test_extend_bottom_right_brute_force(layout, dtype, Hq, Hkv):
    rng, cd, ocache = _tiny_cache(43, layout, dtype, H=Hkv)
    D, nb = 16, 7
    ctx = [0, 3, 21]
    new = [4, 1, 6]
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int64)
    T = int(cu[-1])
    tables = np.stack([rng.permutation(nb)[:2] for _ in ctx]).astype(np.int32)
    q = bf16.to_f64(w.normal_bf16(rng, (T, Hq, D)))
    kn = bf16.to_f64(w.normal_bf16(rng, (T, Hkv, D)))
    vn = bf16.to_f64(w.normal_bf16(rng, (T, Hkv, D)))
    scale = 1 / math.sqrt(D)
    o_or, l_or = attention.extend(q, kn, vn, cu, np.asarray(ctx), ocache, tables, scale)
    G = Hq // Hkv
    for e, (C, n) in enumerate(zip(ctx, new)):
        s0 = int(cu[e])
        for i in range(n):
            for h in range(Hq):
                g = h // G
                cached = [_key_row(cd, tables[e], t, g) for t in range(C)]
                keys = [r[0] for r in cached] + [list(kn[s0 + j, g]) for j in range(i + 1)]
                vals = [r[1] for r in cached] + [list(vn[s0 + j, g]) for j in range(i + 1)]
                o, l = _softmax_attend(list(q[s0 + i, h]), keys, vals, scale)
                np.testing.assert_allclose(o_or[s0 + i, h], o, rtol=0, atol=1e-12)
                assert abs(l_or[s0 + i, h] - l) < 1e-12
