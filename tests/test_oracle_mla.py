"""Pins of the oracle's absorbed MLA decode (CPU only).

The strongest one is the identity that makes absorption exact: attention of
a standard multi-head layer whose keys and values are up-projected from the
latent (k_h = [W_UK_h c ; k_rope], v_h = W_UV_h c) equals, head by head, the
absorbed attention over the latent rows [c ; k_rope] with the query
[W_UK_h^T q_nope ; q_rope], followed by W_UV_h.  The MHA side is computed by
torch's scaled_dot_product_attention (a library routine the oracle does not
call), so a dropped rope term, a transposed projection or a wrong value slice
in the oracle fails it."""
import json
import math
import os

import numpy as np
import pytest

from oracle import bf16, mla
from synth import workloads as w

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_latent_width_golden():
    g = json.load(open(os.path.join(GOLD, "mla_latent.json")))
    assert mla.LATENT_DIMS == g["printed"]["latent_dims"]
    assert mla.VALUE_DIMS + g["reading"]["rope_dims"] == mla.LATENT_DIMS
    ratio = g["printed"]["mha_dims_approx"] / mla.LATENT_DIMS
    assert round(ratio) == g["printed"]["compression_approx"]


def _cache(rng, nb, bs):
    return w.normal_bf16(rng, (nb, bs, mla.LATENT_DIMS))


@pytest.mark.parametrize("bs", [1, 16])
def test_absorbed_equals_up_projected_mha(bs):
    import torch
    rng = np.random.default_rng(71)
    H, dn, dr, dc = 4, 128, 64, 512
    L = 37
    nb = (L + bs - 1) // bs + 3
    cache = _cache(rng, nb, bs)
    table = rng.permutation(nb)[: (L + bs - 1) // bs]
    W_UK = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    W_UV = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    q_nope = rng.standard_normal((H, dn))
    q_rope = rng.standard_normal((H, dr))
    scale = 1.0 / math.sqrt(dn + dr)
    R = mla.gather_latent(cache, table, L, bs)              # [L, 576]
    c, k_rope = R[:, :dc], R[:, dc:]
    # absorbed: one decode request, H heads
    q_abs = np.concatenate([np.einsum("hnc,hn->hc", W_UK, q_nope), q_rope], axis=1)
    o_lat, lse = mla.mla_decode(q_abs[None], cache, table[None], [L], scale, bs)
    o_abs = np.einsum("hnc,hc->hn", W_UV, o_lat[0])
    # standard MHA on the up-projected keys and values (torch, float64)
    K = np.concatenate([np.einsum("hnc,lc->hln", W_UK, c),
                        np.broadcast_to(k_rope, (H, L, dr))], axis=2)   # [H, L, 192]
    V = np.einsum("hnc,lc->hln", W_UV, c)                               # [H, L, 128]
    qh = np.concatenate([q_nope, q_rope], axis=1)[:, None, :]           # [H, 1, 192]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    o_mha = torch.nn.functional.scaled_dot_product_attention(
        t(qh), t(K), t(V), scale=scale).numpy()[:, 0]
    s = scale * np.einsum("hd,hld->hl", qh[:, 0], K)
    lse_mha = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
    assert np.allclose(o_abs, o_mha, atol=1e-12, rtol=1e-10)
    assert np.allclose(lse[0], lse_mha, atol=1e-12)


def test_brute_force_loops():
    """Element-by-element reads of the physical cache (bit-field bf16 decode)
    and a loop softmax, independent of numpy's vector paths."""
    import struct
    rng = np.random.default_rng(72)
    bs, nb, H = 4, 9, 3
    cache = _cache(rng, nb, bs)
    lens = [1, 6, 13]
    tables = np.stack([rng.permutation(nb)[:4] for _ in lens])
    q = rng.standard_normal((len(lens), H, mla.LATENT_DIMS))
    scale = 0.07

    def val(bits):
        return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]

    out, lse = mla.mla_decode(q, cache, tables, lens, scale, bs)
    for b, L in enumerate(lens):
        for h in range(H):
            rows = []
            for j in range(L):
                blk, off = int(tables[b][j // bs]), j % bs
                rows.append([val(cache[blk, off, d]) for d in range(mla.LATENT_DIMS)])
            sc = [scale * sum(q[b, h, d] * rows[j][d] for d in range(mla.LATENT_DIMS))
                  for j in range(L)]
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            z = sum(e)
            o = [sum(e[j] * rows[j][d] for j in range(L)) / z for d in range(mla.VALUE_DIMS)]
            assert max(abs(o[d] - out[b, h, d]) for d in range(mla.VALUE_DIMS)) < 1e-12
            assert abs(m + math.log(z) - lse[b, h]) < 1e-12


def test_closed_forms_and_empty():
    rng = np.random.default_rng(73)
    cache = _cache(rng, 6, 16)
    table = np.array([[4, 1, 3]])
    R = mla.gather_latent(cache, table[0], 40, 16)
    # one token: the output is its value part, lse its score
    q = rng.standard_normal((1, 2, mla.LATENT_DIMS))
    o, l = mla.mla_decode(q, cache, table, [1], 0.1)
    assert np.allclose(o[0], R[0, :512]) and np.allclose(l[0], 0.1 * q[0] @ R[0])
    # zero query: the mean of the value parts, lse = ln L
    o, l = mla.mla_decode(np.zeros((1, 2, 576)), cache, table, [40], 0.1)
    assert np.allclose(o[0], R[:, :512].mean(0)) and np.allclose(l, math.log(40))
    # empty request
    o, l = mla.mla_decode(q, cache, table, [0], 0.1)
    assert (o == 0).all() and np.isneginf(l).all()
    # the value is the first 512 dims: the rope part never reaches the output
    c2 = cache.copy()
    c2[..., 512:] = 0
    q2 = q.copy()
    q2[..., 512:] = 0
    o1, _ = mla.mla_decode(q2, cache, table, [40], 0.1)
    o2, _ = mla.mla_decode(q2, c2, table, [40], 0.1)
    assert np.array_equal(o1, o2)
