"""GPU parity of the absorbed MLA decode ("Beyond just running: native
inference optimisation in vLLM on AMD ROCm", section "AITER MLA backend:
optimised for DeepSeek": one 576-dim latent row per token shared by every
query head, block size 16) against the oracle: bf16 outputs within 1.5e-2,
lse within 1e-3."""
import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import bf16 as ob, mla
from synth import workloads as w

from .gpu_util import BF16_TOL, LSE_TOL, bf16_to_f64, dev, max_err, say, torch

pytestmark = pytest.mark.gpu


def _run(st, msl=None, out=None, lse=None, workspace=None):
    msl = int(st.seq_lens.max()) if msl is None else msl
    o, l = pk.mla_decode(dev(st.cache), dev(st.q), dev(st.block_tables), dev(st.seq_lens), msl,
                         st.scale, out=out, lse=lse, workspace=workspace)
    torch().cuda.synchronize()
    return bf16_to_f64(o), l.cpu().numpy().astype(np.float64)


def _check(st, out, lse, rows=None):
    rows = list(range(st.batch)) if rows is None else rows
    q = ob.to_f64(st.q)
    worst = [0.0, 0.0]
    for b in rows:
        ro, rl = mla.mla_decode(q[b:b + 1], st.cache, st.block_tables[b:b + 1],
                                st.seq_lens[b:b + 1], st.scale, st.block_size)
        if st.seq_lens[b] == 0:
            assert (out[b] == 0).all() and np.isneginf(lse[b]).all()
            continue
        e, el = max_err(out[b], ro[0]), max_err(lse[b], rl[0])
        assert e <= BF16_TOL, (b, e)
        assert el <= LSE_TOL, (b, el)
        worst = [max(worst[0], e), max(worst[1], el)]
    say(f"  max|err| out {worst[0]:.3e} lse {worst[1]:.3e} over {len(rows)} requests")


def _poison(st):
    """NaN in every slot past each request's length (the rest of its last
    block, its spare blocks) and in the poison block."""
    nan = np.uint16(0x7FC0)
    bs = st.block_size
    st.cache[-1] = nan
    for b, L in enumerate(st.seq_lens):
        L = int(L)
        nblk = (L + bs - 1) // bs
        if nblk and L % bs:
            st.cache[st.block_tables[b, nblk - 1], L % bs:] = nan


@pytest.mark.parametrize("heads", [16, 8, 20, 128])
def test_mla_small_ragged(heads):
    st = w.mla_decode_workload(81, 6, heads, 16, 6 * 40 + 64, 1, 600,
                               fixed_lens=[1, 15, 16, 17, 300])
    _poison(st)
    say(f"mla decode {heads} heads lens={st.seq_lens.tolist()}")
    out, lse = _run(st)
    _check(st, out, lse)


@pytest.mark.parametrize("bs", [16, 64])
def test_mla_block_sizes_and_pieces(bs):
    """Lengths that span many pieces (the combine pass) next to short ones."""
    st = w.mla_decode_workload(82, 9, 16, bs, 9 * 5000 // bs + 64, 1, 5000,
                               fixed_lens=[4999, 1, 64, 65, 2048])
    _poison(st)
    say(f"mla decode bs={bs} lens={st.seq_lens.tolist()}")
    out, lse = _run(st)
    _check(st, out, lse)
    again = _run(st)
    assert np.array_equal(out, again[0]) and np.array_equal(lse, again[1])   # deterministic


def test_mla_empty_requests():
    t = torch()
    st = w.mla_decode_workload(83, 7, 16, 16, 7 * 40 + 64, 50, 600)
    st.seq_lens[[0, 3, 6]] = 0
    say(f"mla decode with empty requests lens={st.seq_lens.tolist()}")
    out = t.full((7, 16, 512), float("nan"), dtype=t.bfloat16, device="cuda")
    lse = t.full((7, 16), float("nan"), dtype=t.float32, device="cuda")
    o, l = _run(st, out=out, lse=lse)
    _check(st, o, l)


@pytest.mark.parametrize("batch", [2000, 2001, 2600])
def test_mla_large_batches(batch):
    """Up to 2000 requests the piece kernel plans in its own LDS; above, a
    planning launch leaves the plan in the workspace.  Both sides of the
    boundary, short ragged requests (some empty), sampled requests against
    the oracle."""
    st = w.mla_decode_workload(86, batch, 16, 16, batch * 7 + 64, 1, 100)
    st.seq_lens[::97] = 0
    _poison(st)
    say(f"mla decode batch {batch}, lengths [0, 100]")
    out, lse = _run(st)
    rng = np.random.default_rng(batch)
    rows = sorted(set(rng.choice(batch, 48, replace=False).tolist()) | {0, 1, batch - 2, batch - 1})
    _check(st, out, lse, rows)


def test_mla_needle():
    """One planted latent row whose score dominates for every head of its
    request: the output is that row's value part (a mis-addressed block would
    move it by O(1))."""
    st = w.mla_decode_workload(84, 4, 16, 16, 4 * 800 + 64, 2000, 3000)
    rng = np.random.default_rng(84)
    for b in range(st.batch):
        L = int(st.seq_lens[b])
        tok = int(rng.integers(0, L))
        blk, off = st.block_tables[b, tok // 16], tok % 16
        u = rng.standard_normal(576)
        u /= np.linalg.norm(u)
        st.cache[blk, off, :] = w.f32_to_bf16_bits((30.0 * u).astype(np.float32))
        for h in range(16):
            st.q[b, h] = w.f32_to_bf16_bits((np.sqrt(576) * u + 0.1 * rng.standard_normal(576))
                                            .astype(np.float32))
    say("mla decode needle")
    out, lse = _run(st)
    _check(st, out, lse)


def test_mla_deepseek_share_full_size():
    """One GPU's share of DeepSeek-R1 MLA decode under TP8: batch 128, 16
    query heads, context 10000-11000, block 16: every request."""
    st = w.deepseek_mla_decode()
    say("mla decode deepseek TP8 share: batch 128, 16 heads, ctx [10000, 11000]")
    out, lse = _run(st)
    assert not np.isnan(out).any()
    _check(st, out, lse)
