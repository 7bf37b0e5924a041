"""GPU test of paged_decode_noalloc, the decode entry point that allocates
nothing (its plan and partials live in the library's static scratch):
called through the C ABI, its output must equal paged_decode's with a caller
workspace, bit for bit, on two calls in a row -- the second with a smaller
batch and shorter contexts, so stale scratch contents from the first call
must not leak into it."""
import ctypes

import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from synth import workloads as w

from .gpu_util import BF16_TOL, LSE_TOL, bf16_to_f64, dev, device_cache, max_err, say, torch

pytestmark = pytest.mark.gpu


def _abi_noalloc(dc, st, out, lse):
    t = torch()
    d = dc.desc()
    q, tables, lens = dev(st.q), dev(st.block_tables), dev(st.seq_lens)
    rc = pk.lib().paged_decode_noalloc(
        ctypes.byref(d), q.data_ptr(), st.batch, st.num_q_heads, tables.data_ptr(),
        int(st.block_tables.shape[1]), lens.data_ptr(), int(st.seq_lens.max()), st.scale,
        out.data_ptr(), lse.data_ptr(), t.cuda.current_stream().cuda_stream)
    assert rc == pk.KV_OK, pk.lib().kv_last_error().decode()
    t.cuda.synchronize()


def _with_workspace(dc, st):
    out, lse = pk.paged_decode(dc, dev(st.q), dev(st.block_tables), dev(st.seq_lens),
                               int(st.seq_lens.max()), st.scale)
    torch().cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("layout,dtype", [("nhd", "bf16"), ("preshuffled", "fp8")])
def test_noalloc_matches_workspace_decode_twice(layout, dtype):
    t = torch()
    big = w.decode_workload(61, 32, 32, 4, 128, 16, 32 * 375 + 64, 2048, 6000, layout=layout,
                            dtype=dtype)
    small = w.decode_workload(62, 7, 16, 2, 128, 16, 7 * 40 + 64, 1, 600, layout=layout,
                              dtype=dtype, fixed_lens=[1, 0, 17])
    for name, st in (("big", big), ("small", small)):
        say(f"noalloc decode {layout} {dtype} {name}: batch {st.batch}, "
            f"{st.num_q_heads}:{st.cache.spec.num_kv_heads}, max len {int(st.seq_lens.max())}")
        dc = device_cache(st.cache)
        out = t.full((st.batch, st.num_q_heads, 128), float("nan"), dtype=t.bfloat16, device="cuda")
        lse = t.full((st.batch, st.num_q_heads), float("nan"), dtype=t.float32, device="cuda")
        _abi_noalloc(dc, st, out, lse)
        ref_o, ref_l = _with_workspace(dc, st)
        o, ro = bf16_to_f64(out), bf16_to_f64(ref_o)
        l, rl = lse.cpu().numpy(), ref_l.cpu().numpy()
        # same kernels and plan: identical bits (so within any tolerance)
        assert np.array_equal(o, ro, equal_nan=False), max_err(o, ro)
        assert np.array_equal(l, rl)
        assert max_err(o, ro) <= BF16_TOL and max_err(l[np.isfinite(rl)], rl[np.isfinite(rl)]) <= LSE_TOL


def test_noalloc_rejects_batches_beyond_its_scratch():
    """A decode whose plan needs more than the 64 MiB scratch is refused with
    KV_ENOSPC before anything is launched (no fallback allocation)."""
    t = torch()
    st = w.decode_workload(63, 2048, 128, 1, 128, 16, 2048 * 2 + 64, 1, 16)
    dc = device_cache(st.cache)
    need = pk.paged_decode_workspace_bytes(dc, 2048, 128, 16384)
    assert need > 64 << 20
    out = t.empty((2048, 128, 128), dtype=t.bfloat16, device="cuda")
    d = dc.desc()
    tables = t.zeros((2048, 1024), dtype=t.int32, device="cuda")
    lens = t.ones(2048, dtype=t.int32, device="cuda")
    q = dev(st.q)
    rc = pk.lib().paged_decode_noalloc(ctypes.byref(d), q.data_ptr(), 2048, 128,
                                       tables.data_ptr(), 1024, lens.data_ptr(), 16384, st.scale,
                                       out.data_ptr(), None, t.cuda.current_stream().cuda_stream)
    assert rc == pk.KV_ENOSPC and "scratch" in pk.lib().kv_last_error().decode()
