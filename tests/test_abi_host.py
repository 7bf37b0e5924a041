"""Host-side tests of the C ABI (CPU only): the library loads without a GPU,
exports every function include/pagedkv.h declares, rejects bad arguments with
the documented status codes before any HIP call, and its host-only pieces
(reorder, size queries) agree with the oracle and closed forms."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_cache_mapped_amd as pk
from oracle import batch as obatch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced by host validation


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char|void)\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    L = pk.lib()
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(pk.EXPORTS)
    assert L.kv_abi_version() == 1


def _cache(**kw):
    c = dict(k_cache=FAKE, v_cache=FAKE, num_blocks=64, block_size=16, num_kv_heads=2,
             head_dim=128, dtype=pk.KV_DTYPE_BF16, layout=pk.KV_LAYOUT_NHD, x=0,
             k_scale=1.0, v_scale=1.0)
    c.update(kw)
    return pk.KVCacheT(**c)


def _err():
    return pk.lib().kv_last_error().decode()


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, pk.KV_ENOTSUP),
    ("head_dim", 0, pk.KV_EINVAL),
    ("block_size", 12, pk.KV_EINVAL),
    ("block_size", 512, pk.KV_EINVAL),
    ("num_blocks", 0, pk.KV_EINVAL),
    ("num_kv_heads", 0, pk.KV_EINVAL),
    ("dtype", 7, pk.KV_EINVAL),
    ("layout", 3, pk.KV_EINVAL),
    ("k_cache", 0, pk.KV_EINVAL),
    ("k_cache", FAKE + 8, pk.KV_EINVAL),
    ("k_scale", 2.0, pk.KV_EINVAL),
])
def test_cache_validation(field, value, code):
    c = _cache(**{field: value})
    rc = pk.lib().kv_write(ctypes.byref(c), FAKE, FAKE, FAKE, 4, None)
    assert rc == code, _err()
    assert _err() != "no error"


def test_preshuffled_x_rules():
    L = pk.lib()
    c = _cache(layout=pk.KV_LAYOUT_PRESHUFFLED, x=16)          # bf16 needs x = 8
    assert L.kv_write(ctypes.byref(c), FAKE, FAKE, FAKE, 1, None) == pk.KV_EINVAL
    c = _cache(layout=pk.KV_LAYOUT_PRESHUFFLED, dtype=pk.KV_DTYPE_FP8_E4M3, x=16, block_size=8,
               k_scale=0.5, v_scale=0.5)                        # bs must be a multiple of x
    assert L.kv_write(ctypes.byref(c), FAKE, FAKE, FAKE, 1, None) == pk.KV_EINVAL
    c = _cache(dtype=pk.KV_DTYPE_FP8_E4M3, k_scale=0.0, v_scale=1.0)
    assert L.kv_write(ctypes.byref(c), FAKE, FAKE, FAKE, 1, None) == pk.KV_EINVAL


def test_kv_write_argument_errors():
    L = pk.lib()
    c = _cache()
    assert L.kv_write(ctypes.byref(c), FAKE, FAKE, FAKE, -1, None) == pk.KV_EINVAL
    assert L.kv_write(ctypes.byref(c), None, FAKE, FAKE, 4, None) == pk.KV_EINVAL
    assert L.kv_write(ctypes.byref(c), FAKE + 2, FAKE, FAKE, 4, None) == pk.KV_EINVAL
    assert L.kv_write(None, FAKE, FAKE, FAKE, 4, None) == pk.KV_EINVAL
    # zero tokens: valid no-op, no HIP call
    assert L.kv_write(ctypes.byref(c), None, None, None, 0, None) == pk.KV_OK


def test_decode_argument_errors():
    L = pk.lib()
    c = _cache()
    args = lambda **kw: dict(dict(q=FAKE, batch=4, hq=8, tables=FAKE, mb=32, lens=FAKE, msl=512,
                                  scale=0.1, out=FAKE, lse=None, ws=FAKE, wsb=1 << 30, split=0), **kw)

    def call(**kw):
        a = args(**kw)
        return L.paged_decode_ex(ctypes.byref(c), a["q"], a["batch"], a["hq"], a["tables"], a["mb"],
                                 a["lens"], a["msl"], a["scale"], a["out"], a["lse"], a["ws"],
                                 a["wsb"], a["split"], None)
    assert call(hq=7) == pk.KV_EINVAL                 # not a multiple of H_kv
    assert call(batch=0) == pk.KV_EINVAL
    assert call(msl=0) == pk.KV_EINVAL
    assert call(mb=8) == pk.KV_EINVAL                 # 8 blocks * 16 < 512 tokens
    assert call(q=None) == pk.KV_EINVAL
    assert call(out=FAKE + 4) == pk.KV_EINVAL
    assert call(split=100) == pk.KV_EINVAL            # not a multiple of 32
    assert call(split=128, wsb=16) == pk.KV_ENOSPC    # the plan needs a workspace
    assert call(ws=None) == pk.KV_EINVAL


def test_decode_workspace_closed_form():
    """header + prefix sums + piece list + fp32 partial rows (o then lse).
    Piece p of request b keeps its partial in row p + b, so there are at most
    (pieces + batch) rows per query head whatever the lengths."""
    c = _cache(num_kv_heads=8)
    L = pk.lib()
    B, Hq, msl = 64, 64, 8192
    a256 = lambda x: -(-x // 256) * 256

    def want(max_pieces):
        rows = (max_pieces + B) * Hq
        return 256 + a256(4 * (B + 1)) + a256(4 * max_pieces) + a256(rows * 128 * 4) + a256(rows * 4)

    for split in (128, 512, 1024):
        assert L.paged_decode_workspace_bytes_ex(ctypes.byref(c), B, Hq, msl, split) == \
            want(-(-(B * msl) // split) + 1)
    # automatic pieces (no GPU here: 256 compute units assumed): 8 KV heads of
    # 8 query heads -> one workgroup row of 256 workgroups x 1 wave per group
    # -> 256 target pieces; the longest piece a wave's table slice holds at
    # block size 16 is 4064 tokens
    assert L.paged_decode_workspace_bytes_ex(ctypes.byref(c), B, Hq, msl, 0) == \
        want(max(256, -(-(B * msl) // 4064)) + 1)
    assert L.paged_decode_workspace_bytes_ex(ctypes.byref(c), B, 63, msl, 0) == 0   # invalid -> 0
    # batch * max_seq_len at 2^31 is rejected
    assert L.paged_decode_workspace_bytes_ex(ctypes.byref(c), 65535, Hq, 1 << 16, 0) == 0


def test_decode_workspace_bounded_for_long_requests():
    """The partial rows no longer scale with max_seq_len / 256 per request:
    the fp8 preshuffled workload's shape (batch 128, 64:4, up to 16000
    tokens) needs about 21 MB, not the 270 MB of one slot per 256 tokens."""
    f = _cache(num_kv_heads=4, dtype=pk.KV_DTYPE_FP8_E4M3, layout=pk.KV_LAYOUT_PRESHUFFLED, x=16,
               k_scale=0.1, v_scale=0.1, num_blocks=131072)
    n = pk.lib().paged_decode_workspace_bytes_ex(ctypes.byref(f), 128, 64, 16000, 0)
    assert 0 < n < 32 << 20


def test_pack_sizes_and_errors():
    L = pk.lib()
    # Llama-3.1-70B layer: 8 KV heads x 128 dims x bf16 x 16 tokens -> 32 KiB per block per tensor
    c = _cache(num_kv_heads=8, num_blocks=32768)
    assert L.kv_layer_packed_bytes(ctypes.byref(c), 5000) == 327_680_000
    assert L.kv_layer_packed_bytes(ctypes.byref(c), 1) * 80 // 16 == 320 * 1024
    f = _cache(num_kv_heads=4, dtype=pk.KV_DTYPE_FP8_E4M3, layout=pk.KV_LAYOUT_PRESHUFFLED, x=16,
               k_scale=0.1, v_scale=0.1)
    assert L.kv_layer_packed_bytes(ctypes.byref(f), 3) == 2 * 3 * 16 * 4 * 128
    assert L.kv_pack_layer(ctypes.byref(c), FAKE, 10, FAKE, 100, None) == pk.KV_ENOSPC
    assert L.kv_unpack_layer(ctypes.byref(c), FAKE, 10, FAKE + 1, 1 << 30, None) == pk.KV_EINVAL
    assert L.kv_pack_layer(ctypes.byref(c), FAKE, -1, FAKE, 1 << 30, None) == pk.KV_EINVAL
    assert L.kv_pack_layer(ctypes.byref(c), None, 0, None, 0, None) == pk.KV_OK


def test_prefill_and_extend_argument_errors():
    L = pk.lib()
    assert L.prefill_attn(FAKE, FAKE, FAKE, FAKE, 2, 100, 8, 3, 128, 0.1, 1, FAKE, None, None) == pk.KV_EINVAL
    assert L.prefill_attn(FAKE, FAKE, FAKE, FAKE, 2, 100, 8, 2, 64, 0.1, 1, FAKE, None, None) == pk.KV_ENOTSUP
    assert L.prefill_attn(FAKE, FAKE, FAKE, FAKE, 2, 100, 8, 2, 128, 0.1, 2, FAKE, None, None) == pk.KV_EINVAL
    assert L.prefill_attn(None, FAKE, FAKE, FAKE, 2, 100, 8, 2, 128, 0.1, 1, FAKE, None, None) == pk.KV_EINVAL
    assert L.prefill_attn(None, None, None, None, 0, 0, 8, 2, 128, 0.1, 1, None, None, None) == pk.KV_OK
    c = _cache()
    f = _cache(dtype=pk.KV_DTYPE_FP8_E4M3, k_scale=0.1, v_scale=0.1)
    ext = lambda cc, budget=32768, mctx=100, mb=16, mode=0, scale=0.1: L.extend_attn_ex(
        ctypes.byref(cc), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mb, 2, 64, 32, mctx, 8, budget, scale,
        FAKE, None, FAKE, 1 << 30, mode, None)
    assert ext(c, budget=0) == pk.KV_EINVAL
    assert ext(c, mctx=1000, mb=16) == pk.KV_EINVAL   # table too narrow for the context
    assert ext(c, mode=3) == pk.KV_EINVAL
    assert ext(c, mode=-1) == pk.KV_EINVAL
    # a table of more than 2^30 tokens would overflow the kernels' 32-bit
    # token arithmetic
    assert ext(c, mb=(1 << 26) + 1) == pk.KV_EINVAL
    assert "2^30" in _err()


@pytest.mark.parametrize("scale", [0.0, -0.125, float("nan"), float("inf"), -float("inf")])
def test_attention_calls_reject_bad_scales(scale):
    """A softmax scale must be finite and positive in all three attention calls
    (the tiles take the running maximum on raw scores)."""
    L = pk.lib()
    c = _cache()
    rc = L.prefill_attn(FAKE, FAKE, FAKE, FAKE, 2, 100, 8, 2, 128, scale, 1, FAKE, None, None)
    assert rc == pk.KV_EINVAL and "scale" in _err()
    rc = L.extend_attn(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 64, 32, 100, 8,
                       32768, scale, FAKE, None, FAKE, 1 << 30, None)
    assert rc == pk.KV_EINVAL and "scale" in _err()
    rc = L.paged_decode(ctypes.byref(c), FAKE, 4, 8, FAKE, 32, FAKE, 512, scale, FAKE, None, FAKE,
                        1 << 30, None)
    assert rc == pk.KV_EINVAL and "scale" in _err()


def test_extend_workspace_by_mode():
    """Fused extend needs no workspace; split extend needs one fp32 (o, lse)
    partial per (part, row, query head): parts = context chunks + 1; the
    automatic (hybrid) one a plan and a bounded block of compact partials."""
    L = pk.lib()
    c = _cache(num_kv_heads=8, num_blocks=16384)
    a256 = lambda x: -(-x // 256) * 256
    E, T, Hq, mctx, budget = 2, 16384, 64, 100000, 32768
    ws = lambda mode: L.extend_attn_workspace_bytes_ex(ctypes.byref(c), E, T, Hq, mctx, budget, mode)
    assert ws(pk.KV_EXTEND_FUSED) == 0
    chunk = budget // E                               # 16384, a whole number of 64-key tiles
    parts = -(-mctx // chunk) + 1                     # 7 chunks + the new tokens
    rows = parts * T * Hq
    assert ws(pk.KV_EXTEND_SPLIT) == a256(rows * 128 * 4) + a256(rows * 4)
    # automatic: 128 query tiles x 64 heads fill 256 CUs -> fused, and a
    # context of 7 chunks -> hybrid: the plan (4 header words, per split slot
    # a request and a first compact row), the work list (16 bytes per entry:
    # at most T/R + E query items of fused requests and n_parts x (cap_rows/R
    # + slots) of split ones, R = 256 / P tokens per workgroup, P = 8 query
    # heads for a group of 8) and the partials of at most 64 MiB of compact
    # rows
    slots = min(E, 16)
    cap_rows = min(T, (64 << 20) // (parts * Hq * 129 * 4))
    crow = parts * cap_rows * Hq
    R = 256 // 8
    list_cap = -(-T // R) + E + parts * (-(-cap_rows // R) + slots)
    assert ws(pk.KV_EXTEND_AUTO) == (a256(4 * (4 + 2 * slots)) + a256(16 * list_cap) +
                                     a256(crow * 128 * 4) + a256(crow * 4))
    # a context within one chunk leaves nothing to split: plain fused
    assert L.extend_attn_workspace_bytes_ex(ctypes.byref(c), E, T, Hq, chunk, budget,
                                            pk.KV_EXTEND_AUTO) == 0
    assert ws(7) == 0                                 # invalid mode


@pytest.mark.parametrize("seed", range(5))
def test_reorder_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 40))
    q = rng.integers(0, 5, size=n) * rng.integers(0, 2, size=n) + rng.integers(0, 2, size=n)
    c = rng.integers(0, 3, size=n) * rng.integers(0, 100, size=n)
    for thr in (0, 1, 2):
        perm, counts = pk.reorder_batch(q, c, thr)
        operm, ocounts = obatch.reorder(q, c, thr)
        assert perm == operm and counts == ocounts


def test_reorder_rejects_negative_lengths():
    with pytest.raises(pk.PagedKVError) as e:
        pk.reorder_batch([1, -2], [0, 0])
    assert e.value.code == pk.KV_EINVAL


def test_binding_refuses_tensors_the_abi_would_misread():
    """int64 lengths would be read as int32 pairs and a non-contiguous view with
    the wrong row stride; the binding refuses both before any library call."""
    import torch
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16)
    tables = torch.zeros((2, 4), dtype=torch.int32)
    with pytest.raises(TypeError, match="seq_lens"):
        pk.paged_decode(None, q, tables, torch.ones(2, dtype=torch.int64), 16, 0.1)
    with pytest.raises(ValueError, match="contiguous"):
        pk.paged_decode(None, q, torch.zeros((4, 2), dtype=torch.int32).t(),
                        torch.ones(2, dtype=torch.int32), 16, 0.1)
    with pytest.raises(TypeError, match="q"):
        pk.prefill_attn(q.float(), q, q, torch.zeros(2, dtype=torch.int32), 1, 0.1)
    with pytest.raises(TypeError, match="cu_q_lens"):
        pk.extend_attn(None, q, q, q, torch.zeros(2, dtype=torch.int64),
                       torch.zeros(1, dtype=torch.int32), tables[:1], 2, 0, 0.1)
    with pytest.raises(TypeError, match="slot_mapping"):
        pk.kv_write(None, q, q, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(TypeError, match="k_cache"):
        pk.PagedKVCache(torch.zeros((4, 16, 8, 128), dtype=torch.float16),
                        torch.zeros((4, 16, 8, 128), dtype=torch.float16), 16, 8, 128)
    with pytest.raises(ValueError, match="GPU"):      # right types, but host memory
        pk.PagedKVCache(torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16),
                        torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16), 16, 8, 128)


def test_library_shares_torchs_hip_runtime_when_loaded_first():
    """A host-only call (here the batch reorder) before any torch import must
    not give the process a second HIP runtime: the library has to bind to the
    one that owns torch's devices, streams and allocations."""
    import subprocess
    import sys
    code = (
        "import paged_kv_cache_mapped_amd as pk\n"
        "pk.reorder_batch([1, 5], [3, 0])\n"
        "import torch\n"
        "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
        "print(len(paths))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[-1] == "1", r.stdout
