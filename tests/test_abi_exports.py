"""CPU-only checks of the C ABI: the library loads, exports every function
include/akv.h declares, and rejects bad arguments on the host before any
HIP call (no compute runs here)."""
import ctypes as C
import os
import subprocess

import pytest

from agent_kv_cache_amd import binding as B


def test_library_exports_every_header_function():
    assert os.path.exists(B.LIB_PATH), "libakv.so not built"
    names = B.header_functions()
    assert len(names) >= 14
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(names) <= exported, set(names) - exported


def _desc(**kw):
    d = B.AkvCacheDesc(2, 2, 128, 16, 10, 2, 4, 1.0e4)
    for f in ("k_pool", "v_pool", "block_table", "seq_lens", "next_pos", "positions",
              "token_ids", "free_stack", "free_count", "scratch"):
        setattr(d, f, 4096)          # non-null, aligned; never dereferenced on these paths
    d.scratch_bytes = B.lib().akv_scratch_bytes(C.byref(d))
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_scratch_size_formula():
    L = B.lib()
    d = _desc()
    n = L.akv_scratch_bytes(C.byref(d))
    S = 4 * 16
    assert n >= 2 * 2 * S * 4 + 10 * 4 and n % 256 == 0
    d.n_seqs = 0
    assert L.akv_scratch_bytes(C.byref(d)) == 0


@pytest.mark.parametrize("field,value", [
    ("head_dim", 96), ("head_dim", 256), ("block_size", 32), ("n_layers", 0),
    ("n_kv_heads", 0), ("n_blocks", 0), ("n_seqs", 0), ("n_seqs", 65536), ("max_blocks_per_seq", 0),
    ("rope_base", 0.0), ("rope_base", 0.5), ("rope_base", float("inf")), ("k_pool", None),
    ("scratch", None),
    ("scratch", 4096 + 8), ("scratch_bytes", 16), ("k_pool", 4096 + 2),
])
def test_init_rejects_bad_descriptors(field, value):
    d = _desc(**{field: value})
    h = C.c_void_p()
    assert B.lib().akv_cache_init(C.byref(d), C.byref(h)) == 1
    assert not h.value


@pytest.mark.parametrize("rotary_dim,freq,window", [
    (8, None, None),                      # not a multiple of 16
    (24, None, None),
    (144, None, None),                    # wider than the head
    (-16, None, None),
    (64, [1.0] * 31 + [float("nan")], None),
    (64, [1.0] * 31 + [-1.0], None),
    (64, [1.0] * 31 + [1.5], None),       # frequencies above 1
    (0, None, [0, -1]),                   # negative window
])
def test_init_rejects_bad_rope_variants(rotary_dim, freq, window):
    import numpy as np
    d = _desc(rotary_dim=rotary_dim)
    keep = []
    if freq is not None:
        a = np.asarray(freq, dtype=np.float64)
        keep.append(a)
        d.inv_freq = a.ctypes.data
    if window is not None:
        a = np.asarray(window, dtype=np.int32)
        keep.append(a)
        d.layer_window = a.ctypes.data
    h = C.c_void_p()
    assert B.lib().akv_cache_init(C.byref(d), C.byref(h)) == 1
    assert not h.value


def test_null_handle_calls_are_rejected():
    L = B.lib()
    assert L.akv_drop(None, None, None) == 1
    assert L.akv_drop_reposition(None, None, None, None) == 1
    assert L.akv_reposition(None, None, None, None) == 1
    assert L.akv_append(None, None, 0, None, None, None, None) == 1
    assert L.akv_decode_attention(None, None, None, 0, 1, 1, None, None, 0, None) == 1
    assert L.akv_fork(None, None, None, 0, None, None) == 1
    assert L.akv_segment_attention(None, None, None, None, 1, 1, 0, 1, 1, None, None) == 1
    assert L.akv_sync_status(None, None) == 1
    assert L.akv_profile_enable(None, 1) == 1
    assert L.akv_decode_workspace_bytes(None, 1, 1) == 0
    for code in range(7):
        assert L.akv_status_string(code)
