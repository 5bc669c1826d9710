"""ctypes binding of libakv.so (include/akv.h) -- argument marshalling only.

Every step of the hot path runs in the HIP kernels behind the C ABI; PyTorch
only provides device memory and the current stream.  There is no CPU
fallback: if libakv.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Optional

# AKV_LIBRARY may name another build of the same ABI (e.g. a tuning variant).
LIB_PATH = os.environ.get("AKV_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libakv.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "akv.h")

STATUS = {0: "AKV_OK", 1: "AKV_ERR_ARG", 2: "AKV_ERR_ORDER", 3: "AKV_ERR_POS_MISMATCH",
          4: "AKV_ERR_NO_BLOCKS", 5: "AKV_ERR_CAPACITY", 6: "AKV_ERR_HIP",
          7: "AKV_ERR_SCRATCH"}
KERNELS = {"plan": 0, "move": 1, "commit": 2, "attn": 3, "combine": 4, "append": 5,
           "segment": 6, "release": 7, "rounds": 8}
PAGE = 16


class AkvError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS.get(code, code)}")
        self.code = code


class AkvCacheDesc(C.Structure):
    _fields_ = [
        ("n_layers", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
        ("block_size", C.c_int32), ("n_blocks", C.c_int32), ("n_seqs", C.c_int32),
        ("max_blocks_per_seq", C.c_int32), ("rope_base", C.c_double),
        ("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("block_table", C.c_void_p),
        ("seq_lens", C.c_void_p), ("next_pos", C.c_void_p), ("positions", C.c_void_p),
        ("token_ids", C.c_void_p), ("free_stack", C.c_void_p), ("free_count", C.c_void_p),
        ("scratch", C.c_void_p), ("scratch_bytes", C.c_size_t),
        ("rotary_dim", C.c_int32), ("inv_freq", C.c_void_p), ("layer_window", C.c_void_p),
    ]


_lib = None
_P = C.c_void_p


def lib() -> C.CDLL:
    """Load libakv.so once; raise loudly when it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "or python -m agent_kv_cache_amd.build")
    L = C.CDLL(LIB_PATH)
    sig = {
        "akv_scratch_bytes": (C.c_size_t, [C.POINTER(AkvCacheDesc)]),
        "akv_cache_init": (C.c_int, [C.POINTER(AkvCacheDesc), C.POINTER(_P)]),
        "akv_cache_free": (None, [_P]),
        "akv_cache_reset": (C.c_int, [_P, _P, _P]),
        "akv_append": (C.c_int, [_P, _P, C.c_int64, _P, _P, _P, _P]),
        "akv_append_rope": (C.c_int, [_P, _P, C.c_int64, _P, _P, _P, _P]),
        "akv_release": (C.c_int, [_P, _P, _P]),
        "akv_drop": (C.c_int, [_P, _P, _P]),
        "akv_reposition": (C.c_int, [_P, _P, _P, _P]),
        "akv_drop_reposition": (C.c_int, [_P, _P, _P, _P]),
        "akv_fork": (C.c_int, [_P, _P, _P, C.c_int, _P, _P]),
        "akv_decode_workspace_bytes": (C.c_size_t, [_P, C.c_int32, C.c_int32]),
        "akv_decode_attention": (C.c_int, [_P, _P, _P, C.c_int32, C.c_int32, C.c_int32, _P,
                                           _P, C.c_size_t, _P]),
        "akv_decode_attention_noalloc": (C.c_int, [_P, _P, _P, C.c_int32, C.c_int32, C.c_int32,
                                                   _P, _P]),
        "akv_segment_attention": (C.c_int, [_P, _P, _P, _P, C.c_int32, C.c_int32, C.c_int32,
                                            C.c_int32, C.c_int32, _P, _P]),
        "akv_query_state": (C.c_int, [_P, _P, _P, _P, _P, _P, _P]),
        "akv_sync_status": (C.c_int, [_P, _P]),
        "akv_status_string": (C.c_char_p, [C.c_int]),
        "akv_profile_enable": (C.c_int, [_P, C.c_int]),
        "akv_profile_read": (C.c_int, [_P, C.c_int, C.POINTER(C.c_double),
                                       C.POINTER(C.c_int64), C.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def header_functions() -> list:
    """Names of the functions include/akv.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(akv_[a-z_]+)\s*\(", txt)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(code: int, what: str):
    if code != 0:
        raise AkvError(code, what)


class AkvCache:
    """A paged bf16 KV cache in device memory plus its libakv handle.

    Tensors (all on `device`, owned here):
      k_pool, v_pool : bf16 [L][NB][Hkv][16][d]
      positions, token_ids : int32 [NB][16]
      meta : int32 buffer holding block_table [B][maxpg], seq_lens [B],
             next_pos [B], free_count [1] and free_stack [NB] as views, so the
             whole per-sequence state can be snapshotted with one copy.
    """

    def __init__(self, n_layers: int, n_kv_heads: int, head_dim: int, n_blocks: int,
                 n_seqs: int, max_blocks_per_seq: int, rope_base: float,
                 device: str = "cuda", k_pool=None, v_pool=None, rotary_dim: int = 0,
                 inv_freq=None, layer_window=None):
        """k_pool / v_pool: optional caller-placed bf16 tensors of shape
        [L][NB][Hkv][16][d] (e.g. views of one larger buffer).
        rotary_dim: partial RoPE (0 = head_dim); inv_freq: host sequence of
        rotary_dim/2 frequencies (None = rope_base^(-2i/r)); layer_window:
        host sequence of per-layer sliding-window lengths (0 = full)."""
        import numpy as np
        import torch
        self.L, self.H, self.D = n_layers, n_kv_heads, head_dim
        self.NB, self.B, self.maxpg = n_blocks, n_seqs, max_blocks_per_seq
        self.S = max_blocks_per_seq * PAGE
        self.rope_base = float(rope_base)
        self.device = torch.device(device)
        shape = (n_layers, n_blocks, n_kv_heads, PAGE, head_dim)
        for t in (k_pool, v_pool):
            if t is not None and (tuple(t.shape) != shape or t.dtype != torch.bfloat16
                                  or not t.is_contiguous()):
                raise ValueError(f"pool tensors must be contiguous bf16 {shape}")
        self.k_pool = k_pool if k_pool is not None else torch.empty(
            shape, dtype=torch.bfloat16, device=self.device)
        self.v_pool = v_pool if v_pool is not None else torch.empty(
            shape, dtype=torch.bfloat16, device=self.device)
        self.positions = torch.empty((n_blocks, PAGE), dtype=torch.int32, device=self.device)
        self.token_ids = torch.empty((n_blocks, PAGE), dtype=torch.int32, device=self.device)
        nt = n_seqs * max_blocks_per_seq
        self._o_lens = nt
        self._o_next = nt + n_seqs
        self._o_fc = nt + 2 * n_seqs
        self._o_fs = self._o_fc + 4
        self.meta = torch.zeros(self._o_fs + n_blocks, dtype=torch.int32, device=self.device)
        self.block_table = self.meta[:nt].view(n_seqs, max_blocks_per_seq)
        self.seq_lens = self.meta[self._o_lens:self._o_lens + n_seqs]
        self.next_pos = self.meta[self._o_next:self._o_next + n_seqs]
        self.free_count = self.meta[self._o_fc:self._o_fc + 1]
        self.free_stack = self.meta[self._o_fs:]
        desc = AkvCacheDesc(n_layers, n_kv_heads, head_dim, PAGE, n_blocks, n_seqs,
                            max_blocks_per_seq, self.rope_base)
        self.rotary_dim = int(rotary_dim) or head_dim
        desc.rotary_dim = int(rotary_dim)
        # host arrays are copied by akv_cache_init; keep them alive until then
        self._inv_freq = (None if inv_freq is None
                          else np.ascontiguousarray(inv_freq, dtype=np.float64).reshape(-1))
        if self._inv_freq is not None:
            if self._inv_freq.shape[0] != self.rotary_dim // 2:
                raise ValueError("inv_freq needs rotary_dim / 2 values")
            desc.inv_freq = self._inv_freq.ctypes.data
        self._window = (None if layer_window is None
                        else np.ascontiguousarray(layer_window, dtype=np.int32).reshape(-1))
        if self._window is not None:
            if self._window.shape[0] != n_layers:
                raise ValueError("layer_window needs one value per layer")
            desc.layer_window = self._window.ctypes.data
        nbytes = lib().akv_scratch_bytes(C.byref(desc))
        if nbytes == 0:
            raise AkvError(1, "akv_scratch_bytes")
        self.scratch = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        for f, t in (("k_pool", self.k_pool), ("v_pool", self.v_pool),
                     ("block_table", self.block_table), ("seq_lens", self.seq_lens),
                     ("next_pos", self.next_pos), ("positions", self.positions),
                     ("token_ids", self.token_ids), ("free_stack", self.free_stack),
                     ("free_count", self.free_count), ("scratch", self.scratch)):
            setattr(desc, f, t.data_ptr())
        desc.scratch_bytes = nbytes
        self.desc = desc
        h = _P()
        _check(lib().akv_cache_init(C.byref(desc), C.byref(h)), "akv_cache_init")
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.akv_cache_free(h)
            self.handle = None

    # -- ops ---------------------------------------------------------------
    def reset(self, page_order=None, stream=None):
        arr = None
        if page_order is not None:
            import numpy as np
            po = np.ascontiguousarray(page_order, dtype=np.int32)
            arr = po.ctypes.data_as(_P)
        _check(lib().akv_cache_reset(self.handle, arr, _stream(stream)), "akv_cache_reset")

    def append(self, counts, n_new: int, k_new=None, v_new=None, token_ids=None, stream=None):
        _check(lib().akv_append(self.handle, _ptr(counts), int(n_new), _ptr(k_new), _ptr(v_new),
                                _ptr(token_ids), _stream(stream)), "akv_append")

    def append_rope(self, counts, n_new: int, k_raw=None, v_new=None, token_ids=None,
                    stream=None):
        """akv_append with the keys given before RoPE (rotated at their new
        positions inside the append)."""
        _check(lib().akv_append_rope(self.handle, _ptr(counts), int(n_new), _ptr(k_raw),
                                     _ptr(v_new), _ptr(token_ids), _stream(stream)),
               "akv_append_rope")

    def release(self, release_mask, stream=None):
        """Free the flagged sequences (uint8 device [B]): pages back to the
        free stack, length and next position 0."""
        _check(lib().akv_release(self.handle, _ptr(release_mask), _stream(stream)), "akv_release")

    def drop(self, drop_mask, stream=None):
        _check(lib().akv_drop(self.handle, _ptr(drop_mask), _stream(stream)), "akv_drop")

    def reposition(self, old_pos=None, new_pos=None, stream=None):
        _check(lib().akv_reposition(self.handle, _ptr(old_pos), _ptr(new_pos), _stream(stream)),
               "akv_reposition")

    def drop_reposition(self, drop_mask, new_pos=None, stream=None):
        _check(lib().akv_drop_reposition(self.handle, _ptr(drop_mask), _ptr(new_pos),
                                         _stream(stream)), "akv_drop_reposition")

    def fork(self, dst_of, drop_mask=None, reposition: bool = False, new_pos=None,
             stream=None):
        """New position versions: dst_of[b] = destination sequence of source b
        or -1 (host list)."""
        import numpy as np
        arr = np.ascontiguousarray(dst_of, dtype=np.int32)
        if arr.shape != (self.B,):
            raise ValueError("dst_of needs one entry per sequence")
        _check(lib().akv_fork(self.handle, arr.ctypes.data_as(_P), _ptr(drop_mask),
                              int(bool(reposition)), _ptr(new_pos), _stream(stream)), "akv_fork")

    def decode_workspace_bytes(self, n_layers: int, n_q_heads: int) -> int:
        return int(lib().akv_decode_workspace_bytes(self.handle, n_layers, n_q_heads))

    def decode_attention(self, q, out, workspace, active_len=None, layer_begin: int = 0,
                         n_layers: Optional[int] = None, stream=None):
        nL = self.L - layer_begin if n_layers is None else n_layers
        Hq = q.shape[-2]
        _check(lib().akv_decode_attention(self.handle, _ptr(q), _ptr(active_len), layer_begin,
                                          nL, Hq, _ptr(out), _ptr(workspace),
                                          workspace.numel() * workspace.element_size()
                                          if workspace is not None else 0, _stream(stream)),
               "akv_decode_attention")

    def decode_attention_noalloc(self, q, out, active_len=None, layer_begin: int = 0,
                                 n_layers: Optional[int] = None, stream=None):
        """akv_decode_attention with the library's static per-GPU workspace
        (allocates nothing; concurrent calls on one GPU race)."""
        nL = self.L - layer_begin if n_layers is None else n_layers
        _check(lib().akv_decode_attention_noalloc(self.handle, _ptr(q), _ptr(active_len),
                                                  layer_begin, nL, q.shape[-2], _ptr(out),
                                                  _stream(stream)),
               "akv_decode_attention_noalloc")

    def segment_attention(self, q, seg_seq, seg_q_off, max_q: int, out, layer_begin: int = 0,
                          n_layers: Optional[int] = None, stream=None):
        """q/out [n_q][n_layers][Hq][d] bf16; seg_seq [n_seg], seg_q_off
        [n_seg + 1] int32 device arrays; max_q >= every segment's rows."""
        nL = self.L - layer_begin if n_layers is None else n_layers
        n_seg = seg_seq.numel()
        if seg_q_off.numel() != n_seg + 1:
            raise ValueError("seg_q_off needs n_segments + 1 entries")
        _check(lib().akv_segment_attention(self.handle, _ptr(q), _ptr(seg_seq), _ptr(seg_q_off),
                                           n_seg, int(max_q), layer_begin, nL, q.shape[-2],
                                           _ptr(out), _stream(stream)),
               "akv_segment_attention")

    def sync_status(self, stream=None) -> int:
        return int(lib().akv_sync_status(self.handle, _stream(stream)))

    def profile_enable(self, on: bool = True):
        _check(lib().akv_profile_enable(self.handle, int(on)), "akv_profile_enable")

    def profile_read(self, kernel: str, reset: bool = False):
        ms, n = C.c_double(), C.c_int64()
        _check(lib().akv_profile_read(self.handle, KERNELS[kernel], C.byref(ms), C.byref(n),
                                      int(reset)), "akv_profile_read")
        return ms.value, n.value

    # -- state export (for checks) -------------------------------------------
    def query_state(self, stream=None, with_last_src: bool = False):
        """akv_query_state: device int32 tensors (lens [B], next_pos [B],
        positions [B][S], token_ids [B][S]) in active order, -1 past each
        length; with_last_src adds the gather map of the last drop /
        reposition / fork ([B][S], -1 where the call wrote nothing)."""
        import torch
        mk = lambda *sh: torch.empty(sh, dtype=torch.int32, device=self.device)
        lens, nxt, pos, tok = mk(self.B), mk(self.B), mk(self.B, self.S), mk(self.B, self.S)
        lsrc = mk(self.B, self.S) if with_last_src else None
        _check(lib().akv_query_state(self.handle, _ptr(lens), _ptr(nxt), _ptr(pos), _ptr(tok),
                                     _ptr(lsrc), _stream(stream)), "akv_query_state")
        return (lens, nxt, pos, tok, lsrc) if with_last_src else (lens, nxt, pos, tok)

    def last_src(self, b: int):
        """Host int64 array: sequence b's gather map of the last drop /
        reposition / fork (up to its first -1)."""
        import numpy as np
        row = self.query_state(with_last_src=True)[4][b].cpu().numpy().astype(np.int64)
        neg = np.flatnonzero(row < 0)
        return row[:neg[0]] if neg.size else row

    def seq_state(self, b: int):
        """(token_ids, positions, page ids) of sequence b's active entries, on the host
        (ids and positions through akv_query_state; page ids read from the table)."""
        import numpy as np
        lens, _, pos, tok = self.query_state()
        n = int(lens[b].item())
        npg = (n + PAGE - 1) // PAGE
        pages = self.block_table[b, :npg].cpu().numpy()
        return (tok[b, :n].cpu().numpy().astype(np.int64),
                pos[b, :n].cpu().numpy().astype(np.int64), pages)

    def gather_rows(self, b: int, layer: int, which: str = "k"):
        """bf16 rows [n, Hkv, d] of sequence b at `layer`, in active order (device tensor)."""
        n = int(self.seq_lens[b].item())
        npg = (n + PAGE - 1) // PAGE
        pool = self.k_pool if which == "k" else self.v_pool
        pages = self.block_table[b, :npg].long()
        rows = pool[layer, pages]                      # [npg, H, 16, d]
        return rows.permute(0, 2, 1, 3).reshape(npg * PAGE, self.H, self.D)[:n]
