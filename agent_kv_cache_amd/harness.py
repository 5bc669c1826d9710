"""Set-up helpers for caches shaped like the pages' agent workloads.

Allocation and filling only: sizes the page pool, appends seeded bf16 data
through akv_append in chunks, uploads drop masks.  No step of the method is
computed here.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .binding import PAGE, AkvCache
from .workloads import Shape, randn_bf16

CHUNK = 4096  # tokens per generated data chunk (fixes the seed of every chunk)


def pages_for(n: int) -> int:
    return (int(n) + PAGE - 1) // PAGE


def moved_pages(n: int, mask: Optional[np.ndarray]) -> int:
    """Upper bound of fresh pages a drop of `mask` over n entries takes."""
    if mask is None or not mask[:n].any():
        return 0
    f = int(np.flatnonzero(mask[:n])[0])
    r = n - int(mask[:n].astype(bool).sum())
    return max(0, pages_for(r) - f // PAGE)


def chunk_seed(data_seed: int, b: int, c: int, which: int) -> int:
    return (data_seed * 1_000_003 + b * 65_537 + c * 31 + which) % (2 ** 63)


def seq_chunk(shape: Shape, data_seed: int, b: int, c: int, n: int, which: str, device):
    """bf16 [L, n, Hkv, d] data of tokens [c*CHUNK, c*CHUNK + n) of sequence b."""
    w = 0 if which == "k" else 1
    return randn_bf16((shape.n_layers, n, shape.n_kv_heads, shape.head_dim),
                      chunk_seed(data_seed, b, c, w), device=device)


def make_cache(shape: Shape, seq_lens: Sequence[int], extra_pages: int,
               max_blocks_per_seq: Optional[int] = None, device: str = "cuda",
               **cache_kw) -> AkvCache:
    """cache_kw: rotary_dim / inv_freq / layer_window, passed to AkvCache."""
    nb = sum(pages_for(n) for n in seq_lens) + int(extra_pages)
    maxpg = max_blocks_per_seq or max(1, max(pages_for(n) for n in seq_lens))
    return AkvCache(shape.n_layers, shape.n_kv_heads, shape.head_dim, max(nb, 1),
                    len(seq_lens), maxpg, shape.rope_base, device=device, **cache_kw)


def default_token_base(b: int) -> int:
    """First token id of sequence b in the seeded fills: (b mod 128) * 2^24,
    so that every id of a sequence up to 2^24 tokens fits int32 (the cache's
    id type); ids repeat across sequences 128 apart."""
    return (int(b) & 127) << 24


def fill(cache: AkvCache, shape: Shape, seq_lens: Sequence[int], data_seed: int,
         gen_device: str = "cuda", token_base: Optional[List[int]] = None,
         max_tokens_per_call: int = 16384, progress=None):
    """Append every sequence's tokens chunk by chunk (seeded per chunk).

    Token ids of sequence b are token_base[b] + 0, 1, ... (default
    default_token_base(b)).
    Each akv_append call carries at most `max_tokens_per_call` tokens so the
    set-up temporaries stay small next to a large pool.
    """
    import torch
    dev = cache.device
    B = len(seq_lens)
    nchunks = max((int(n) + CHUNK - 1) // CHUNK for n in seq_lens) if B else 0
    for c in range(nchunks):
        group = []
        for b, n in enumerate(seq_lens):
            m = max(0, min(CHUNK, int(n) - c * CHUNK))
            if m:
                group.append((b, m))
        while group:
            take, tot = [], 0
            while group and (not take or tot + group[0][1] <= max_tokens_per_call):
                take.append(group.pop(0))
                tot += take[-1][1]
            counts = [0] * B
            ks, vs, toks = [], [], []
            for b, m in take:
                counts[b] = m
                ks.append(seq_chunk(shape, data_seed, b, c, m, "k", gen_device).to(dev))
                vs.append(seq_chunk(shape, data_seed, b, c, m, "v", gen_device).to(dev))
                base = default_token_base(b) if token_base is None else token_base[b]
                toks.append(torch.arange(base + c * CHUNK, base + c * CHUNK + m,
                                         dtype=torch.int32, device=dev))
            k = torch.cat(ks, dim=1).contiguous() if len(ks) > 1 else ks[0]
            v = torch.cat(vs, dim=1).contiguous() if len(vs) > 1 else vs[0]
            del ks, vs
            cache.append(torch.tensor(counts, dtype=torch.int32, device=dev), tot, k, v,
                         torch.cat(toks))
            del k, v
        if progress:
            progress(c + 1, nchunks)


def mask_tensor(cache: AkvCache, masks: Sequence[Optional[np.ndarray]]):
    """u8 [B][S] device mask, row b = masks[b] padded with zeros."""
    import torch
    m = np.zeros((cache.B, cache.S), dtype=np.uint8)
    for b, mb in enumerate(masks):
        if mb is not None:
            m[b, :len(mb)] = mb
    return torch.from_numpy(m).to(cache.device)


def pos_tensor(cache: AkvCache, rows: Sequence[Optional[np.ndarray]]):
    """int32 [B][S] device array, row b = rows[b] padded with zeros."""
    import torch
    a = np.zeros((cache.B, cache.S), dtype=np.int32)
    for b, r in enumerate(rows):
        if r is not None:
            a[b, :len(r)] = r
    return torch.from_numpy(a).to(cache.device)
