"""Helpers for the GPU parity tests: mirror seeded inputs into the oracle and
compare the device state with it.  Test infrastructure only."""
from __future__ import annotations

import sys
from typing import List, Optional, Sequence

import numpy as np

from agent_kv_cache_amd import harness as Hn
from agent_kv_cache_amd.workloads import Shape, randn_bf16
from oracle import akv_oracle as O


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_for(shape: Shape, seq_lens: Sequence[int], data_seed: int, layers=None,
               gen_device: str = "cpu", with_kv: bool = True, seqs=None,
               rotary_dim=None, theta=None, window=None) -> O.OracleCache:
    """Oracle holding the same seeded inputs as harness.fill (optionally only
    some layers: then the oracle's layer axis indexes `layers`; optionally
    only some sequences: then oracle sequence i is sequence seqs[i]).
    rotary_dim / theta / window (per layer of the full cache) as in
    OracleCache."""
    lay = list(range(shape.n_layers)) if layers is None else list(layers)
    sel = list(range(len(seq_lens))) if seqs is None else list(seqs)
    win = None if window is None else [window[l] for l in lay]
    oc = O.OracleCache(len(lay), shape.n_kv_heads, shape.head_dim, shape.rope_base,
                       n_seqs=len(sel), with_kv=with_kv, rotary_dim=rotary_dim, theta=theta,
                       window=win)
    for i, b in enumerate(sel):
        n = seq_lens[b]
        for c in range((int(n) + Hn.CHUNK - 1) // Hn.CHUNK):
            m = min(Hn.CHUNK, int(n) - c * Hn.CHUNK)
            tid = Hn.default_token_base(b) + c * Hn.CHUNK + np.arange(m)
            if with_kv:
                k = Hn.seq_chunk(shape, data_seed, b, c, m, "k", gen_device)[lay]
                v = Hn.seq_chunk(shape, data_seed, b, c, m, "v", gen_device)[lay]
                oc.append(i, tid, to_f64(k.permute(1, 0, 2, 3)), to_f64(v.permute(1, 0, 2, 3)))
            else:
                oc.append(i, tid)
    return oc


def check_meta(cache, oc: O.OracleCache, seqs=None):
    """Token ids (compaction indices), positions, lengths, next_pos: bit-exact.
    Oracle sequence i is cache sequence seqs[i] (default: the same index)."""
    lens = cache.seq_lens.cpu().numpy()
    nxt = cache.next_pos.cpu().numpy()
    sel = list(range(len(oc.seqs))) if seqs is None else list(seqs)
    for i, s in enumerate(oc.seqs):
        b = sel[i]
        assert lens[b] == len(s), (b, lens[b], len(s))
        assert nxt[b] == s.next_pos, (b, nxt[b], s.next_pos)
        tok, pos, _ = cache.seq_state(b)
        assert np.array_equal(tok, s.token_ids), b
        assert np.array_equal(pos, s.pos), b


def check_kv(cache, oc: O.OracleCache, layers=None, k_ulp: int = 1, seqs=None):
    """K within k_ulp bf16 steps of the oracle's bf16 value, V bit-exact.
    Oracle sequence i is cache sequence seqs[i].  Returns the largest K ulp
    distance seen."""
    lay = list(range(cache.L)) if layers is None else list(layers)
    sel = list(range(len(oc.seqs))) if seqs is None else list(seqs)
    worst = 0
    for i, b in enumerate(sel):
        s = oc.seqs[i]
        for oi, l in enumerate(lay):
            kg = bits(cache.gather_rows(b, l, "k"))
            vg = bits(cache.gather_rows(b, l, "v"))
            ko = O.bf16_bits(s.k[:, oi])
            vo = O.bf16_bits(s.v[:, oi])
            assert kg.shape == ko.shape, (kg.shape, ko.shape)
            if ko.size:
                dist = O.bf16_ulp_distance(kg, ko)
                worst = max(worst, int(dist.max()))
                assert dist.max() <= k_ulp, (b, l, int(dist.max()))
            assert np.array_equal(vg, vo), (b, l)
    return worst


def oracle_from_device(cache, b: int, layers, rope_base: float, **kw) -> O.OracleCache:
    """A one-sequence oracle holding sequence b's current device state: token
    ids, positions and next position, and the exact bf16 K/V bytes of the
    listed layers (the oracle's layer axis indexes `layers`).  Used to hold a
    single op to the per-op bar: the oracle applies the op to the very bytes
    the GPU started from."""
    import torch
    tok, pos, _ = cache.seq_state(b)
    oc = O.OracleCache(len(layers), cache.H, cache.D, rope_base, n_seqs=1, **kw)
    s = oc.seqs[0]
    s.token_ids = tok.astype(np.int64)
    s.pos = pos.astype(np.int64)
    s.next_pos = int(cache.next_pos[b].item())
    s.k = np.stack([to_f64(cache.gather_rows(b, l, "k")) for l in layers], axis=1)
    s.v = np.stack([to_f64(cache.gather_rows(b, l, "v")) for l in layers], axis=1)
    assert s.k.shape == (len(tok), len(layers), cache.H, cache.D)
    return oc


def share_counts(cache):
    """Reference counts the library keeps: the int32 per-page array in its
    scratch (extra holders beyond the first)."""
    import torch
    # the layout is internal; recompute its offset the way the library does
    # (256-B aligned regions in a fixed order) -- test-only introspection
    B, S, NB, L = cache.B, cache.S, cache.NB, cache.L
    al = lambda x: (x + 255) & ~255
    o = 0
    o = al(o + 64 * 4)                 # control words
    o = al(o + 64 * 8)                 # frequencies
    o = al(o + B * 24 * 4)             # per-sequence records
    o = al(o + B * S * 4)              # gather map
    o = al(o + B * S * 4)              # rotation deltas
    o = al(o + NB * 4)                 # staging
    o = al(o + B * ((S // 16 + 255) // 256) * 2 * 4)   # plan chunks
    o = al(o + B * 4)                  # fork map
    o = al(o + L * 4)                  # windows
    o = al(o + B * S * 4)              # last_src
    o = al(o + 64 * 16 * 4)            # groups
    return cache.scratch[o:o + NB * 4].view(torch.int32).cpu().numpy()


def check_pool(cache):
    """Every page free exactly once with no holder, or held by exactly
    1 + share[p] page-table entries and not free."""
    lens = cache.seq_lens.cpu().numpy()
    tab = cache.block_table.cpu().numpy()
    held = np.zeros(cache.NB, np.int64)
    for b in range(cache.B):
        pg = tab[b, :Hn.pages_for(int(lens[b]))]
        assert (pg >= 0).all()
        np.add.at(held, pg, 1)
    fc = int(cache.free_count.item())
    free = cache.free_stack[:fc].cpu().numpy()
    assert len(np.unique(free)) == fc, "a page is on the free stack twice"
    assert (held[free] == 0).all(), "a free page is still held"
    share = share_counts(cache)
    hp = np.flatnonzero(held)
    assert np.array_equal(held[hp], 1 + share[hp]), "reference counts differ from the tables"
    assert fc + len(hp) == cache.NB, "pages lost"
    return int(held.max()) if hp.size else 0


def q_tensor(shape: Shape, B: int, n_layers: int, seed: int, device="cpu"):
    return randn_bf16((B, n_layers, shape.n_q_heads, shape.head_dim), seed, device=device)


# The attention bar: |got - ref| <= 1e-2 + h(got), where h(x) is half the
# bf16 spacing of the binade holding |x| -- exactly the largest error of
# rounding the kernel's fp32 result to the bf16 output (the fp32 value o and
# its rounding got = bf16(o) satisfy h(|o|) <= h(|got|)).  h is 2^-9 below
# 1, 2^-8 in [1, 2), 2^-7 in [2, 4); it only matters where few entries are
# visible and |o| approaches |v|.  Every check also reports the raw max
# |got - ref|.
TOL = 1e-2


def bf16_half_spacing(x) -> np.ndarray:
    """Half the bf16 spacing at |x|: 2^(e-9) for |x| in [2^(e-1), 2^e), the
    subnormal spacing's half 2^-134 below 2^-126, and 0 at 0."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)
    return np.where(ax > 0, np.ldexp(1.0, np.maximum(e - 9, -134)), 0.0)


def attn_errors(got, ref):
    """(raw max |got - ref|, max of |got - ref| - h(got)); the second is the
    figure held to 1e-2.  A non-finite output counts as an infinite error."""
    if ref.size == 0:
        return 0.0, 0.0
    if not np.isfinite(got).all():
        return float("inf"), float("inf")
    d = np.abs(got - ref)
    return float(d.max()), float((d - bf16_half_spacing(got)).max())


def check_attention(cache, oc: O.OracleCache, q, out, layers=None, active=None, tol=TOL,
                    seqs=None, what="attention"):
    """out [B][nL][Hq][d] vs the fp64 oracle.  Asserts the bar above and
    returns the raw max |got - ref|.  Oracle sequence i is cache sequence
    seqs[i]."""
    qn = to_f64(q)
    on = to_f64(out)
    lay = list(range(q.shape[1])) if layers is None else list(layers)
    sel = list(range(len(oc.seqs))) if seqs is None else list(seqs)
    raw = bar = 0.0
    for i, b in enumerate(sel):
        n = None if active is None else int(active[b])
        ref = oc.decode_attention(i, qn[b][lay] if layers is not None else qn[b], n)
        got = on[b][lay] if layers is not None else on[b]
        r, e = attn_errors(got, ref)
        raw, bar = max(raw, r), max(bar, e)
    say(f"{what}: max |got - ref| {raw:.3e}; less the output's bf16 half-spacing {bar:.3e} "
        f"(bar {tol:g})")
    assert bar <= tol, (raw, bar)
    return raw


def append_seeded(cache, oc, sh, per_seq, seed, tid_base):
    """Append per_seq[b] seeded tokens to every sequence b, on both sides."""
    B = cache.B
    N = int(sum(per_seq))
    if N == 0:
        return
    k = randn_bf16((sh.n_layers, N, sh.n_kv_heads, sh.head_dim), seed)
    v = randn_bf16((sh.n_layers, N, sh.n_kv_heads, sh.head_dim), seed + 1)
    tid = np.arange(N, dtype=np.int64) + tid_base
    import torch
    cache.append(torch.tensor(per_seq, dtype=torch.int32, device=cache.device), N,
                 k.to(cache.device), v.to(cache.device),
                 torch.tensor(tid, dtype=torch.int32, device=cache.device))
    o = 0
    for b in range(B):
        sl = slice(o, o + per_seq[b])
        if per_seq[b]:
            oc.append(b, tid[sl], to_f64(k[:, sl].permute(1, 0, 2, 3)),
                      to_f64(v[:, sl].permute(1, 0, 2, 3)))
        o += per_seq[b]


def snapshot(cache, b):
    tok, pos, _ = cache.seq_state(b)
    ks = [bits(cache.gather_rows(b, l, "k")) for l in range(cache.L)]
    vs = [bits(cache.gather_rows(b, l, "v")) for l in range(cache.L)]
    return tok, pos, int(cache.next_pos[b]), ks, vs


def same_state(a, b):
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]
    for x, y in zip(a[3] + a[4], b[3] + b[4]):
        assert np.array_equal(x, y)


def run_segments(cache, q, segs, max_q=None, layer_begin=0, n_layers=None):
    """segs: list of (sequence, row count); q rows are laid out segment by segment."""
    import torch
    dev = cache.device
    seq = torch.tensor([s for s, _ in segs], dtype=torch.int32, device=dev)
    off = torch.tensor(np.concatenate([[0], np.cumsum([n for _, n in segs])]).astype(np.int32),
                       device=dev)
    out = torch.full_like(q, float("nan"))
    mq = max([n for _, n in segs] + [1]) if max_q is None else max_q
    cache.segment_attention(q, seq, off, mq, out, layer_begin=layer_begin, n_layers=n_layers)
    return out


def check_segments(oc, q, out, segs, oracle_seq=None, tol=TOL, rows=None):
    """Segment attention vs the oracle (bar as check_attention; returns the
    raw max |got - ref|).  rows: optional list, per segment, of the row
    indices to check (the oracle then runs only the segment's last rows from
    the first checked one on: a segment's last k rows are a segment of their
    own over the same sequence)."""
    qn, on = to_f64(q), to_f64(out)
    o = 0
    pairs, picks = [], []
    for j, (s, n) in enumerate(segs):
        sel = np.arange(n) if rows is None else np.asarray(rows[j], dtype=np.int64)
        lo = int(sel.min()) if sel.size else n
        pairs.append(((s if oracle_seq is None else oracle_seq[s]), qn[o + lo:o + n]))
        picks.append((o, lo, sel))
        o += n
    refs = O.segment_attention(oc, pairs)
    raw = bar = 0.0
    for (o, lo, sel), ref in zip(picks, refs):
        if sel.size:
            r, e = attn_errors(on[o + sel], ref[sel - lo])
            raw, bar = max(raw, r), max(bar, e)
    say(f"segments: max |got - ref| {raw:.3e}; less the output's bf16 half-spacing {bar:.3e} "
        f"(bar {tol:g})")
    assert bar <= tol, (raw, bar)
    return raw
