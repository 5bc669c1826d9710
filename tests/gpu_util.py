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
               gen_device: str = "cpu", with_kv: bool = True, seqs=None) -> O.OracleCache:
    """Oracle holding the same seeded inputs as harness.fill (optionally only
    some layers: then the oracle's layer axis indexes `layers`; optionally
    only some sequences: then oracle sequence i is sequence seqs[i])."""
    lay = list(range(shape.n_layers)) if layers is None else list(layers)
    sel = list(range(len(seq_lens))) if seqs is None else list(seqs)
    oc = O.OracleCache(len(lay), shape.n_kv_heads, shape.head_dim, shape.rope_base,
                       n_seqs=len(sel), with_kv=with_kv)
    for i, b in enumerate(sel):
        n = seq_lens[b]
        for c in range((int(n) + Hn.CHUNK - 1) // Hn.CHUNK):
            m = min(Hn.CHUNK, int(n) - c * Hn.CHUNK)
            tid = (b << 24) + c * Hn.CHUNK + np.arange(m)
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


def q_tensor(shape: Shape, B: int, n_layers: int, seed: int, device="cpu"):
    return randn_bf16((B, n_layers, shape.n_q_heads, shape.head_dim), seed, device=device)


def check_attention(cache, oc: O.OracleCache, q, out, layers=None, active=None, tol=1e-2,
                    seqs=None):
    """out [B][nL][Hq][d] vs the fp64 oracle; returns the max abs error.
    Oracle sequence i is cache sequence seqs[i]."""
    qn = to_f64(q)
    on = to_f64(out)
    lay = list(range(q.shape[1])) if layers is None else list(layers)
    sel = list(range(len(oc.seqs))) if seqs is None else list(seqs)
    worst = 0.0
    for i, b in enumerate(sel):
        n = None if active is None else int(active[b])
        ref = oc.decode_attention(i, qn[b][lay] if layers is not None else qn[b], n)
        got = on[b][lay] if layers is not None else on[b]
        err = float(np.abs(got - ref).max()) if ref.size else 0.0
        worst = max(worst, err)
    assert worst <= tol, worst
    return worst
