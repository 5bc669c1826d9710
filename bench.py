#!/usr/bin/env python3
"""Benchmark of the agent-cache hot path on one MI355X.

One step = restore the per-sequence state (page table, lengths, next
positions, free stack: one small device copy) + fused drop+reposition
(plan, move/re-rotate, commit kernels) + decode attention over all layers
(split-K kernel + combine).

The default run measures every configuration of the method's workloads and
prints ONE JSON line.  The headline (`value`, `roofline`, `cpu_baseline`) is
the largest single-GPU configuration, the ragged batch (64 sequences of
8K..64K tokens, Llama-8B KV shape, shuffled pages, ~40% dropped, ~155 GB of
KV); the Llama-8B-shaped single sequence, the one-layer 4K case, the
Llama-70B shape and the 50-turn history follow under `configs` (the
latency-bound one-layer step also as one HIP graph replay, `graph_ms_per_step`).
`--workload NAME` runs one of them (or the restore / append workloads) alone.

`value` = algorithmic KV bytes of the whole step (drop+reposition and
decode) / wall time per step, in GB/s.  The `roofline` object covers the
dominant kernel (per-launch algorithmic bytes / average launch time from HIP
events recorded on the launch stream); `parts` gives both parts, with the
move and decode kernels' per-step median / min / max from a second, untimed
pass of the same steps; `cpu_baseline` times the fp64 oracle on a bounded
sample in a process pool on the host's cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "KV GB/s for drop+reposition and decode attention; % of HBM peak, 1 GPU"


def algorithmic_bytes(shape, seq_lens, masks, layer_window=None):
    """Bytes the method must move, for caches whose positions are 0..n-1.

    drop+reposition: survivors whose slot changes (at or after the first
    dropped entry) read and write K and V once; survivors whose position
    changes in place read and write K (none for canonical input positions);
    plus the mask bytes, the positions read for every survivor and the
    positions and token ids moved with the moved rows.  Partial RoPE moves
    the same bytes (the unrotated part of K is copied).
    decode: K and V of every entry the query sees once, q in and out, the
    page ids.  After the canonical reposition a sliding window of W reads
    the last W - 1 survivors of its layer.
    """
    L, H, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
    lrow = H * D * 2                         # one token's K (or V), one layer
    row = L * lrow                           # all layers
    win = [0] * L if layer_window is None else list(layer_window)
    moved = surv = total = pages = seen = 0
    for n, m in zip(seq_lens, masks):
        m = np.asarray(m[:n]).astype(bool)
        r = n - int(m.sum())
        surv += r
        total += n
        pages += (r + 15) // 16
        seen += sum(min(r, w - 1) if w else r for w in win)
        if m.any():
            f = int(np.flatnonzero(m)[0])
            moved += r - f
    b_move = moved * (2 * row) * 2 + moved * 12
    b_dr = b_move + total + 4 * surv
    b_att = seen * 2 * lrow + 2 * (len(seq_lens) * L * shape.n_q_heads * D * 2) + 4 * pages
    return dict(moved=moved, survivors=surv, tokens=total, b_move=b_move, b_dr=b_dr,
                b_att=b_att, b_att_kv=seen * 2 * lrow)


def variant_tag(args):
    """Suffix naming a RoPE-variant run in its counter records ('' for the
    plain configuration)."""
    tag = ""
    if args.rotary_dim:
        tag += f"_rotary{args.rotary_dim}"
    if args.freq != "base":
        tag += f"_{args.freq}_freq"
    if args.window:
        tag += f"_window{args.window}" + ("_alternate" if args.window_every == 2
                                           else f"_every{args.window_every}")
    return tag


def rope_options(args, shape):
    """Cache options for the RoPE-variant runs (partial RoPE, a frequency
    table, alternating sliding-window layers), as AkvCache keywords."""
    kw = {}
    r = args.rotary_dim or shape.head_dim
    if args.rotary_dim:
        kw["rotary_dim"] = args.rotary_dim
    if args.freq != "base":
        # the published schedules, written out here for the benchmark only
        # (same definitions as the test oracle's llama3_theta / yarn_theta)
        i = np.arange(r // 2, dtype=np.float64)
        th = np.power(shape.rope_base, -2.0 * i / r)
        if args.freq == "llama3":
            C, f, lo, hi = 8192.0, 8.0, 1.0, 4.0
            w = 2 * np.pi / th
            sm = (C / w - lo) / (hi - lo)
            th = np.where(w < C / hi, th, np.where(w > C / lo, th / f,
                                                  (1 - sm) * th / f + sm * th))
        else:
            C, f = 4096.0, 32.0
            at = lambda t: r * np.log(C / (t * 2 * np.pi)) / (2 * np.log(shape.rope_base))
            a, b = max(int(np.floor(at(32.0))), 0), min(int(np.ceil(at(1.0))), r - 1)
            ramp = np.clip((i - a) / max(b - a, 1e-3), 0.0, 1.0)
            th = th * (1 - ramp) + th / f * ramp
        kw["inv_freq"] = th
    if args.window:
        kw["layer_window"] = [args.window if l % args.window_every != args.window_every - 1
                              else 0 for l in range(shape.n_layers)]
    return kw


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle (as it stands) in a process pool on the host
# ---------------------------------------------------------------------------
def host_info():
    """CPU model, logical cores this process may run on, host RAM."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    ram = None
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram = round(int(line.split()[1]) / 2 ** 20, 1)
                break
    except OSError:
        pass
    return {"cpu_model": model, "cpus_available": len(os.sched_getaffinity(0)),
            "host_ram_gib": ram}


MAX_POOL = 16       # worker processes (a one-GPU share of the host)


def _pool(n_units):
    """A spawn-context process pool (fresh interpreters that never touch the
    GPU) of min(16, available cores, units) workers, BLAS one thread each."""
    import multiprocessing as mp
    n = max(1, min(MAX_POOL, len(os.sched_getaffinity(0)), n_units))
    keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    old = {k: os.environ.get(k) for k in keys}
    for k in keys:
        os.environ[k] = "1"
    try:
        return mp.get_context("spawn").Pool(n), n
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _pool_map(fn, tasks, timeout=600.0):
    """Run fn over tasks in the pool; (results, pool wall seconds, workers).
    A pool whose workers cannot start or do not finish within `timeout` is
    terminated and the failure raised (the benchmark never waits forever)."""
    pool, nw = _pool(len(tasks))
    try:
        t0 = time.perf_counter()
        res = pool.map_async(fn, tasks, chunksize=1).get(timeout=timeout)
        wall = time.perf_counter() - t0
        pool.close()
    except BaseException:
        pool.terminate()
        raise
    finally:
        pool.join()
    return res, wall, nw


def _critical_path(results):
    """results: (pid, seconds...) per unit.  Per part, the largest per-worker
    sum of op seconds: the time the pool needs for the op work (the untimed
    conversion of each unit's inputs into the oracle's arrays excluded)."""
    per = {}
    for r in results:
        acc = per.setdefault(r[0], [0.0] * (len(r) - 1))
        for i, t in enumerate(r[1:]):
            acc[i] += t
    parts = [max(v[i] for v in per.values()) for i in range(len(results[0]) - 1)]
    total = max(sum(v) for v in per.values())
    return parts, total, len(per)


def _cpu_step_unit(task):
    """One (sequence, layer) unit in a pool worker: the oracle holds that
    layer of the sequence (with the run's partial RoPE, frequency table and
    that layer's window, if any), applies the fused drop + reposition and the
    decode attention; returns (pid, seconds of each)."""
    from oracle import akv_oracle as O
    n = task["k"].shape[0]
    oc = O.OracleCache(1, task["H"], task["D"], task["base"], rotary_dim=task.get("rotary_dim"),
                       theta=task.get("theta"),
                       window=[task["window"]] if task.get("window") else None)
    oc.append(0, np.arange(n), O.bf16_from_bits(task["k"])[:, None],
              O.bf16_from_bits(task["v"])[:, None])
    t0 = time.perf_counter()
    oc.drop_reposition(0, task["mask"])
    t1 = time.perf_counter()
    oc.decode_attention(0, task["q"][None])
    t2 = time.perf_counter()
    return os.getpid(), t1 - t0, t2 - t1


def _u16(t):
    """Host uint16 bit patterns of a bf16 tensor."""
    import torch
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def cpu_baseline(wl, layers, seqs=None, ropt=None):
    """The fp64 oracle as it stands, on a bounded sample of the workload
    (the listed layers of the listed sequences, every token), one (sequence,
    layer) unit per task of a process pool, with the run's RoPE options
    (`ropt`, as for the cache); bytes are the algorithmic bytes of the
    sample itself (its layers and sequences)."""
    import torch

    from agent_kv_cache_amd import harness as Hn
    from agent_kv_cache_amd.workloads import randn_bf16

    sh = wl.shape
    ropt = ropt or {}
    win = ropt.get("layer_window")
    seqs = list(range(wl.n_seqs)) if seqs is None else list(seqs)
    q = randn_bf16((wl.n_seqs, sh.n_layers, sh.n_q_heads, sh.head_dim), 202, device="cuda")
    tasks = []
    for b in seqs:
        n = wl.seq_lens[b]
        ks, vs = [], []
        for c in range((n + Hn.CHUNK - 1) // Hn.CHUNK):
            m = min(Hn.CHUNK, n - c * Hn.CHUNK)
            ks.append(_u16(Hn.seq_chunk(sh, wl.data_seed, b, c, m, "k", "cuda")[layers]))
            vs.append(_u16(Hn.seq_chunk(sh, wl.data_seed, b, c, m, "v", "cuda")[layers]))
        k, v = np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)
        for i, l in enumerate(layers):
            tasks.append(dict(H=sh.n_kv_heads, D=sh.head_dim, base=sh.rope_base,
                              k=np.ascontiguousarray(k[i]), v=np.ascontiguousarray(v[i]),
                              mask=np.asarray(wl.masks[b][:n]),
                              q=q[b, l].double().cpu().numpy(),
                              rotary_dim=ropt.get("rotary_dim"), theta=ropt.get("inv_freq"),
                              window=win[l] if win else 0))
    del q
    torch.cuda.empty_cache()
    res, wall, nw = _pool_map(_cpu_step_unit, tasks)
    (t_dr, t_dec), t_all, used = _critical_path(res)
    # the sample's own algorithmic bytes: its layers (with their windows) and
    # sequences, as if they were the whole cache
    ab = algorithmic_bytes(dataclasses.replace(sh, n_layers=len(layers)),
                           [wl.seq_lens[b] for b in seqs], [wl.masks[b] for b in seqs],
                           [win[l] for l in layers] if win else None)
    cpu_s = sum(r[1] + r[2] for r in res)
    variant = "".join(f", {k} {v}" for k, v in (
        ("rotary_dim", ropt.get("rotary_dim")),
        ("layer windows", sorted(set(win)) if win else None)) if v)
    if ropt.get("inv_freq") is not None:
        variant += ", explicit frequency table"
    return {
        "value": round((ab["b_dr"] + ab["b_att"]) / t_all / 1e9, 4),
        "unit": "GB/s",
        "cores": used,
        "kind": "oracle",
        "sample": f"{wl.name}: layer(s) {layers} of {sh.n_layers} x {len(seqs)} of {wl.n_seqs} "
                  f"sequence(s), every token ({len(tasks)} (sequence, layer) units); fused "
                  f"drop+reposition then decode per unit in a {nw}-process pool: "
                  f"{cpu_s:.1f} s of op work, {t_all:.2f} s on the busiest worker "
                  f"({wall:.1f} s pool wall time including unpacking the inputs); bytes are "
                  f"the sample's own algorithmic bytes{variant}",
        "drop_reposition_gbps": round(ab["b_dr"] / t_dr / 1e9, 4),
        "decode_gbps": round(ab["b_att"] / t_dec / 1e9, 4),
        **host_info(),
    }


def _cpu_append_unit(task):
    """One layer of the append in a pool worker: the oracle appends the
    layer's keys as given (plain) and, into a second empty cache, rotated at
    their positions (RoPE fused); returns (pid, seconds of each)."""
    from oracle import akv_oracle as O
    k = O.bf16_from_bits(task["k"])[:, None]
    v = O.bf16_from_bits(task["v"])[:, None]
    tid = np.arange(k.shape[0])
    kw = dict(rotary_dim=task.get("rotary_dim"), theta=task.get("theta"))
    oc = O.OracleCache(1, task["H"], task["D"], task["base"], **kw)
    t0 = time.perf_counter()
    oc.append(0, tid, k, v)
    t1 = time.perf_counter()
    oc = O.OracleCache(1, task["H"], task["D"], task["base"], **kw)
    t2 = time.perf_counter()
    oc.append_rotated(0, tid, k, v)
    t3 = time.perf_counter()
    return os.getpid(), t1 - t0, t3 - t2


def _cpu_history_unit(task):
    """One layer of the 50-turn history in a pool worker: the oracle replays
    every op on that layer (appends untimed), then the final decode."""
    from oracle import akv_oracle as O
    oc = O.OracleCache(1, task["H"], task["D"], task["base"])
    t_ops = 0.0
    for op in task["ops"]:
        if op[0] == "append":
            _, tid, k, v = op
            oc.append(0, tid, O.bf16_from_bits(k)[:, None], O.bf16_from_bits(v)[:, None])
            continue
        t0 = time.perf_counter()
        if op[0] == "drop":
            oc.drop(0, op[1])
        elif op[0] == "repos":
            oc.reposition(0)
        else:
            oc.drop_reposition(0, op[1])
        t_ops += time.perf_counter() - t0
    t0 = time.perf_counter()
    oc.decode_attention(0, task["q"][None])
    return os.getpid(), t_ops, time.perf_counter() - t0


def run_history(args):
    """The 50-turn agent history (configuration 4): appends are the model's
    work and are not timed; every drop / drop+reposition / reposition op is
    timed with the library's kernel events (plan + move + commit), and its
    algorithmic bytes are counted from the device state read back around it.
    Ends with one decode step over the final state."""
    import torch

    from agent_kv_cache_amd import harness as Hn
    from agent_kv_cache_amd import workloads as W

    sh = W.SHAPES["history_50_turns"]
    hist = W.history_50_turns()
    row = sh.n_layers * sh.n_kv_heads * sh.head_dim * 2
    # per-sequence page capacity: the run's largest active length (it also
    # bounds the move's one-shot grid, whose blocks past an op's units exit
    # at once)
    maxpg = Hn.pages_for(hist.max_active())
    cache = Hn.make_cache(sh, [1], 4096, max_blocks_per_seq=maxpg)
    cache.reset()
    dev = cache.device
    tot_bytes = tot_ms = mv_bytes = mv_ms = 0.0
    n_ops = 0
    per_op = []
    cpu_layers = list(range(0, sh.n_layers, 3))  # the CPU baseline's layer sample (12 of 36)
    cpu_ops = []                                 # the same op list for the oracle
    for op in hist.ops:
        if op[0] == "append":
            mid, n = op[1], op[2]
            k = W.randn_bf16((sh.n_layers, n, sh.n_kv_heads, sh.head_dim), 104_000 + 2 * mid, "cuda")
            v = W.randn_bf16((sh.n_layers, n, sh.n_kv_heads, sh.head_dim), 104_001 + 2 * mid, "cuda")
            tid = torch.arange(hist.msg_start[mid], hist.msg_start[mid] + n, dtype=torch.int32,
                               device=dev)
            cache.append(torch.tensor([n], dtype=torch.int32, device=dev), n, k, v, tid)
            if not args.no_cpu_baseline:
                cpu_ops.append(("append", tid.cpu().numpy().astype(np.int64),
                                _u16(k[cpu_layers]), _u16(v[cpu_layers])))
            continue
        tok0, pos0, _ = cache.seq_state(0)
        mask = (W.mask_for_messages(tok0, hist, op[1]) if op[0] != "repos"
                else np.zeros(len(tok0), np.uint8))
        if not args.no_cpu_baseline:
            cpu_ops.append((op[0], mask))
        mt = Hn.mask_tensor(cache, [mask])
        torch.cuda.synchronize()
        cache.profile_read("plan", reset=True)
        cache.profile_enable(True)
        if op[0] == "drop":
            cache.drop(mt)
        elif op[0] == "repos":
            cache.reposition()
        else:
            cache.drop_reposition(mt)
        cache.profile_enable(False)
        if cache.sync_status() != 0:
            raise RuntimeError(f"device status after {op}")
        ms = sum(cache.profile_read(k)[0] for k in ("plan", "move", "commit", "rounds"))
        mv_ms += cache.profile_read("move")[0]
        keep = mask == 0
        r = int(keep.sum())
        f = int(np.flatnonzero(mask)[0]) if mask.any() else len(mask)
        moved = int(keep[f:].sum())
        new_pos = np.arange(r) if op[0] != "drop" else pos0[keep]
        inplace = int((new_pos[:int(keep[:f].sum())] != pos0[:f][keep[:f]]).sum())
        b = moved * 4 * row + 12 * moved + inplace * 2 * row + len(mask) + 4 * r
        mv_bytes += moved * 4 * row + 12 * moved + inplace * 2 * row
        tot_bytes += b
        tot_ms += ms
        n_ops += 1
        per_op.append((op[0], len(mask), r, moved, inplace, round(ms, 4)))
    tok, _, _ = cache.seq_state(0)
    q = W.randn_bf16((1, sh.n_layers, sh.n_q_heads, sh.head_dim), 204, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(sh.n_layers, sh.n_q_heads)),
                     dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        cache.decode_attention(q, out, ws)
    torch.cuda.synchronize()
    cache.profile_read("attn", reset=True)
    cache.profile_enable(True)
    for _ in range(args.steps):
        cache.decode_attention(q, out, ws)
    cache.profile_enable(False)
    att_ms = (cache.profile_read("attn")[0] + cache.profile_read("combine")[0]) / args.steps
    b_att = len(tok) * 2 * row + 2 * sh.n_layers * sh.n_q_heads * sh.head_dim * 2
    cpu = None
    if not args.no_cpu_baseline:
        del cache, ws, out
        torch.cuda.empty_cache()
        tasks = []
        for i, l in enumerate(cpu_layers):
            ops = [("append", o[1], np.ascontiguousarray(o[2][i]), np.ascontiguousarray(o[3][i]))
                   if o[0] == "append" else o for o in cpu_ops]
            tasks.append(dict(H=sh.n_kv_heads, D=sh.head_dim, base=sh.rope_base, ops=ops,
                              q=q[0, l].double().cpu().numpy()))
        res, wall, nw = _pool_map(_cpu_history_unit, tasks)
        (t_ops, t_dec), t_all, used = _critical_path(res)
        frac = len(cpu_layers) / sh.n_layers
        cpu = {
            "value": round((tot_bytes + b_att) * frac / t_all / 1e9, 4),
            "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"history_50_turns: layers {cpu_layers} of {sh.n_layers}, the whole "
                      f"history replayed per layer ({n_ops} drop / reposition ops timed, appends "
                      f"untimed) then the decode, one layer per process of a {nw}-process pool: "
                      f"{t_all:.2f} s on the busiest worker ({wall:.1f} s pool wall time with "
                      f"the appends); bytes are the sample's share of the algorithmic bytes",
            "drop_reposition_gbps": round(tot_bytes * frac / t_ops / 1e9, 4),
            "decode_gbps": round(b_att * frac / t_dec / 1e9, 4),
            **host_info(),
        }
    out_d = {
        "metric": METRIC, "workload": "history_50_turns: 50-turn history, 131072 tokens appended, "
        "L=36 Hkv=8 d=64, 47 drops / 16 repositions, decode 64 q heads",
        "value": round((tot_bytes + b_att) / ((tot_ms + att_ms) * 1e-3) / 1e9, 2), "unit": "GB/s",
        "roofline": {"bound": "hbm", "kernel": "move_kernel",
                     "achieved": round(mv_bytes / (mv_ms * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(mv_bytes / (mv_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic": counted_traffic("move_kernel_history_50_turns_counters.json"),
                     "launch_bytes_note": "per-op launches of different sizes: achieved = "
                                          "moved bytes of all ops / move kernel time of all ops"},
        "ops": n_ops, "ops_ms_total": round(tot_ms, 4), "ops_bytes_total": int(tot_bytes),
        "move_ms_total": round(mv_ms, 4), "move_bytes_total": int(mv_bytes),
        "drop_reposition_gbps": round(tot_bytes / (tot_ms * 1e-3) / 1e9, 1),
        "drop_reposition_frac_of_peak": round(tot_bytes / (tot_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "decode_ms": round(att_ms, 4), "decode_bytes": b_att,
        "decode_gbps": round(b_att / (att_ms * 1e-3) / 1e9, 1),
        "decode_frac_of_peak": round(b_att / (att_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "final_active": len(tok),
        "per_op": per_op[-6:],
    }
    if cpu:
        out_d["cpu_baseline"] = cpu
    return out_d


def counted_traffic(name):
    """HBM bytes per launch from a committed rocprofv3 counter record under
    profiles/ (FETCH_SIZE and WRITE_SIZE scaled by what they read for a
    plain copy of known size), used only while every kernel source file the
    record names is unchanged since the counters were taken; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    pj = json.load(open(path))
    files = pj.get("source_files") or {pj.get("source_file", ""): pj.get("source_sha256")}
    for rel, digest in files.items():
        src = os.path.join(ROOT, rel)
        if not (rel and os.path.exists(src)
                and hashlib.sha256(open(src, "rb").read()).hexdigest() == digest):
            return None
    return pj.get("hbm_bytes_per_launch")


def restore_counts(rs):
    """Per-version survivors, rows, attention flops and fork bytes."""
    sh = rs.shape
    row = sh.n_layers * sh.n_kv_heads * sh.head_dim * 2
    out = []
    for m, n in rs.versions:
        ln = int((m == 0).sum())
        pairs = n * (ln - n) + n * (n + 1) // 2          # (row, visible entry) pairs
        flops = 4 * pairs * sh.head_dim * sh.n_q_heads * sh.n_layers
        # fork: the version shares the source's leading full pages before the
        # first dropped entry (the source's positions are 0..n-1, so the
        # canonical reposition changes nothing before it); every other
        # survivor's K and V are read and written, its position and token id
        # moved; the mask and the survivors' positions are read
        f = int(np.flatnonzero(m)[0]) if m.any() else len(m)
        shared = (min(f, ln) // 16) * 16
        copied = ln - shared
        fork_b = copied * (2 * row) * 2 + copied * 12 + len(m) + 4 * ln
        kv_b = ln * 2 * row
        out.append(dict(len=ln, rows=n, pairs=pairs, flops=flops, fork_bytes=fork_b, kv_bytes=kv_b,
                        shared=shared, copied=copied))
    return out


def _cpu_restore_unit(task):
    """One restore segment in a pool worker: the oracle holds layer 0, kv
    head 0 of the source, forks the segment's version (drop + canonical
    reposition) and runs the segment attention of its last rows."""
    from oracle import akv_oracle as O
    D = task["D"]
    oc = O.OracleCache(1, 1, D, task["base"], n_seqs=2)
    n = task["k"].shape[0]
    oc.append(0, np.arange(n), O.bf16_from_bits(task["k"]).reshape(n, 1, 1, D),
              O.bf16_from_bits(task["v"]).reshape(n, 1, 1, D))
    t0 = time.perf_counter()
    oc.fork(0, 1, task["mask"], reposition=True)
    t1 = time.perf_counter()
    O.segment_attention(oc, [(1, task["q"])])
    t2 = time.perf_counter()
    return os.getpid(), t1 - t0, t2 - t1


def restore_cpu_baseline(rs, rows_per_segment: int):
    """The oracle on one layer and one kv head, one segment per process of a
    pool: fork every version, then the last `rows_per_segment` rows of each
    segment (the rows with the longest prefixes; a segment's last k rows form
    a valid segment on their own)."""
    import torch

    from agent_kv_cache_amd import harness as Hn
    from agent_kv_cache_amd.workloads import randn_bf16

    sh = rs.shape
    nv = len(rs.versions)
    G = sh.n_q_heads // sh.n_kv_heads
    n = rs.n_tokens
    ks, vs = [], []
    for c in range((n + Hn.CHUNK - 1) // Hn.CHUNK):
        m = min(Hn.CHUNK, n - c * Hn.CHUNK)
        ks.append(_u16(Hn.seq_chunk(sh, rs.data_seed, 0, c, m, "k", "cuda")[0, :, 0]))
        vs.append(_u16(Hn.seq_chunk(sh, rs.data_seed, 0, c, m, "v", "cuda")[0, :, 0]))
    k, v = np.concatenate(ks), np.concatenate(vs)
    torch.cuda.empty_cache()
    cnt = restore_counts(rs)
    tasks, flops = [], 0
    for j, (mask, rows) in enumerate(rs.versions):
        kk = min(rows_per_segment, rows)
        q = randn_bf16((kk, 1, G, sh.head_dim), 300 + j).double().numpy()
        tasks.append(dict(D=sh.head_dim, base=sh.rope_base, k=k, v=v, mask=mask, q=q))
        ln = cnt[j]["len"]
        flops += 4 * sum(ln - kk + i + 1 for i in range(kk)) * sh.head_dim * G
    res, wall, nw = _pool_map(_cpu_restore_unit, tasks)
    (t_fork, t_seg), t_all, used = _critical_path(res)
    fork_b = sum(c["fork_bytes"] for c in cnt) / (sh.n_layers * sh.n_kv_heads)
    return {
        "value": round(flops / t_seg / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": used,
        "kind": "oracle",
        "sample": f"layer 0 of {sh.n_layers}, kv head 0 of {sh.n_kv_heads} and its {G} "
                  f"query heads; per segment (one per process of a {nw}-process pool) the fork "
                  f"of its version and the segment attention of its last {rows_per_segment} rows: "
                  f"{t_seg:.2f} s of segment attention on the busiest worker, {t_fork:.2f} s of "
                  f"forks; bytes and flops scaled to the sample",
        "fork_gbps": round(fork_b / t_fork / 1e9, 4),
        **host_info(),
    }


def run_restore(args):
    """Restore of the Llama-8B-shaped request after eviction: one step = reset the cache
    metadata, make the 7 position versions with akv_fork (drop + canonical
    reposition, source untouched), then one segment-batch attention launch
    over all 32 layers for the 7 segments (32768 query rows)."""
    import torch

    from agent_kv_cache_amd import harness as Hn
    from agent_kv_cache_amd import workloads as W

    rs = W.restore_llama8b_32k()
    sh = rs.shape
    nv = len(rs.versions)
    cnt = restore_counts(rs)
    lens = [rs.n_tokens] + [0] * nv
    extra = sum(Hn.pages_for(c["len"]) for c in cnt) + 8
    cache = Hn.make_cache(sh, lens, extra, max_blocks_per_seq=Hn.pages_for(rs.n_tokens))
    cache.reset()
    Hn.fill(cache, sh, lens, rs.data_seed, gen_device="cuda")
    dev = cache.device
    masks = [Hn.mask_tensor(cache, [m]) for m, _ in rs.versions]
    rows = [c["rows"] for c in cnt]
    nq = sum(rows)
    seg_seq = torch.arange(1, 1 + nv, dtype=torch.int32, device=dev)
    seg_off = torch.tensor(np.concatenate([[0], np.cumsum(rows)]).astype(np.int32), device=dev)
    max_q = max(rows)
    q = W.randn_bf16((nq, sh.n_layers, sh.n_q_heads, sh.head_dim), 203, device="cuda")
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    if cache.sync_status() != 0:
        raise RuntimeError("set-up failed on the device")
    snap = cache.meta.clone()

    def step():
        cache.meta.copy_(snap)
        for j in range(nv):
            dst = [-1] * (1 + nv)
            dst[0] = 1 + j
            cache.fork(dst, masks[j], reposition=True)
        cache.segment_attention(q, seg_seq, seg_off, max_q, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if cache.sync_status() != 0:
        raise RuntimeError("device reported an error during warm-up")
    cache.profile_read("plan", reset=True)
    cache.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    cache.profile_enable(False)
    if cache.sync_status() != 0:
        raise RuntimeError("device status after the timed steps")
    kt = {k: cache.profile_read(k) for k in ("plan", "move", "commit", "segment")}

    def tot(k):
        return kt[k][0] / args.steps

    flops = sum(c["flops"] for c in cnt)
    fork_b = sum(c["fork_bytes"] for c in cnt)
    ms_step = (t1 - t0) * 1e3 / args.steps
    seg_ms = tot("segment")
    fork_ms = tot("plan") + tot("move") + tot("commit")
    move_b = sum(c["copied"] * 2 * (sh.n_layers * sh.n_kv_heads * sh.head_dim * 2) * 2
                 for c in cnt)
    seg_tf = flops / (seg_ms * 1e-3) / 1e12
    peak_tf = 2500.0
    traffic = counted_traffic("segment_fa_kernel_restore_llama8b_32k_counters.json")
    res = {
        "metric": "restore: segment-batch attention TFLOP/s (bf16 MFMA) and fork GB/s, 1 GPU",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": f"{rs.name}: {rs.description}",
            "layers": sh.n_layers, "kv_heads": sh.n_kv_heads, "head_dim": sh.head_dim,
            "q_heads": sh.n_q_heads, "rope_base": sh.rope_base, "page_tokens": 16,
            "tokens": rs.n_tokens, "segments": nv, "query_rows": nq,
            "version_lens": [c["len"] for c in cnt], "segment_rows": rows,
            "version_shared_entries": [c["shared"] for c in cnt],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma", "kernel": "segment_fa_kernel",
            "achieved": round(seg_tf, 1), "peak": peak_tf, "unit": "TFLOP/s",
            "frac": round(seg_tf / peak_tf, 4), "traffic": traffic,
        },
        "parts": {
            "segment_attention": {"flops": flops, "ms": round(seg_ms, 4),
                                  "tflops": round(seg_tf, 1),
                                  "unique_kv_bytes": sum(c["kv_bytes"] for c in cnt)},
            "fork": {"algorithmic_bytes": fork_b, "ms": round(fork_ms, 4),
                     "gbps": round(fork_b / (fork_ms * 1e-3) / 1e9, 1),
                     "frac_of_peak": round(fork_b / (fork_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "kernel_ms": {k: round(tot(k), 4) for k in ("plan", "move", "commit")},
                     "move_kernel_gbps": round(move_b / (tot("move") * 1e-3) / 1e9, 1),
                     "launches_per_step": nv},
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = restore_cpu_baseline(rs, args.cpu_rows)
    return res


def run_append(args):
    """Append of the Llama-8B-shaped request's 32768 tokens in one call (a prefill's KV
    write), plain (keys already rotated) and with the RoPE step fused in
    (akv_append_rope).  One step = reset the cache metadata + one append.
    Algorithmic bytes: K and V of every new token read once and written once,
    plus its position and token id."""
    import torch

    from agent_kv_cache_amd import harness as Hn
    from agent_kv_cache_amd import workloads as W

    wl = W.llama8b_32k()
    sh = wl.shape
    n = wl.seq_lens[0]
    ropt = rope_options(args, sh)
    cache = Hn.make_cache(sh, [n], 8, **ropt)
    cache.reset()
    dev = cache.device
    k = W.randn_bf16((sh.n_layers, n, sh.n_kv_heads, sh.head_dim), 205, device="cuda")
    v = W.randn_bf16((sh.n_layers, n, sh.n_kv_heads, sh.head_dim), 206, device="cuda")
    tid = torch.arange(n, dtype=torch.int32, device=dev)
    counts = torch.tensor([n], dtype=torch.int32, device=dev)
    snap = cache.meta.clone()
    row = sh.n_layers * sh.n_kv_heads * sh.head_dim * 2
    alg = n * 2 * row * 2 + n * 12
    res = {}
    for name, fn in (("append", cache.append), ("append_rope", cache.append_rope)):
        def step():
            cache.meta.copy_(snap)
            fn(counts, n, k, v, tid)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        if cache.sync_status() != 0:
            raise RuntimeError("device status during warm-up")
        cache.profile_read("append", reset=True)
        cache.profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        cache.profile_enable(False)
        if cache.sync_status() != 0:
            raise RuntimeError("device status after the timed steps")
        ms, cnt = cache.profile_read("append")
        kms = ms / max(cnt, 1)
        res[name] = {"ms": round(kms, 4), "gbps": round(alg / (kms * 1e-3) / 1e9, 1),
                     "frac_of_peak": round(alg / (kms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "ms_per_step_wall": round((t1 - t0) * 1e3 / args.steps, 4),
                     # HBM bytes per launch from the committed counter record of
                     # this kernel and variant (None once its sources changed)
                     "traffic": counted_traffic(
                         f"{name}_kernel_append_llama8b_32k{variant_tag(args)}_counters.json")}
    fr = res["append_rope"]
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on every layer of the same append, one layer per task
        layers = list(range(sh.n_layers))
        tasks = [dict(H=sh.n_kv_heads, D=sh.head_dim, base=sh.rope_base,
                      k=_u16(k[l]), v=_u16(v[l]), rotary_dim=ropt.get("rotary_dim"),
                      theta=ropt.get("inv_freq")) for l in layers]
        del cache
        torch.cuda.empty_cache()
        out, wall, nw = _pool_map(_cpu_append_unit, tasks)
        (t_plain, t_rope), t_all, used = _critical_path(out)
        ab = n * 2 * (len(layers) * sh.n_kv_heads * sh.head_dim * 2) * 2 + n * 12
        cpu = {"value": round(ab / t_rope / 1e9, 4), "unit": "GB/s", "cores": used,
               "kind": "oracle",
               "sample": f"append of {n} tokens: layers {layers} of {sh.n_layers}, one layer per task "
                         f"of a {nw}-process pool, the plain append and the RoPE-fused "
                         f"append per layer: {t_all:.2f} s on the busiest worker ({wall:.1f} s "
                         f"pool wall time including unpacking the inputs); bytes are the "
                         f"sample's share of the algorithmic bytes; value is the RoPE-fused "
                         f"append",
               "append_plain_gbps": round(ab / t_plain / 1e9, 4),
               **host_info()}
    return {
        "metric": "append GB/s (K/V write of new tokens, plain and RoPE-fused), 1 GPU",
        "value": fr["gbps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": fr["ms_per_step_wall"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "append of 32768 tokens to one sequence, Llama-8B shape "
                               "(32 layers, 8 kv heads, d 128)",
                   "tokens": n, "algorithmic_bytes": alg,
                   **({"rotary_dim": args.rotary_dim} if args.rotary_dim else {})},
        "roofline": {"bound": "hbm", "kernel": "append_copy_kernel (RoPE fused)",
                     "achieved": fr["gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": fr["frac_of_peak"], "traffic": fr["traffic"]},
        "parts": res,
        **({"cpu_baseline": cpu} if cpu else {}),
    }


def calibrate(nbytes: int, reps: int):
    """Achieved GB/s of torch's device copy (read+write), fill (write) and a
    max-reduction (read) over `nbytes`: the plain streaming kernels that bound
    what a copy-shaped or read-shaped kernel can reach on this GPU."""
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    out = {}
    for name, fn, moved in (("copy", lambda: b.copy_(a), 2 * n * 4),
                            ("fill", lambda: b.fill_(7), n * 4),
                            ("read_max", lambda: torch.amax(a), n * 4)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(reps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / reps
        out[name] = {"bytes": moved, "ms": round(ms, 4), "gbps": round(moved / ms / 1e6, 1),
                     "frac_of_peak": round(moved / ms / 1e6 / PEAK_HBM_GBPS, 4)}
    return {"calibration": out, "buffer_bytes": nbytes}


# Oracle sample per workload: (layers, sequences or None = all), about
# 5-25 s of single-core oracle work on an EPYC host, spread over the pool.
CPU_SAMPLE = {
    "one_layer_4k": ([0], None),
    "llama8b_32k": (list(range(32)), None),
    "ragged_batch_64": ([0, 31], None),
    "llama70b_4x64k": ([0, 20, 40, 60], None),
}


def run_step(name, args):
    """One drop+reposition + decode workload: set up, time the steps, and
    return its JSON line (GPU memory released before returning)."""
    import torch

    from agent_kv_cache_amd import harness as Hn
    from agent_kv_cache_amd import workloads as W

    wl = W.WORKLOADS[name]()
    sh = wl.shape
    extra = sum(Hn.moved_pages(n, m) for n, m in zip(wl.seq_lens, wl.masks)) + 8
    ropt = rope_options(args, sh)
    cache = Hn.make_cache(sh, wl.seq_lens, extra, **ropt)
    cache.reset(None if wl.block_order is None else
                np.concatenate([wl.block_order, np.arange(len(wl.block_order), cache.NB,
                                                          dtype=np.int32)]))
    Hn.fill(cache, sh, wl.seq_lens, wl.data_seed, gen_device="cuda")
    mask = Hn.mask_tensor(cache, wl.masks)
    q = W.randn_bf16((wl.n_seqs, sh.n_layers, sh.n_q_heads, sh.head_dim), 202, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(sh.n_layers, sh.n_q_heads)),
                     dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    if cache.sync_status() != 0:
        raise RuntimeError("set-up failed on the device")
    snap = cache.meta.clone()
    stream = torch.cuda.current_stream()

    def step():
        cache.meta.copy_(snap)
        cache.drop_reposition(mask)
        cache.decode_attention(q, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if cache.sync_status() != 0:
        raise RuntimeError("device reported an error during warm-up")
    cache.profile_read("plan", reset=True)
    cache.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    cache.profile_enable(False)
    st = cache.sync_status()
    if st != 0:
        raise RuntimeError(f"device status {st}")
    kt = {k: cache.profile_read(k) for k in ("plan", "move", "commit", "rounds", "attn",
                                              "combine")}

    ab = algorithmic_bytes(sh, wl.seq_lens, wl.masks, ropt.get("layer_window"))
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = (ab["b_dr"] + ab["b_att"]) / (ms_step * 1e-3) / 1e9

    def avg(k):
        """Event-timed milliseconds of kernel k per step (the move: the
        op's first-round launches, one-shot and persistent; rounds: the
        later (move, commit) rounds a pool that may run short enqueues)."""
        return kt[k][0] / args.steps

    dr_ms = avg("plan") + avg("move") + avg("commit") + avg("rounds")
    att_ms = avg("attn") + avg("combine")
    move_gbps = ab["b_move"] / (avg("move") * 1e-3) / 1e9
    attn_gbps = (ab["b_att"]) / (avg("attn") * 1e-3) / 1e9
    dom = "move" if avg("move") >= avg("attn") else "attn"
    dom_gbps = move_gbps if dom == "move" else attn_gbps
    # HBM bytes per launch from the committed rocprofv3 counter record of this
    # kernel and workload (FETCH_SIZE and WRITE_SIZE scaled by what they read
    # for a plain copy of known size), used only while the kernel source is
    # unchanged since the counters were taken.
    traffic = counted_traffic(f"{dom}_kernel_{wl.name}{variant_tag(args)}_counters.json")

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.description}",
            "layers": sh.n_layers, "kv_heads": sh.n_kv_heads, "head_dim": sh.head_dim,
            "q_heads": sh.n_q_heads, "rope_base": sh.rope_base, "page_tokens": 16,
            "sequences": wl.n_seqs, "tokens": ab["tokens"], "survivors": ab["survivors"],
            "moved_tokens": ab["moved"], "parallelism": "single GPU",
            **({"rotary_dim": args.rotary_dim} if args.rotary_dim else {}),
            **({"rope_freq": args.freq} if args.freq != "base" else {}),
            **({"layer_window": ropt["layer_window"]} if args.window else {}),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "move_kernel" if dom == "move" else "attn_kernel",
            "achieved": round(dom_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(dom_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
        },
        "parts": {
            "drop_reposition": {
                "algorithmic_bytes": ab["b_dr"], "ms": round(dr_ms, 4),
                "gbps": round(ab["b_dr"] / (dr_ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(ab["b_dr"] / (dr_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                "kernel_ms": {k: round(avg(k), 4) for k in ("plan", "move", "commit", "rounds")},
                "move_kernel_gbps": round(move_gbps, 1),
            },
            "decode_attention": {
                "algorithmic_bytes": ab["b_att"], "ms": round(att_ms, 4),
                "gbps": round(ab["b_att"] / (att_ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(ab["b_att"] / (att_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                "kernel_ms": {k: round(avg(k), 4) for k in ("attn", "combine")},
                "attn_kernel_gbps": round(attn_gbps, 1),
            },
        },
    }
    # Per-step spread of the two kernels: the same steps once more, each
    # step's event times read back on their own (outside the timed region).
    # (a reset clears every kernel's accumulator: read both, then reset)
    spread = {"move": [], "attn": []}
    cache.profile_read("move", reset=True)
    cache.profile_enable(True)
    for _ in range(args.steps):
        step()
        for k in spread:
            spread[k].append(cache.profile_read(k)[0])
        cache.profile_read("move", reset=True)
    cache.profile_enable(False)
    if cache.sync_status() != 0:
        raise RuntimeError("device status after the spread pass")
    for part, k in (("drop_reposition", "move"), ("decode_attention", "attn")):
        v = np.sort(np.array(spread[k]))
        res["parts"][part][f"{k}_ms_per_step"] = {
            "median": round(float(np.median(v)), 4), "min": round(float(v[0]), 4),
            "max": round(float(v[-1]), 4), "steps": len(v)}
    if wl.n_seqs == 1 and sh.n_layers > 1:
        # Secondary: the same decode as one launch per layer (as a model's
        # forward issues it), timed over the state the steps left; its
        # outputs are compared with the one-launch outputs of the last step.
        L = sh.n_layers
        wsl = torch.empty(max(256, cache.decode_workspace_bytes(1, sh.n_q_heads)),
                          dtype=torch.uint8, device="cuda")
        ql = [q[:, l:l + 1].contiguous() for l in range(L)]
        ol = [torch.empty_like(x) for x in ql]

        def per_layer():
            for l in range(L):
                cache.decode_attention(ql[l], ol[l], wsl, layer_begin=l, n_layers=1)
        for _ in range(args.warmup):
            per_layer()
        torch.cuda.synchronize()
        cache.profile_read("attn", reset=True)
        cache.profile_enable(True)
        for _ in range(args.steps):
            per_layer()
        cache.profile_enable(False)
        if cache.sync_status() != 0:
            raise RuntimeError("device status after the per-layer decode")
        pl_ms = (cache.profile_read("attn")[0] + cache.profile_read("combine")[0]) / args.steps
        diff = max(float((ol[l].float() - out[:, l:l + 1].float()).abs().max()) for l in range(L))
        res["parts"]["decode_attention"]["per_layer_launches"] = {
            "launches": L, "ms": round(pl_ms, 4),
            "gbps": round(ab["b_att"] / (pl_ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(ab["b_att"] / (pl_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "max_abs_diff_vs_one_launch": diff}
        del wsl, ql, ol
    if args.graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        tg1 = time.perf_counter()
        if cache.sync_status() != 0:
            raise RuntimeError("device status after graph replays")
        gms = (tg1 - tg0) * 1e3 / args.steps
        res["graph_ms_per_step"] = round(gms, 4)
        res["graph_value"] = round((ab["b_dr"] + ab["b_att"]) / (gms * 1e-3) / 1e9, 2)
    if not args.no_cpu_baseline:
        layers, seqs = CPU_SAMPLE[wl.name]
        res["cpu_baseline"] = cpu_baseline(wl, layers, seqs, ropt)
    del cache, q, out, ws, mask, snap
    torch.cuda.empty_cache()
    return res


def compact(line):
    """The fields of a workload line kept under the default run's `configs`."""
    keep = ("value", "unit", "ms_per_step", "steps", "warmup", "roofline", "parts",
            "cpu_baseline", "ops", "ops_ms_total", "ops_bytes_total", "drop_reposition_gbps",
            "drop_reposition_frac_of_peak", "decode_ms", "decode_gbps", "decode_frac_of_peak",
            "final_active", "graph_ms_per_step", "graph_value")
    out = {k: line[k] for k in keep if k in line}
    out["workload"] = line.get("config", {}).get("workload", line.get("workload"))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all",
                    choices=["all", "one_layer_4k", "llama8b_32k", "ragged_batch_64",
                             "history_50_turns", "llama70b_4x64k", "restore", "append"],
                    help="all (default): the ragged batch as the headline, the other "
                         "configurations under `configs`")
    ap.add_argument("--cpu-rows", type=int, default=256,
                    help="restore: rows per segment in the oracle sample")
    ap.add_argument("--rotary-dim", type=int, default=0,
                    help="partial RoPE: rotate only the first R dims of each head")
    ap.add_argument("--freq", default="base", choices=["base", "llama3", "yarn"],
                    help="RoPE frequency schedule (Llama 3.1 or YaRN tables)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding-window length for decode in all but every "
                         "--window-every-th layer")
    ap.add_argument("--window-every", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed "
                         "(reported as graph_ms_per_step; per-kernel times stay eager)")
    ap.add_argument("--calibrate", type=int, default=0, metavar="BYTES",
                    help="instead of the workload, time plain device copy / fill / read "
                         "kernels over BYTES (the reference kernels whose counter readings "
                         "scale the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the hot path shards by kv head / layer with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from agent_kv_cache_amd.binding import lib

    torch.cuda.set_device(0)
    if args.calibrate:
        print(json.dumps(calibrate(args.calibrate, args.steps)), flush=True)
        return
    lib()
    if args.workload == "history_50_turns":
        print(json.dumps(run_history(args)), flush=True)
        return
    if args.workload == "restore":
        print(json.dumps(run_restore(args)), flush=True)
        return
    if args.workload == "append":
        print(json.dumps(run_append(args)), flush=True)
        return
    if args.workload != "all":
        print(json.dumps(run_step(args.workload, args)), flush=True)
        return
    # default: every configuration, the largest single-GPU one as the headline
    t0 = time.time()
    res = run_step("ragged_batch_64", args)
    print(f"[bench] ragged_batch_64 done ({time.time() - t0:.0f} s)", file=sys.stderr, flush=True)
    res["configs"] = {}
    for name in ("llama8b_32k", "one_layer_4k", "llama70b_4x64k"):
        # the latency-bound one-layer step is also timed as one HIP graph replay
        a = argparse.Namespace(**{**vars(args), "graph": args.graph or name == "one_layer_4k"})
        res["configs"][name] = compact(run_step(name, a))
        print(f"[bench] {name} done ({time.time() - t0:.0f} s)", file=sys.stderr, flush=True)
    res["configs"]["history_50_turns"] = compact(run_history(args))
    print(f"[bench] history_50_turns done ({time.time() - t0:.0f} s)", file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
