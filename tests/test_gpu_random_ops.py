"""Seeded random operation sequences against the oracle on a tight page pool.

Six sequences, appends, drops, repositions (canonical and explicit), fused
drop + reposition, forks (with and without a drop / reposition: pages shared
with the source) and releases, in random order, on a pool too small for some
ops: those run in sequence groups or, when a sequence cannot fit, are
rejected.  After every op: an op whose worst-case page need fits the free
pool must succeed, an append exactly when its new pages fit; a successful op
matches the oracle applied to the same op (ids, positions, lengths, next positions bit for bit; K within one
bf16 step, V bit for bit, every few ops and at the end); a rejected op must
be plausible (the free pool smaller than the op's worst-case need) and leave
the cache unchanged; and the pool is accounted for exactly (every page free
once or held by 1 + its extra references).  Ends with a decode checked
against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from agent_kv_cache_amd import harness as Hn  # noqa: E402
from agent_kv_cache_amd import workloads as W  # noqa: E402

from gpu_util import (check_attention, check_kv, check_meta, check_pool, q_tensor,  # noqa: E402
                      say, to_f64)
from oracle import akv_oracle as O  # noqa: E402

SH = W.Shape(2, 2, 64, 4, 1.0e4)
B, MAXPG = 6, 40


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from agent_kv_cache_amd.binding import lib
    lib()


def _pages(n):
    return (int(n) + 15) // 16


def _rand_mask(rng, n):
    m = np.zeros(n, np.uint8)
    for _ in range(int(rng.integers(0, 3))):
        if n:
            s = int(rng.integers(0, n))
            m[s:s + int(rng.integers(1, max(2, n // 3)))] = 1
    return m


def _state(cache):
    return (cache.meta.clone(), cache.positions.clone(), cache.token_ids.clone())


def _unchanged(cache, st):
    assert torch.equal(cache.meta, st[0])
    assert torch.equal(cache.positions, st[1]) and torch.equal(cache.token_ids, st[2])


@pytest.mark.parametrize("seed,pool", [(11, 150), (12, 150), (13, 72), (14, 56), (15, 44)])
def test_random_op_sequences(seed, pool):
    rng = np.random.default_rng(seed)
    cache = Hn.make_cache(SH, [0] * B, pool, max_blocks_per_seq=MAXPG)
    cache.reset(rng.permutation(cache.NB).astype(np.int32))
    oc = O.OracleCache(SH.n_layers, SH.n_kv_heads, SH.head_dim, SH.rope_base, n_seqs=B)
    dev = cache.device
    tid_next = 1
    counts = {"ok": 0, "rejected": 0}
    n_rot = 0        # applied ops that may re-rotate keys (end-to-end bound, R12 reading)
    for step in range(60):
        lens = [len(s) for s in oc.seqs]
        kind = rng.choice(["append", "append", "drop", "repos", "drop_repos", "fork", "fork",
                           "release"])
        fc = int(cache.free_count.item())
        st = _state(cache)
        need = None          # worst-case fresh pages of the op (None: never rejected)
        if kind == "append":
            cnt = [int(rng.integers(0, 140)) if rng.random() < 0.6 else 0 for _ in range(B)]
            cnt = [min(c, MAXPG * 16 - n) for c, n in zip(cnt, lens)]
            N = sum(cnt)
            if N == 0:
                continue
            k = W.randn_bf16((SH.n_layers, N, SH.n_kv_heads, SH.head_dim), 9000 + 2 * step)
            v = W.randn_bf16((SH.n_layers, N, SH.n_kv_heads, SH.head_dim), 9001 + 2 * step)
            tid = np.arange(tid_next, tid_next + N)
            tid_next += N
            cache.append(torch.tensor(cnt, dtype=torch.int32, device=dev), N, k.to(dev),
                         v.to(dev), torch.tensor(tid, dtype=torch.int32, device=dev))
            need = sum(_pages(n + c) - _pages(n) for n, c in zip(lens, cnt))

            def apply():
                o = 0
                for b in range(B):
                    if cnt[b]:
                        sl = slice(o, o + cnt[b])
                        oc.append(b, tid[sl], to_f64(k[:, sl].permute(1, 0, 2, 3)),
                                  to_f64(v[:, sl].permute(1, 0, 2, 3)))
                    o += cnt[b]
        elif kind in ("drop", "drop_repos"):
            masks = [_rand_mask(rng, n) for n in lens]
            mt = Hn.mask_tensor(cache, masks)
            (cache.drop if kind == "drop" else cache.drop_reposition)(mt)
            need = sum(_pages(n) for n in lens)

            def apply():
                for b in range(B):
                    if kind == "drop":
                        oc.drop(b, masks[b])
                    else:
                        oc.drop_reposition(b, masks[b])
        elif kind == "repos":
            explicit = rng.random() < 0.5
            rows = []
            for n in lens:
                gaps = rng.integers(1, 4, size=n) if explicit else np.ones(n, np.int64)
                rows.append((np.cumsum(gaps) - 1 + int(rng.integers(0, 5))) if explicit
                            else np.arange(n))
            cache.reposition(None, Hn.pos_tensor(cache, rows) if explicit else None)
            need = sum(_pages(n) for n in lens)      # copy on write of shared pages

            def apply():
                for b in range(B):
                    oc.reposition(b, rows[b] if explicit else None)
        elif kind == "fork":
            srcs = [b for b in range(B) if lens[b]]
            dsts = [b for b in range(B) if not lens[b]]
            if not srcs or not dsts:
                continue
            src, dst = int(rng.choice(srcs)), int(rng.choice(dsts))
            m = _rand_mask(rng, lens[src]) if rng.random() < 0.6 else None
            rep = bool(rng.random() < 0.5)
            dst_of = [-1] * B
            dst_of[src] = dst
            rows = [None] * B
            rows[src] = m
            cache.fork(dst_of, Hn.mask_tensor(cache, rows) if m is not None else None,
                       reposition=rep)
            need = _pages(lens[src])

            def apply():
                oc.fork(src, dst, m, reposition=rep)
        else:
            sel = (rng.random(B) < 0.3).astype(np.uint8)
            if not sel.any():
                continue
            cache.release(torch.tensor(sel, device=dev))

            def apply():
                for b in np.flatnonzero(sel):
                    oc.release(int(b))
        status = cache.sync_status()
        if need is not None and fc >= need:
            # the worst case fits the free pool: the op may not be refused
            assert status == 0, (step, kind, status, fc, need)
        if kind == "append":
            # an append's need is exact (a version's partial last page is its own)
            assert (status != 0) == (fc < need), (step, fc, need, status)
        if status == 0:
            apply()
            counts["ok"] += 1
            n_rot += kind in ("repos", "drop_repos", "fork")
        else:
            # a rejection must be plausible and leave everything as it was
            assert status in (4, 5), (step, kind, status)
            assert need is not None and fc < need, (step, kind, fc, need)
            _unchanged(cache, st)
            counts["rejected"] += 1
        check_meta(cache, oc)
        check_pool(cache)
        if step % 6 == 5:
            check_kv(cache, oc, k_ulp=max(1, n_rot))
    worst = check_kv(cache, oc, k_ulp=max(1, n_rot))
    q = q_tensor(SH, B, SH.n_layers, 99 + seed, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(SH.n_layers, SH.n_q_heads)),
                     dtype=torch.uint8, device=dev)
    cache.decode_attention(q, out, ws)
    assert cache.sync_status() == 0
    check_attention(cache, oc, q, out, what=f"random ops seed {seed} decode")
    say(f"random ops seed {seed}: {counts['ok']} ops applied, {counts['rejected']} rejected, "
        f"{cache.NB} pages; K within {worst} step(s) of the oracle's chain")
