"""A cache of 600 short sequences (some empty) against the oracle: more
sequences than one pass of the plan's per-sequence finalize (256), a deep
sequence search in the move, forks of many sources in one call, an append, a
release of a scattered set and a batched decode.  After every op the ids,
positions, lengths and next positions match the oracle bit for bit, K is
within one bf16 step and V bit-exact, and the pool is accounted for exactly."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from agent_kv_cache_amd import harness as Hn  # noqa: E402
from agent_kv_cache_amd import workloads as W  # noqa: E402

from gpu_util import (append_seeded, check_attention, check_kv, check_meta, check_pool,  # noqa: E402
                      oracle_for, q_tensor, say)

SH = W.Shape(2, 2, 64, 4, 1.0e4)
B, MAXPG = 600, 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from agent_kv_cache_amd.binding import lib
    lib()


def _masks(rng, oc, p):
    return [(rng.random(len(s)) < p).astype(np.uint8) for s in oc.seqs]


def _check(cache, oc, what):
    check_meta(cache, oc)
    check_pool(cache)
    worst = check_kv(cache, oc, k_ulp=1)
    say(f"{what}: state matches the oracle (K within {worst} step)")


def test_many_short_sequences():
    rng = np.random.default_rng(91)
    lens = [int(n) if rng.random() < 0.85 else 0 for n in rng.integers(1, 200, size=B)]
    cache = Hn.make_cache(SH, lens, 2500, max_blocks_per_seq=MAXPG)
    cache.reset(rng.permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, SH, lens, 92, gen_device="cpu")
    assert cache.sync_status() == 0
    oc = oracle_for(SH, lens, 92)
    say(f"case {B} sequences, {sum(lens)} tokens, {cache.NB} pages")

    m = _masks(rng, oc, 0.2)
    cache.drop(Hn.mask_tensor(cache, m))
    assert cache.sync_status() == 0
    for b in range(B):
        oc.drop(b, m[b])
    _check(cache, oc, "drop")

    m = _masks(rng, oc, 0.1)
    cache.drop_reposition(Hn.mask_tensor(cache, m))
    assert cache.sync_status() == 0
    for b in range(B):
        oc.drop_reposition(b, m[b])
    _check(cache, oc, "drop + reposition")

    # forks of 40 sources into 40 empty sequences in one call, each with a
    # drop and a canonical reposition (unchanged leading pages shared)
    srcs = [b for b in range(B) if len(oc.seqs[b]) > 20][:40]
    dsts = [b for b in range(B) if len(oc.seqs[b]) == 0][:40]
    assert len(srcs) == len(dsts) == 40
    dst_of = [-1] * B
    rows = [None] * B
    for s_, d_ in zip(srcs, dsts):
        dst_of[s_] = d_
        rows[s_] = (rng.random(len(oc.seqs[s_])) < 0.15).astype(np.uint8)
    cache.fork(dst_of, Hn.mask_tensor(cache, rows), reposition=True)
    assert cache.sync_status() == 0
    for s_, d_ in zip(srcs, dsts):
        oc.fork(s_, d_, rows[s_], reposition=True)
    _check(cache, oc, "forks")

    per_seq = [int(min(rng.integers(0, 40), MAXPG * 16 - len(s))) for s in oc.seqs]
    append_seeded(cache, oc, SH, per_seq, 93, 1 << 22)
    assert cache.sync_status() == 0
    _check(cache, oc, "append")

    sel = (rng.random(B) < 0.3).astype(np.uint8)
    cache.release(torch.tensor(sel, device=cache.device))
    assert cache.sync_status() == 0
    for b in np.flatnonzero(sel):
        oc.release(int(b))
    _check(cache, oc, "release")

    m = _masks(rng, oc, 0.25)
    cache.drop_reposition(Hn.mask_tensor(cache, m))
    assert cache.sync_status() == 0
    for b in range(B):
        oc.drop_reposition(b, m[b])
    _check(cache, oc, "drop + reposition after the release")

    q = q_tensor(SH, B, SH.n_layers, 94, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(SH.n_layers, SH.n_q_heads)),
                     dtype=torch.uint8, device=cache.device)
    cache.decode_attention(q, out, ws)
    assert cache.sync_status() == 0
    check_attention(cache, oc, q, out, what=f"decode over {B} sequences")


def test_decode_with_more_sequence_layer_rows_than_one_grid_axis_holds():
    """2100 sequences x 32 layers = 67200 (sequence, layer) rows, more than
    the 65535 one axis of a launch grid holds: the decode's one-dimensional
    grid covers them.  A fused drop + reposition first; ids and positions of
    every sequence, K/V and attention of 70 sampled sequences on 3 layers
    against the oracle."""
    sh = W.Shape(32, 1, 64, 2, 1.0e4)
    n_seq = 2100
    rng = np.random.default_rng(95)
    lens = [int(n) for n in rng.integers(1, 48, size=n_seq)]
    assert n_seq * sh.n_layers > 65535
    cache = Hn.make_cache(sh, lens, 4500, max_blocks_per_seq=4)
    cache.reset()
    Hn.fill(cache, sh, lens, 96, gen_device="cpu")
    assert cache.sync_status() == 0
    say(f"case {n_seq} sequences x {sh.n_layers} layers, {sum(lens)} tokens")
    masks = [(rng.random(n) < 0.3).astype(np.uint8) for n in lens]
    cache.drop_reposition(Hn.mask_tensor(cache, masks))
    assert cache.sync_status() == 0
    meta = oracle_for(sh, lens, 96, with_kv=False)
    for b in range(n_seq):
        meta.drop_reposition(b, masks[b])
    check_meta(cache, meta)
    seqs = sorted(rng.choice(n_seq, size=70, replace=False).tolist())
    lay = [0, 17, 31]
    oc = oracle_for(sh, lens, 96, layers=lay, seqs=seqs)
    for i, b in enumerate(seqs):
        oc.drop_reposition(i, masks[b])
    check_kv(cache, oc, k_ulp=1, seqs=seqs, layers=lay)
    q = q_tensor(sh, n_seq, sh.n_layers, 97, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(sh.n_layers, sh.n_q_heads)),
                     dtype=torch.uint8, device=cache.device)
    cache.decode_attention(q, out, ws)
    assert cache.sync_status() == 0
    check_attention(cache, oc, q, out, layers=lay, seqs=seqs,
                    what=f"decode over {n_seq * sh.n_layers} (sequence, layer) rows")
