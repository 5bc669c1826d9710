"""Position versions that share pages with their source (akv_fork): the
version holds the source's leading full pages whose entries it leaves as they
are (one more reference each) and copies the rest.  Against the oracle, whose
versions are plain copies: the observable state must be the same.  After every
step the pool is accounted for exactly: a page is either free (once, with no
holder) or held, and its reference count equals the number of page-table
entries pointing at it."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from agent_kv_cache_amd import harness as Hn  # noqa: E402
from agent_kv_cache_amd import workloads as W  # noqa: E402

from gpu_util import (append_seeded, check_attention, check_kv, check_meta,  # noqa: E402
                      check_pool, oracle_for, q_tensor, say, snapshot, same_state)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from agent_kv_cache_amd.binding import lib
    lib()


SH = W.Shape(2, 2, 64, 4, 1.0e4)


def _setup(lens, seed, extra=300, maxpg=80):
    cache = Hn.make_cache(SH, lens, extra, max_blocks_per_seq=maxpg)
    cache.reset(np.random.default_rng(seed).permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, SH, lens, seed, gen_device="cpu")
    assert cache.sync_status() == 0
    return cache, oracle_for(SH, lens, seed)


def _fork(cache, oc, src, dst, mask=None, repos=False):
    dst_of = [-1] * cache.B
    dst_of[src] = dst
    mm = None
    if mask is not None:
        rows = [None] * cache.B
        rows[src] = mask
        mm = Hn.mask_tensor(cache, rows)
    before = snapshot(cache, src)
    cache.fork(dst_of, mm, reposition=repos)
    assert cache.sync_status() == 0
    oc.fork(src, dst, mask, reposition=repos)
    same_state(before, snapshot(cache, src))


def _release(cache, oc, seqs):
    sel = np.zeros(cache.B, np.uint8)
    sel[list(seqs)] = 1
    cache.release(torch.tensor(sel, device=cache.device))
    assert cache.sync_status() == 0
    for b in seqs:
        oc.release(b)


def test_fork_shares_the_unchanged_prefix_and_survives_its_source():
    lens = [1000, 0, 0, 0]
    cache, oc = _setup(lens, 71)
    say("case fork: drop a span at 300, canonical positions -> 18 pages shared")
    m = W.spans_to_mask(1000, [(300, 100)])
    _fork(cache, oc, 0, 1, m, repos=True)
    tab = cache.block_table.cpu().numpy()
    assert np.array_equal(tab[1, :18], tab[0, :18])            # 300 // 16 pages shared
    assert not np.isin(tab[1, 18:57], tab[0, :63]).any()        # the rest copied
    assert check_pool(cache) == 2
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    say("case fork of the whole sequence: every full page shared, the partial last copied")
    _fork(cache, oc, 0, 2)
    tab = cache.block_table.cpu().numpy()
    assert np.array_equal(tab[2, :62], tab[0, :62]) and tab[2, 62] != tab[0, 62]
    assert check_pool(cache) == 3
    say("case release the source; both versions keep their entries")
    _release(cache, oc, [0])
    check_pool(cache)
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    say("case append to a version (into its own partial page)")
    append_seeded(cache, oc, SH, [0, 0, 37, 0], 7100, 1 << 20)
    assert cache.sync_status() == 0
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    check_pool(cache)
    say("case release every version in one call: every page free again")
    _release(cache, oc, [1, 2])
    assert check_pool(cache) == 0
    assert int(cache.free_count.item()) == cache.NB


def test_drop_and_copy_on_write_inside_a_shared_prefix():
    lens = [900, 0, 0, 0]
    cache, oc = _setup(lens, 72)
    _fork(cache, oc, 0, 1)                        # all 56 full pages shared
    _fork(cache, oc, 1, 2, W.spans_to_mask(900, [(700, 50)]))   # fork of a fork
    assert check_pool(cache) == 3
    say("case drop inside the shared prefix of the version")
    rows = [None, W.spans_to_mask(900, [(100, 40), (500, 2)]), None, None]
    cache.drop(Hn.mask_tensor(cache, rows))
    assert cache.sync_status() == 0
    oc.drop(1, rows[1])
    check_pool(cache)
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=0)
    say("case reposition in place of pages other sequences hold (copy on write)")
    src0 = snapshot(cache, 0)
    src1 = snapshot(cache, 1)
    # only sequence 2 moves (to 2i + 5); the others keep their own positions
    pos_rows = [oc.seqs[b].pos.copy() for b in range(4)]
    pos_rows[2] = np.arange(len(oc.seqs[2])) * 2 + 5
    cache.reposition(None, Hn.pos_tensor(cache, pos_rows))
    assert cache.sync_status() == 0
    for b in range(4):
        oc.reposition(b, pos_rows[b])
    same_state(src0, snapshot(cache, 0))
    same_state(src1, snapshot(cache, 1))
    tab = cache.block_table.cpu().numpy()
    assert not np.isin(tab[2, :Hn.pages_for(len(oc.seqs[2]))], tab[0, :57]).any()
    check_pool(cache)
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    say("case drop + canonical reposition of the source while versions hold its prefix")
    rows = [W.spans_to_mask(900, [(0, 3)]), None, None, None]
    cache.drop_reposition(Hn.mask_tensor(cache, rows))
    assert cache.sync_status() == 0
    for b in range(4):
        if len(oc.seqs[b]):
            oc.drop_reposition(b, rows[b] if rows[b] is not None
                               else np.zeros(len(oc.seqs[b]), np.uint8))
    check_pool(cache)
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    _release(cache, oc, [0, 1, 2])
    assert check_pool(cache) == 0 and int(cache.free_count.item()) == cache.NB


def test_prefix_reuse_at_new_positions():
    """Reusing a compatible prefix of a stored sequence at other positions
    ([CE] Appendix A.1.2: the longer prefix whose positions can be converted
    is taken and its keys turned to the new positions): a fork that keeps the
    prefix (drops the rest) and repositions it.  Pages whose entries keep
    their positions are shared; the others are copied with K re-rotated."""
    lens = [1000, 0, 0, 0]
    cache, oc = _setup(lens, 73)
    say("case the stored sequence has a position gap (drop without reposition)")
    rows = [W.spans_to_mask(1000, [(200, 100)]), None, None, None]
    cache.drop(Hn.mask_tensor(cache, rows))
    assert cache.sync_status() == 0
    oc.drop(0, rows[0])
    n = len(oc.seqs[0])
    assert n == 900
    say("case prefix of 500 entries at canonical positions 0..499: 12 pages shared")
    keep = np.zeros(n, np.uint8)
    keep[500:] = 1
    _fork(cache, oc, 0, 1, keep, repos=True)
    tab = cache.block_table.cpu().numpy()
    assert np.array_equal(tab[1, :12], tab[0, :12])             # entries 0..191 keep 0..191
    assert not np.isin(tab[1, 12:32], tab[0, :57]).any()        # from the gap on: copied
    assert np.array_equal(oc.seqs[1].pos, np.arange(500))
    check_pool(cache)
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    say("case prefix of 320 entries moved to p + 37 (every position changes: nothing shared)")
    keep = np.zeros(n, np.uint8)
    keep[320:] = 1
    newp = (oc.seqs[0].pos[:320] + 37).astype(np.int32)
    dst_of = [2, -1, -1, -1]
    pos_rows = [newp, None, None, None]
    before = snapshot(cache, 0)
    cache.fork(dst_of, Hn.mask_tensor(cache, [keep, None, None, None]), reposition=True,
               new_pos=Hn.pos_tensor(cache, pos_rows))
    assert cache.sync_status() == 0
    oc.fork(0, 2, keep, reposition=True, new_pos=newp)
    same_state(before, snapshot(cache, 0))
    tab = cache.block_table.cpu().numpy()
    assert not np.isin(tab[2, :20], tab[0, :57]).any()
    assert np.array_equal(oc.seqs[2].pos, newp)
    check_pool(cache)
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    say("case release the source: both reused prefixes keep their entries")
    _release(cache, oc, [0])
    check_pool(cache)
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    say("case decode over the reused prefixes")
    q = q_tensor(SH, cache.B, SH.n_layers, 74, device=cache.device)
    out = torch.empty_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(SH.n_layers, SH.n_q_heads)),
                     dtype=torch.uint8, device=cache.device)
    cache.decode_attention(q, out, ws)
    assert cache.sync_status() == 0
    check_attention(cache, oc, q, out, what="decode over reused prefixes")
