"""A drop / reposition whose fresh pages do not fit the free pool at once
runs in sequence groups (each group's old pages freed before the next takes
fresh ones).  Pools that fit every sequence but not the whole op, against
the oracle; more groups than the rounds enqueued, and a sequence that does
not fit alone, are rejected with the cache unchanged."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from agent_kv_cache_amd import harness as Hn  # noqa: E402
from agent_kv_cache_amd import workloads as W  # noqa: E402

from gpu_util import bits, check_kv, check_meta, oracle_for, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from agent_kv_cache_amd.binding import lib
    lib()


SH = W.Shape(3, 2, 64, 4, 1.0e4)
LENS = [1000, 1000, 999, 1000]


def _cache(extra, seed, max_groups=None):
    old = os.environ.get("AKV_MAX_OP_GROUPS")
    if max_groups is not None:
        os.environ["AKV_MAX_OP_GROUPS"] = str(max_groups)
    try:
        c = Hn.make_cache(SH, LENS, extra)
    finally:
        if max_groups is not None:
            if old is None:
                os.environ.pop("AKV_MAX_OP_GROUPS")
            else:
                os.environ["AKV_MAX_OP_GROUPS"] = old
    c.reset()
    Hn.fill(c, SH, LENS, seed, gen_device="cpu")
    assert c.sync_status() == 0
    return c


def test_ops_split_into_sequence_groups():
    # 70 spare pages: each sequence's rebuild (<= 63 pages) fits, the op's
    # (~4 x 55) does not
    c = _cache(70, 61)
    oc = oracle_for(SH, LENS, 61)
    say(f"case grouped drop: {c.NB} pages, 70 free, 4 sequences of ~63 pages")
    m1 = [W.spans_to_mask(n, [(100, 50)]) for n in LENS]
    c.drop(Hn.mask_tensor(c, m1))
    assert c.sync_status() == 0
    srcs = [oc.drop(b, m) for b, m in enumerate(m1)]
    check_meta(c, oc)
    check_kv(c, oc, k_ulp=0)
    rows = c.query_state(with_last_src=True)[4].cpu().numpy()
    for b, src in enumerate(srcs):
        assert np.array_equal(rows[b, :len(src)], src)
    assert int(c.free_count.item()) == 70 + 4 * 3            # 50 entries = 3 pages freed each
    say("case grouped drop+reposition: in-place re-rotation before the first dropped page")
    m2 = [W.spans_to_mask(len(oc.seqs[b]), [(300, 10)]) for b in range(4)]
    c.drop_reposition(Hn.mask_tensor(c, m2))
    assert c.sync_status() == 0
    for b, m in enumerate(m2):
        oc.drop_reposition(b, m)
    check_meta(c, oc)
    worst = check_kv(c, oc, k_ulp=1)
    say(f"grouped ops match the oracle (K within {worst} step)")
    # the pool is intact: every page is either held or free, exactly once
    held = [c.block_table[b, :Hn.pages_for(len(oc.seqs[b]))].cpu().numpy() for b in range(4)]
    fc = int(c.free_count.item())
    free = c.free_stack[:fc].cpu().numpy()
    allp = np.concatenate(held + [free])
    assert np.array_equal(np.sort(allp), np.arange(c.NB))


def test_too_many_groups_and_too_big_a_sequence_are_rejected():
    c = _cache(70, 62, max_groups=2)       # the op needs 4 groups, 2 rounds are enqueued
    snap = c.meta.clone()
    kb = bits(c.k_pool)
    say("case grouped drop needing more groups than the rounds enqueued")
    m = [W.spans_to_mask(n, [(0, 20)]) for n in LENS]
    c.drop(Hn.mask_tensor(c, m))
    assert c.sync_status() == 4
    assert torch.equal(c.meta, snap) and np.array_equal(bits(c.k_pool), kb)
    say("case a sequence that does not fit the free pool on its own")
    c2 = _cache(40, 63)                    # 40 spare pages < one sequence's ~62
    snap = c2.meta.clone()
    c2.drop(Hn.mask_tensor(c2, m))
    assert c2.sync_status() == 4
    assert torch.equal(c2.meta, snap)
    say("case the same op with enough groups runs")
    c3 = _cache(70, 62)
    oc = oracle_for(SH, LENS, 62)
    c3.drop(Hn.mask_tensor(c3, m))
    assert c3.sync_status() == 0
    for b, mb in enumerate(m):
        oc.drop(b, mb)
    check_meta(c3, oc)
    check_kv(c3, oc, k_ulp=0)
