"""Host-side checks of the synthetic workload recipes (no GPU)."""
import numpy as np

from agent_kv_cache_amd import workloads as W
from oracle import akv_oracle as O


def test_restore_c2_segments_cover_the_request_once():
    r = W.restore_c2()
    wl = W.c2()
    n = r.n_tokens
    spans = sorted(wl.spans[0])
    oc = O.OracleCache(1, 1, 8, 1e4, n_seqs=1 + len(r.versions), with_kv=False)
    oc.append(0, np.arange(n))
    covered = np.zeros(n, dtype=int)
    for j, (mask, rows) in enumerate(r.versions):
        oc.fork(0, j + 1, mask, reposition=True)
        s = oc.seqs[j + 1]
        own = s.token_ids[len(s) - rows:]
        covered[own] += 1
        assert np.array_equal(own, np.arange(own[0], own[0] + rows)) if rows else True
        assert np.array_equal(s.pos, np.arange(len(s)))
        assert s.next_pos == len(s)
        present = np.zeros(n, bool)
        present[s.token_ids] = True
        for k, (st, ln) in enumerate(spans):
            if k < j - 1:
                assert not present[st:st + ln].any()        # dropped before segment j
            elif k == j - 1:
                assert present[st:st + ln].all()            # segment j's own tool span
        # everything before the segment that is not a dropped span is visible
        if rows:
            lo = int(own[0])
            dropped = np.zeros(n, bool)
            for st, ln in spans[:max(0, j - 1)]:
                dropped[st:st + ln] = True
            assert np.array_equal(present[:lo], ~dropped[:lo])
    assert (covered == 1).all()
    assert oc.seqs[0].next_pos == n and len(oc.seqs[0]) == n


def test_workloads_are_deterministic():
    for name, fn in W.WORKLOADS.items():
        a, b = fn(), fn()
        assert a.seq_lens == b.seq_lens, name
        for x, y in zip(a.masks, b.masks):
            assert np.array_equal(x, y), name
    ra, rb = W.restore_c2(), W.restore_c2()
    for (ma, na), (mb, nb) in zip(ra.versions, rb.versions):
        assert na == nb and np.array_equal(ma, mb)
