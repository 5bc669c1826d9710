"""Host-side checks of the synthetic workload recipes (no GPU)."""
import numpy as np

from agent_kv_cache_amd import workloads as W
from oracle import akv_oracle as O


def test_restore_segments_cover_the_request_once():
    r = W.restore_llama8b_32k()
    wl = W.llama8b_32k()
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
    ra, rb = W.restore_llama8b_32k(), W.restore_llama8b_32k()
    for (ma, na), (mb, nb) in zip(ra.versions, rb.versions):
        assert na == nb and np.array_equal(ma, mb)


def test_history_max_active_matches_a_metadata_replay():
    """The page capacity of the long-history cache is sized from
    History.max_active(); check it against the oracle's own replay of the
    run (lengths after every op, token sets from the message ids)."""
    h = W.history_50_turns()
    oc = O.OracleCache(1, 1, 8, 1.5e5, n_seqs=1, with_kv=False)
    top = 0
    for op in h.ops:
        if op[0] == "append":
            mid, n = op[1], op[2]
            oc.append(0, np.arange(h.msg_start[mid], h.msg_start[mid] + n))
        elif op[0] == "repos":
            oc.reposition(0)
        else:
            tok = oc.seqs[0].token_ids
            mask = W.mask_for_messages(tok, h, op[1])
            (oc.drop if op[0] == "drop" else oc.drop_reposition)(0, mask)
        top = max(top, len(oc.seqs[0]))
    assert h.max_active() == top
    assert len(oc.seqs[0]) < top <= h.total_tokens
