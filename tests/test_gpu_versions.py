"""GPU parity of position versions (akv_fork) and segment-batch attention
(akv_segment_attention) against the fp64 oracle, through the C ABI.

Bars as for the other GPU tests: token ids, positions, lengths, next_pos
bit-exact; K within 1 bf16 step of the oracle per rotation; V bit-exact;
attention within 1e-2 max abs error.  A fork leaves its source bitwise
unchanged.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from agent_kv_cache_amd import harness as Hn  # noqa: E402
from agent_kv_cache_amd import workloads as W  # noqa: E402
from agent_kv_cache_amd.binding import AkvError  # noqa: E402
from oracle import akv_oracle as O  # noqa: E402

from gpu_util import (bits, check_kv, check_meta, oracle_for, say, to_f64,  # noqa: E402
                      append_seeded as _append, check_segments as _check_segments,
                      run_segments as _segments, snapshot as _snapshot, same_state as _same)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from agent_kv_cache_amd.binding import lib
    lib()


# ---------------------------------------------------------------------------
# Figure 10: four versions, four segments in one launch
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 128])
def test_fig10_versions_and_segments(d):
    sh = W.Shape(2, 2, d, 4, 1.0e4)
    B = 4
    say(f"case fig10 versions d={d}")
    cache = Hn.make_cache(sh, [0] * B, 16, max_blocks_per_seq=2)
    cache.reset()
    oc = O.OracleCache(sh.n_layers, sh.n_kv_heads, d, sh.rope_base, n_seqs=B)
    names = "ABCDEF"
    kv = {n: (W.randn_bf16((sh.n_layers, 1, sh.n_kv_heads, d), 40 + 2 * i),
              W.randn_bf16((sh.n_layers, 1, sh.n_kv_heads, d), 41 + 2 * i))
          for i, n in enumerate(names)}

    def app(b, n):
        k, v = kv[n]
        cnt = [0] * B
        cnt[b] = 1
        tid = names.index(n)
        cache.append(torch.tensor(cnt, dtype=torch.int32, device=cache.device), 1,
                     k.to(cache.device), v.to(cache.device),
                     torch.tensor([tid], dtype=torch.int32, device=cache.device))
        oc.append(b, [tid], to_f64(k.permute(1, 0, 2, 3)), to_f64(v.permute(1, 0, 2, 3)))

    def mask(b, drop):
        return np.array([names[t] in drop for t in oc.seqs[b].token_ids], np.uint8)

    def fork(src, dst, drop, repos):
        dst_of = [-1] * B
        dst_of[src] = dst
        m = None
        if drop:
            mm = [None] * B
            mm[src] = mask(src, drop)
            m = Hn.mask_tensor(cache, mm)
        src_before = _snapshot(cache, src)
        cache.fork(dst_of, m, reposition=repos)
        assert cache.sync_status() == 0
        oc.fork(src, dst, None if not drop else mask(src, drop), reposition=repos)
        _same(src_before, _snapshot(cache, src))

    for n in "ABC":
        app(0, n)
    fork(0, 1, "B", True)
    app(1, "D")
    fork(1, 2, "D", False)
    app(2, "E")
    fork(2, 3, None, True)
    app(3, "F")
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    want = {0: {"A": 0, "B": 1, "C": 2}, 1: {"A": 0, "C": 1, "D": 2},
            2: {"A": 0, "C": 1, "E": 3}, 3: {"A": 0, "C": 1, "E": 2, "F": 3}}
    for b in range(B):
        tok, pos, _ = cache.seq_state(b)
        assert {names[t]: int(p) for t, p in zip(tok, pos)} == want[b]
    assert [int(x) for x in cache.next_pos.cpu()] == [3, 3, 4, 4]
    segs = [(0, 3), (1, 1), (2, 1), (3, 1)]
    q = W.randn_bf16((6, sh.n_layers, sh.n_q_heads, d), 77).to(cache.device)
    out = _segments(cache, q, segs)
    assert cache.sync_status() == 0
    err = _check_segments(oc, q, out, segs)
    say("fig10 segment max abs err", err)


# ---------------------------------------------------------------------------
# forks on random ragged caches
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("seed", [0, 1])
def test_fork_random(d, seed):
    rng = np.random.default_rng(500 + seed)
    sh = W.Shape(3, 2, d, 8, 5.0e5)
    lens = [0, 1, 40, 333, 700, 129, 0, 0, 0, 0]
    B = len(lens)
    say(f"case fork random d={d} seed={seed}")
    cache = Hn.make_cache(sh, lens, 400, max_blocks_per_seq=48)
    cache.reset(np.random.default_rng(seed).permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, sh, lens, seed, gen_device="cpu")
    assert cache.sync_status() == 0
    oc = oracle_for(sh, lens, seed)
    snaps = {b: _snapshot(cache, b) for b in range(6)}
    # copy, drop + canonical repos, drop only, drop + explicit positions
    masks = [None] * B
    newp = [None] * B
    for b in (3, 4, 5):
        masks[b] = (rng.uniform(size=lens[b]) < 0.35).astype(np.uint8)
    masks[4][:20] = 0
    r5 = lens[5] - int(masks[5].sum())
    newp[5] = (np.cumsum(rng.integers(1, 4, size=r5)) + 7).astype(np.int32)
    # 1 -> 6, 4 -> 8, 3 -> 7, 5 -> 9: one call per transform kind
    cache.fork([-1, 6] + [-1] * 8)
    oc.fork(1, 6)
    cache.fork([-1] * 4 + [8] + [-1] * 5, Hn.mask_tensor(cache, masks))
    oc.fork(4, 8, masks[4])
    cache.fork([-1] * 3 + [7] + [-1] * 6, Hn.mask_tensor(cache, masks), reposition=True)
    oc.fork(3, 7, masks[3], reposition=True)
    cache.fork([-1] * 5 + [9] + [-1] * 4, Hn.mask_tensor(cache, masks), reposition=True,
               new_pos=Hn.pos_tensor(cache, newp))
    oc.fork(5, 9, masks[5], reposition=True, new_pos=newp[5])
    assert cache.sync_status() == 0
    for b in range(6):
        _same(snaps[b], _snapshot(cache, b))
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    # a plain copy is bitwise the source
    c6 = _snapshot(cache, 6)
    for x, y in zip(snaps[1][3] + snaps[1][4], c6[3] + c6[4]):
        assert np.array_equal(x, y)


def test_fork_many_in_one_call_then_segments():
    """Several forks in one call (same mode), then segments over sources and
    versions together, GQA 4, ragged rows across query blocks."""
    rng = np.random.default_rng(71)
    sh = W.Shape(2, 2, 128, 8, 5.0e5)
    lens = [260, 97, 515, 0, 0, 0]
    B = len(lens)
    say("case multi-fork + segments")
    cache = Hn.make_cache(sh, lens, 200, max_blocks_per_seq=40)
    cache.reset(np.random.default_rng(3).permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, sh, lens, 9, gen_device="cpu")
    oc = oracle_for(sh, lens, 9)
    masks = [(rng.uniform(size=n) < 0.25).astype(np.uint8) for n in lens]
    cache.fork([3, 4, 5, -1, -1, -1], Hn.mask_tensor(cache, masks), reposition=True)
    for s, t in ((0, 3), (1, 4), (2, 5)):
        oc.fork(s, t, masks[s], reposition=True)
    assert cache.sync_status() == 0
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    # each version gets its own new tokens (the segment's queries)
    _append(cache, oc, sh, [0, 0, 0, 37, 5, 16], 990, 1 << 27)
    assert cache.sync_status() == 0
    segs = [(3, 37), (4, 5), (5, 16), (0, 1), (2, 33), (2, 0), (1, 97)]
    nq = sum(n for _, n in segs)
    q = W.randn_bf16((nq, sh.n_layers, sh.n_q_heads, 128), 991).to(cache.device)
    out = _segments(cache, q, segs)
    assert cache.sync_status() == 0
    err = _check_segments(oc, q, out, segs)
    say("multi-fork segments max abs err", err)


def test_fork_errors():
    sh = W.Shape(1, 2, 64, 4, 1.0e4)
    lens = [20, 30, 5, 0]
    cache = Hn.make_cache(sh, lens, 8, max_blocks_per_seq=4)
    cache.reset()
    Hn.fill(cache, sh, lens, 1, gen_device="cpu")
    assert cache.sync_status() == 0
    say("case fork errors")
    before = [_snapshot(cache, b) for b in range(4)]
    cache.fork([1, -1, -1, -1])            # destination not empty: device check
    assert cache.sync_status() == 1
    for bad in ([0, -1, -1, -1],           # onto itself
                [3, -1, -1, 3],            # destination used twice
                [-1, -1, -1, 4],           # out of range
                [3, -1, -1, -2],           # bad code
                [-1, 3, -1, 1]):           # a destination that is also a source
        with pytest.raises(AkvError):
            cache.fork(bad)
    with pytest.raises(AkvError):
        cache.fork([3, -1, -1, -1], None, reposition=False,
                   new_pos=Hn.pos_tensor(cache, [None] * 4))
    # pool exhaustion: 2 spare pages.  A plain copy of 60 entries shares its
    # 3 full pages and copies 1 (fits); dropping the first entry leaves
    # nothing to share, and 59 entries need 4 fresh pages (rejected)
    big = Hn.make_cache(sh, [60, 0], 2, max_blocks_per_seq=4)
    big.reset()
    Hn.fill(big, sh, [60, 0], 2, gen_device="cpu")
    b0 = _snapshot(big, 0)
    first = Hn.mask_tensor(big, [np.r_[1, np.zeros(59, np.uint8)].astype(np.uint8), None])
    big.fork([1, -1], first)
    assert big.sync_status() == 4
    _same(b0, _snapshot(big, 0))
    assert int(big.seq_lens[1]) == 0
    big.fork([1, -1])
    assert big.sync_status() == 0 and int(big.seq_lens[1]) == 60
    for b in range(4):
        _same(before[b], _snapshot(cache, b))
    # the cache still works after the rejected calls
    cache.fork([-1, -1, 3, -1])
    assert cache.sync_status() == 0
    c3 = _snapshot(cache, 3)
    for x, y in zip(before[2][3] + before[2][4], c3[3] + c3[4]):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# segment attention on its own
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_segment_attention_gqa(G, d):
    H = 2
    sh = W.Shape(2, H, d, H * G, 1.0e4)
    lens = [1, 16, 100, 513, 257]
    say(f"case segments G={G} d={d}")
    cache = Hn.make_cache(sh, lens, 0)
    cache.reset(np.random.default_rng(G).permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, sh, lens, 20 + G, gen_device="cpu")
    oc = oracle_for(sh, lens, 20 + G)
    # whole-sequence prefill, decode-like single rows, ragged blocks, repeats
    segs = [(0, 1), (1, 16), (2, 100), (3, 45), (4, 1), (3, 17), (4, 257)]
    nq = sum(n for _, n in segs)
    q = W.randn_bf16((nq, sh.n_layers, sh.n_q_heads, d), 100 + G).to(cache.device)
    out = _segments(cache, q, segs)
    assert cache.sync_status() == 0
    err = _check_segments(oc, q, out, segs)
    say("segments max abs err", err)
    # a layer sub-range: out only covers those layers
    q1 = q[:, 1:2].contiguous()
    out1 = _segments(cache, q1, segs, layer_begin=1, n_layers=1)
    assert torch.equal(out1, out[:, 1:2])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 3, 4, 16])
def test_segment_attention_short_segments(G, d):
    """Every segment within one 16-column tile (16 // G rows): the split-KV
    kernel; many segments over few sequences, ragged lengths."""
    H = 2
    sh = W.Shape(3, H, d, H * G, 5.0e5)
    lens = [5, 16, 17, 300, 1111]
    tb = 16 // G
    say(f"case short segments G={G} d={d}")
    cache = Hn.make_cache(sh, lens, 0)
    cache.reset(np.random.default_rng(40 + G).permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, sh, lens, 60 + G, gen_device="cpu")
    oc = oracle_for(sh, lens, 60 + G)
    rng = np.random.default_rng(G)
    segs = [(b, int(rng.integers(0, tb + 1))) for b in range(len(lens)) for _ in range(3)]
    segs = [(b, min(n, lens[b])) for b, n in segs]
    nq = sum(n for _, n in segs)
    q = W.randn_bf16((max(nq, 1), sh.n_layers, sh.n_q_heads, d), 700 + G).to(cache.device)
    out = _segments(cache, q, segs, max_q=tb)
    assert cache.sync_status() == 0
    err = _check_segments(oc, q, out, segs)
    say("short segments max abs err", err)


def test_segment_attention_sharp_and_errors():
    sh = W.Shape(1, 1, 128, 4, 1.0e4)
    lens = [40, 70]
    cache = Hn.make_cache(sh, lens, 0)
    cache.reset()
    Hn.fill(cache, sh, lens, 5, gen_device="cpu")
    oc = oracle_for(sh, lens, 5)
    say("case segments sharp softmax + errors")
    segs = [(0, 40), (1, 9)]
    q = (W.randn_bf16((49, 1, 4, 128), 6) * 4).to(cache.device)   # large logits
    out = _segments(cache, q, segs)
    assert cache.sync_status() == 0
    _check_segments(oc, q, out, segs)
    # more rows than entries: ARG latched, rows zero
    out = _segments(cache, q[:41].contiguous(), [(0, 41)])
    assert cache.sync_status() == 1
    assert torch.count_nonzero(out) == 0
    # max_q below a segment's rows: ARG latched
    _segments(cache, q[:9].contiguous(), [(1, 9)], max_q=4)
    assert cache.sync_status() == 1
    # sequence out of range: ARG latched
    _segments(cache, q[:1].contiguous(), [(5, 1)])
    assert cache.sync_status() == 1
    # host checks
    dev = cache.device
    seq = torch.zeros(1, dtype=torch.int32, device=dev)
    off = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    o1 = torch.empty_like(q[:1])
    with pytest.raises(AkvError):
        cache.segment_attention(q[:1], seq, off, 0, o1)
    q17 = torch.zeros((1, 1, 17, 128), dtype=torch.bfloat16, device=dev)   # GQA ratio 17
    with pytest.raises(AkvError):
        cache.segment_attention(q17, seq, off, 1, torch.empty_like(q17))
    with pytest.raises(AkvError):
        cache.segment_attention(q[:1], seq, off, 1, o1, layer_begin=1)
    # still fine afterwards
    out = _segments(cache, q, segs)
    assert cache.sync_status() == 0
    _check_segments(oc, q, out, segs)
