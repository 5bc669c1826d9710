"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: compaction indices (token ids per slot), positions, lengths and
next_pos bit-exact; re-rotated keys within 1 bf16 step of the oracle's
one-step-rounded fp64 result; V bit-exact; decode attention within 1e-2
max abs error.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from agent_kv_cache_amd import harness as Hn  # noqa: E402
from agent_kv_cache_amd import workloads as W  # noqa: E402
from agent_kv_cache_amd.binding import AkvError  # noqa: E402
from oracle import akv_oracle as O  # noqa: E402

from gpu_util import (bits, check_attention, check_kv, check_meta, oracle_for,  # noqa: E402
                      q_tensor, say)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from agent_kv_cache_amd.binding import lib
    lib()  # fail loudly if the library is missing


def _setup(shape, lens, seed=1, extra=None, order_seed=None, maxpg=None, **cache_kw):
    cache = Hn.make_cache(shape, lens, sum(Hn.pages_for(n) for n in lens) if extra is None else extra,
                          max_blocks_per_seq=maxpg, **cache_kw)
    order = None
    if order_seed is not None:
        order = np.random.default_rng(order_seed).permutation(cache.NB).astype(np.int32)
    cache.reset(order)
    Hn.fill(cache, shape, lens, seed, gen_device="cpu")
    assert cache.sync_status() == 0
    return cache


def _decode(cache, q, active=None):
    out = torch.empty_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(q.shape[1], q.shape[2])),
                     dtype=torch.uint8, device=cache.device)
    act = None if active is None else torch.tensor(active, dtype=torch.int32, device=cache.device)
    cache.decode_attention(q, out, ws, active_len=act)
    return out


# ---------------------------------------------------------------------------
# configuration 1, full
# ---------------------------------------------------------------------------
def test_one_layer_drop_reposition_decode():
    wl = W.one_layer_4k()
    sh = wl.shape
    say("case one_layer_4k: append 4096, drop [1024,2048) + repos, decode 32 heads")
    cache = _setup(sh, wl.seq_lens, seed=wl.data_seed)
    oc = oracle_for(sh, wl.seq_lens, wl.data_seed)
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=0)
    cache.drop_reposition(Hn.mask_tensor(cache, wl.masks))
    assert cache.sync_status() == 0
    oc.drop_reposition(0, wl.masks[0])
    check_meta(cache, oc)
    assert int(cache.next_pos[0]) == 3072
    worst = check_kv(cache, oc, k_ulp=1)
    say("one_layer_4k worst K ulp", worst)
    q = q_tensor(sh, 1, 1, 201).to(cache.device)
    out = _decode(cache, q)
    err = check_attention(cache, oc, q, out)
    say("one_layer_4k attention max abs err", err)


# ---------------------------------------------------------------------------
# small random caches: many sequences, shuffled pages, every op kind
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_small_random_op_chains(d, seed):
    rng = np.random.default_rng(100 + seed)
    sh = W.Shape(2, 2, d, 8, 1.0e4 if seed == 0 else 5.0e5)
    B = 5
    lens = [0, 1, 17, 70, 129][: B]
    rng.shuffle(lens)
    say(f"case small chain d={d} seed={seed} lens={lens}")
    cache = _setup(sh, lens, seed=seed, extra=60, order_seed=seed, maxpg=24)
    oc = oracle_for(sh, lens, seed)
    check_meta(cache, oc)
    for step in range(6):
        kind = ["drop", "drop_repos", "repos", "drop_repos_explicit", "repos_explicit", "drop"][step]
        masks, newp = [], []
        for b in range(B):
            n = len(oc.seqs[b])
            m = (rng.uniform(size=n) < rng.uniform(0, 0.6)).astype(np.uint8)
            masks.append(m)
            r = n - int(m.sum()) if "drop" in kind else n
            newp.append(np.cumsum(rng.integers(1, 5, size=r)) + int(rng.integers(0, 50)))
        say(" step", step, kind)
        if kind == "drop":
            cache.drop(Hn.mask_tensor(cache, masks))
            for b in range(B):
                oc.drop(b, masks[b])
        elif kind == "drop_repos":
            cache.drop_reposition(Hn.mask_tensor(cache, masks))
            for b in range(B):
                oc.drop_reposition(b, masks[b])
        elif kind == "drop_repos_explicit":
            cache.drop_reposition(Hn.mask_tensor(cache, masks), Hn.pos_tensor(cache, newp))
            for b in range(B):
                oc.drop_reposition(b, masks[b], newp[b])
        elif kind == "repos":
            cache.reposition()
            for b in range(B):
                oc.reposition(b)
        else:
            old = [oc.seqs[b].pos.copy() for b in range(B)]
            cache.reposition(Hn.pos_tensor(cache, old), Hn.pos_tensor(cache, newp))
            for b in range(B):
                oc.reposition(b, newp[b])
        assert cache.sync_status() == 0
        check_meta(cache, oc)
        # chain bound: one rounding per non-identity rotation so far
        check_kv(cache, oc, k_ulp=step + 1)
        # append a few tokens to exercise partial pages after the op
        if step == 2:
            add = [int(x) for x in rng.integers(0, 20, size=B)]
            N = sum(add)
            k = W.randn_bf16((sh.n_layers, N, sh.n_kv_heads, d), 900 + seed)
            v = W.randn_bf16((sh.n_layers, N, sh.n_kv_heads, d), 950 + seed)
            tid = np.arange(N) + (1 << 28)
            cache.append(torch.tensor(add, dtype=torch.int32, device=cache.device), N,
                         k.to(cache.device), v.to(cache.device),
                         torch.tensor(tid, dtype=torch.int32, device=cache.device))
            o = 0
            for b in range(B):
                sl = slice(o, o + add[b])
                oc.append(b, tid[sl], k[:, sl].permute(1, 0, 2, 3).double().numpy(),
                          v[:, sl].permute(1, 0, 2, 3).double().numpy())
                o += add[b]
            assert cache.sync_status() == 0
            check_meta(cache, oc)
    q = q_tensor(sh, B, sh.n_layers, 300 + seed).to(cache.device)
    out = _decode(cache, q)
    check_attention(cache, oc, q, out)
    act = [int(rng.integers(0, len(s) + 1)) for s in oc.seqs]
    out = _decode(cache, q, act)
    check_attention(cache, oc, q, out, active=act)


def test_brute_force_every_mask_len_9():
    """All 512 masks of one 9-entry sequence (spanning a page boundary with
    an offset start), drop + canonical reposition, vs the oracle."""
    sh = W.Shape(1, 1, 64, 2, 1.0e4)
    B = 8
    lens = [9 + 16 * (b % 2) for b in range(B)]
    say("case brute force masks, 64 launches of 8 sequences")
    for chunk in range(0, 512, B):
        cache = _setup(sh, lens, seed=chunk, extra=40)
        oc = oracle_for(sh, lens, chunk)
        masks = []
        for b in range(B):
            code = chunk + b
            m9 = np.array([(code >> i) & 1 for i in range(9)], np.uint8)
            m = np.zeros(lens[b], np.uint8)
            o = 0 if lens[b] == 9 else 12           # window [12, 21) crosses a page edge
            m[o:o + 9] = m9
            masks.append(m)
        cache.drop_reposition(Hn.mask_tensor(cache, masks))
        assert cache.sync_status() == 0
        for b in range(B):
            oc.drop_reposition(b, masks[b])
        check_meta(cache, oc)
        check_kv(cache, oc, k_ulp=1)


def test_fused_equals_sequential_bitwise():
    sh = W.Shape(3, 2, 128, 8, 5.0e5)
    lens = [300, 45, 1000]
    rng = np.random.default_rng(7)
    masks = [(rng.uniform(size=n) < 0.3).astype(np.uint8) for n in lens]
    say("case fused vs sequential")
    a = _setup(sh, lens, seed=3, order_seed=4)
    b = _setup(sh, lens, seed=3, order_seed=4)
    a.drop_reposition(Hn.mask_tensor(a, masks))
    b.drop(Hn.mask_tensor(b, masks))
    b.reposition()
    assert a.sync_status() == 0 and b.sync_status() == 0
    for s in range(len(lens)):
        ta, pa, _ = a.seq_state(s)
        tb, pb, _ = b.seq_state(s)
        assert np.array_equal(ta, tb) and np.array_equal(pa, pb)
        for l in range(sh.n_layers):
            assert np.array_equal(bits(a.gather_rows(s, l, "k")), bits(b.gather_rows(s, l, "k")))
            assert np.array_equal(bits(a.gather_rows(s, l, "v")), bits(b.gather_rows(s, l, "v")))
    assert np.array_equal(a.next_pos.cpu().numpy(), b.next_pos.cpu().numpy())


@pytest.mark.parametrize("d,r", [(128, 128), (64, 64), (128, 64), (64, 48)])
def test_move_launch_shapes_agree_bitwise(monkeypatch, d, r):
    """The one-shot and the persistent move grid give identical bytes: the
    same ops on two identically filled caches, the second with the one-shot
    grid switched off (AKV_MOVE_ONESHOT_CAP=0, read at cache creation).  Head
    sizes and rotary widths cover both thread mappings of the move (half rows
    for full RoPE at d = 128, full rows otherwise)."""
    sh = W.Shape(3, 2, d, 8, 5.0e5)
    lens = [700, 45, 1000, 0]
    rng = np.random.default_rng(17)
    masks = [(rng.uniform(size=n) < 0.35).astype(np.uint8) for n in lens]
    say(f"case one-shot vs persistent move grid d={d} r={r}")
    kw = {"rotary_dim": r} if r != d else {}
    a = _setup(sh, lens, seed=5, extra=2 * sum(Hn.pages_for(n) for n in lens) + 8, order_seed=6, **kw)
    monkeypatch.setenv("AKV_MOVE_ONESHOT_CAP", "0")
    b = _setup(sh, lens, seed=5, extra=2 * sum(Hn.pages_for(n) for n in lens) + 8, order_seed=6, **kw)
    monkeypatch.delenv("AKV_MOVE_ONESHOT_CAP")
    for c in (a, b):
        c.drop_reposition(Hn.mask_tensor(c, masks))
        # every entry to its own gapped position: every row a different delta
        newp = [np.arange(int(n)) * 7 + 3 + 11 * s for s, n in enumerate(c.seq_lens.cpu().numpy())]
        c.reposition(None, Hn.pos_tensor(c, newp))
        c.drop(Hn.mask_tensor(c, [np.zeros(int(n), np.uint8) if s != 2 else
                                  (np.arange(int(n)) % 5 == 1).astype(np.uint8)
                                  for s, n in enumerate(c.seq_lens.cpu().numpy())]))
        c.fork([3, -1, -1, -1], None, reposition=True)
        assert c.sync_status() == 0
    for s in range(len(lens)):
        ta, pa, _ = a.seq_state(s)
        tb, pb, _ = b.seq_state(s)
        assert np.array_equal(ta, tb) and np.array_equal(pa, pb), s
        for l in range(sh.n_layers):
            assert np.array_equal(bits(a.gather_rows(s, l, "k")), bits(b.gather_rows(s, l, "k"))), (s, l)
            assert np.array_equal(bits(a.gather_rows(s, l, "v")), bits(b.gather_rows(s, l, "v"))), (s, l)
    assert np.array_equal(a.next_pos.cpu().numpy(), b.next_pos.cpu().numpy())
    assert np.array_equal(a.seq_lens.cpu().numpy(), b.seq_lens.cpu().numpy())


def test_identity_reposition_is_bitwise_copy():
    sh = W.Shape(2, 2, 128, 4, 5.0e5)
    lens = [100, 33]
    say("case identity reposition")
    c = _setup(sh, lens, seed=11)
    before = [bits(c.gather_rows(s, l, "k")) for s in range(2) for l in range(2)]
    old = [np.arange(n) for n in lens]
    c.reposition(Hn.pos_tensor(c, old), Hn.pos_tensor(c, old))
    assert c.sync_status() == 0
    after = [bits(c.gather_rows(s, l, "k")) for s in range(2) for l in range(2)]
    for x, y in zip(before, after):
        assert np.array_equal(x, y)


def test_errors_leave_state_unchanged():
    sh = W.Shape(2, 2, 64, 4, 1.0e4)
    lens = [40, 20]
    say("case error paths")
    c = _setup(sh, lens, seed=5, extra=0)      # no spare pages at all
    snap = c.meta.clone()
    kb = bits(c.k_pool)
    # not strictly increasing new positions
    bad = [np.arange(40), np.array([0, 1, 1] + list(range(3, 20)))]
    c.reposition(None, Hn.pos_tensor(c, bad))
    assert c.sync_status() == 2
    # old positions that do not match
    c.reposition(Hn.pos_tensor(c, [np.arange(40) + 1, np.arange(20)]), None)
    assert c.sync_status() == 3
    # pool exhausted: a drop needs fresh pages
    m = [np.r_[np.ones(3, np.uint8), np.zeros(37, np.uint8)], np.zeros(20, np.uint8)]
    c.drop(Hn.mask_tensor(c, m))
    assert c.sync_status() == 4
    assert torch.equal(c.meta, snap)
    assert np.array_equal(bits(c.k_pool), kb)
    # a latched error turns later ops into no-ops until it is read
    c.reposition(None, Hn.pos_tensor(c, bad))
    c.reposition()                       # would succeed, but the error is latched
    assert c.sync_status() == 2
    assert torch.equal(c.meta, snap)
    # capacity: appending past max_blocks_per_seq
    cnt = torch.tensor([10_000, 0], dtype=torch.int32, device=c.device)
    k = torch.zeros((2, 10_000, 2, 64), dtype=torch.bfloat16, device=c.device)
    c.append(cnt, 10_000, k, k, torch.zeros(10_000, dtype=torch.int32, device=c.device))
    assert c.sync_status() == 5
    assert torch.equal(c.meta, snap)
    # host-checked arguments
    with pytest.raises(AkvError):
        c.drop(None)
    q = torch.zeros((2, 2, 5, 64), dtype=torch.bfloat16, device=c.device)
    with pytest.raises(AkvError):
        _decode(c, q)                    # 5 query heads is not a multiple of 2


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 16])
def test_decode_gqa_ratios(G, d):
    sh = W.Shape(2, 2, d, 2 * G, 5.0e5)
    lens = [1, 16, 250, 513]
    say(f"case decode G={G} d={d}")
    c = _setup(sh, lens, seed=20 + G + d)
    oc = oracle_for(sh, lens, 20 + G + d)
    q = q_tensor(sh, len(lens), 2, 40 + G + d).to(c.device)
    out = _decode(c, q)
    check_attention(c, oc, q, out)
    out = _decode(c, q, [0, 3, 250, 100])
    check_attention(c, oc, q, out, active=[0, 3, 250, 100])


@pytest.mark.parametrize("d", [64, 128])
def test_decode_sharp_softmax(d):
    """Scaled-up queries make the softmax nearly one-hot: checks the running
    max and the rescaling across pages and splits."""
    sh = W.Shape(1, 1, d, 4, 5.0e5)
    lens = [3000]
    c = _setup(sh, lens, seed=31)
    oc = oracle_for(sh, lens, 31)
    q = (q_tensor(sh, 1, 1, 32) * 6).to(torch.bfloat16).to(c.device)
    out = _decode(c, q)
    check_attention(c, oc, q, out)


# ---------------------------------------------------------------------------
# configuration 2 at full size (Llama-3.1-8B shape, 32768 tokens)
# ---------------------------------------------------------------------------
@pytest.mark.timeout(400)
def test_llama8b_full_size_sampled():
    wl = W.llama8b_32k()
    sh = wl.shape
    say("case llama8b_32k full size: fill 32768 tokens x 32 layers")
    extra = Hn.moved_pages(wl.seq_lens[0], wl.masks[0])
    cache = Hn.make_cache(sh, wl.seq_lens, extra)
    cache.reset()
    Hn.fill(cache, sh, wl.seq_lens, wl.data_seed, gen_device="cuda")
    layers = [0, 17, 31]
    oc = oracle_for(sh, wl.seq_lens, wl.data_seed, layers=layers, gen_device="cuda")
    say("llama8b_32k drop+repos")
    cache.drop_reposition(Hn.mask_tensor(cache, wl.masks))
    assert cache.sync_status() == 0
    oc.drop_reposition(0, wl.masks[0])
    check_meta(cache, oc)
    worst = check_kv(cache, oc, layers=layers, k_ulp=1)
    say("llama8b_32k worst K ulp on sampled layers", worst)
    q = q_tensor(sh, 1, sh.n_layers, 202, device="cuda")
    out = _decode(cache, q)
    err = check_attention(cache, oc, q, out, layers=layers)
    say("llama8b_32k attention max abs err (sampled layers)", err)
    # the same decode as one launch per layer (split-K over one layer's rows
    # and the combine kernel), as the benchmark also times it
    out_pl = torch.zeros_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(1, sh.n_q_heads)), dtype=torch.uint8,
                     device=cache.device)
    for l in layers:
        ol = torch.empty_like(q[:, l:l + 1])
        cache.decode_attention(q[:, l:l + 1].contiguous(), ol, ws, layer_begin=l, n_layers=1)
        out_pl[:, l:l + 1] = ol
    assert cache.sync_status() == 0
    err = check_attention(cache, oc, q, out_pl, layers=layers, what="per-layer launches")
    say("llama8b_32k per-layer attention max abs err (sampled layers)", err)


def test_degenerate_masks_and_positions():
    """Drop everything, drop nothing, reposition non-canonical positions in
    place, refill an emptied sequence, and decode over empty sequences."""
    sh = W.Shape(2, 2, 128, 4, 5.0e5)
    lens = [40, 37, 0]
    say("case degenerate masks")
    c = _setup(sh, lens, seed=41, extra=20, maxpg=8)
    oc = oracle_for(sh, lens, 41)
    # seq 0: drop nothing; seq 1: drop everything; seq 2: empty
    masks = [np.zeros(40, np.uint8), np.ones(37, np.uint8), np.zeros(0, np.uint8)]
    c.drop(Hn.mask_tensor(c, masks))
    for b in range(3):
        oc.drop(b, masks[b])
    assert c.sync_status() == 0
    check_meta(c, oc)
    assert int(c.seq_lens[1]) == 0 and int(c.next_pos[1]) == 37   # drop keeps next_pos
    # positions with gaps, then a reposition with nothing dropped: in place
    m0 = np.zeros(40, np.uint8); m0[5:9] = 1
    c.drop(Hn.mask_tensor(c, [m0, None, None]))
    oc.drop(0, m0)
    c.drop_reposition(Hn.mask_tensor(c, [np.zeros(36, np.uint8), None, None]))
    for b in range(3):
        oc.drop_reposition(b, np.zeros(len(oc.seqs[b]), np.uint8))
    assert c.sync_status() == 0
    check_meta(c, oc)
    check_kv(c, oc, k_ulp=1)
    assert int(c.next_pos[1]) == 0                                   # empty after repos
    # refill the emptied sequence and decode everything
    k = W.randn_bf16((2, 5, 2, 128), 42)
    v = W.randn_bf16((2, 5, 2, 128), 43)
    tid = np.arange(5) + (1 << 27)
    c.append(torch.tensor([0, 5, 0], dtype=torch.int32, device=c.device), 5, k.to(c.device),
             v.to(c.device), torch.tensor(tid, dtype=torch.int32, device=c.device))
    oc.append(1, tid, k.permute(1, 0, 2, 3).double().numpy(), v.permute(1, 0, 2, 3).double().numpy())
    assert c.sync_status() == 0
    check_meta(c, oc)
    q = q_tensor(sh, 3, 2, 44).to(c.device)
    out = _decode(c, q)
    check_attention(c, oc, q, out)
    assert not out[2].float().abs().sum().item()                     # empty sequence -> 0


def test_active_len_out_of_range_is_latched():
    sh = W.Shape(1, 2, 64, 4, 1.0e4)
    lens = [50, 20]
    say("case active_len out of range")
    c = _setup(sh, lens, seed=51)
    oc = oracle_for(sh, lens, 51)
    q = q_tensor(sh, 2, 1, 52).to(c.device)
    out = _decode(c, q, [60, 20])          # 60 > 50: clamped to 50, error latched
    assert c.sync_status() == 1
    check_attention(c, oc, q, out, active=[50, 20])
    out = _decode(c, q, [-3, 20])          # negative: clamped to 0
    assert c.sync_status() == 1
    assert not out[0].float().abs().sum().item()


def test_graph_capture_replays_match_eager():
    """One step (state restore, fused drop+reposition, decode) captured in a
    HIP graph and replayed several times with eager work and host syncs in
    between; every replay must equal the eager step bit for bit."""
    sh = W.Shape(4, 8, 128, 32, 5.0e5)
    lens = [3000, 1777]
    rng = np.random.default_rng(61)
    masks = [(rng.uniform(size=n) < 0.3).astype(np.uint8) for n in lens]
    say("case graph capture")
    c = _setup(sh, lens, seed=61)
    mask = Hn.mask_tensor(c, masks)
    q = q_tensor(sh, 2, 4, 62).to(c.device)
    out = torch.empty_like(q)
    ws = torch.empty(max(256, c.decode_workspace_bytes(4, 32)), dtype=torch.uint8, device=c.device)
    snap = c.meta.clone()

    def step():
        c.meta.copy_(snap)
        c.drop_reposition(mask)
        c.decode_attention(q, out, ws)

    step()
    torch.cuda.synchronize()
    assert c.sync_status() == 0
    ref_meta = c.meta.clone()
    ref_out = out.clone()
    ref_k = [c.gather_rows(b, l, "k").clone() for b in range(2) for l in range(4)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                              # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.zero_()
        junk = torch.randn(1 << 20, device=c.device).sum()      # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.meta, ref_meta), rep
        assert torch.equal(out, ref_out), rep
        got_k = [c.gather_rows(b, l, "k") for b in range(2) for l in range(4)]
        assert all(torch.equal(x, y) for x, y in zip(got_k, ref_k)), rep
        del junk
    assert c.sync_status() == 0
