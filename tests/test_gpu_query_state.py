"""akv_query_state through the C ABI: lengths, next positions and every
sequence's positions / token ids in active order, against the oracle after a
fused drop + reposition and against plain reads of the caller-owned tables."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from agent_kv_cache_amd import harness as Hn  # noqa: E402
from agent_kv_cache_amd import workloads as W  # noqa: E402

from gpu_util import oracle_for, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from agent_kv_cache_amd.binding import lib
    lib()


def test_query_state_matches_oracle_and_tables():
    sh = W.Shape(1, 2, 64, 4, 1e4)
    lens = [300, 0, 77, 1000]
    cache = Hn.make_cache(sh, lens, 80)
    cache.reset(np.random.default_rng(5).permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, sh, lens, 80, gen_device="cpu")
    oc = oracle_for(sh, lens, 80, with_kv=False)
    masks = [W.spans_to_mask(300, [(10, 50)]), None, np.zeros(77, np.uint8),
             W.spans_to_mask(1000, [(0, 1), (500, 333)])]
    say("case query_state after drop+reposition, 4 sequences, shuffled pages")
    cache.drop_reposition(Hn.mask_tensor(cache, masks))
    assert cache.sync_status() == 0
    for b, m in enumerate(masks):
        if m is not None:
            oc.drop_reposition(b, m)
    ln, nx, pos, tok = (t.cpu().numpy() for t in cache.query_state())
    for b in range(len(lens)):
        s = oc.seqs[b]
        n = len(s)
        assert ln[b] == n and nx[b] == s.next_pos
        assert np.array_equal(pos[b, :n], s.pos) and np.array_equal(tok[b, :n], s.token_ids)
        assert (pos[b, n:] == -1).all() and (tok[b, n:] == -1).all()
        # the same entries read straight from the caller-owned page table
        pages = cache.block_table[b, :Hn.pages_for(n)].long()
        assert np.array_equal(cache.positions[pages].reshape(-1)[:n].cpu().numpy(), pos[b, :n])
        assert np.array_equal(cache.token_ids[pages].reshape(-1)[:n].cpu().numpy(), tok[b, :n])
    assert np.array_equal(ln, cache.seq_lens.cpu().numpy())
    assert np.array_equal(nx, cache.next_pos.cpu().numpy())


def test_query_state_optional_outputs():
    from agent_kv_cache_amd.binding import lib
    sh = W.Shape(1, 1, 64, 2, 1e4)
    cache = Hn.make_cache(sh, [40], 8)
    cache.reset()
    Hn.fill(cache, sh, [40], 81, gen_device="cpu")
    say("case query_state with only the lengths requested")
    lens = torch.full((1,), -7, dtype=torch.int32, device=cache.device)
    stream = torch.cuda.current_stream().cuda_stream
    assert lib().akv_query_state(cache.handle, lens.data_ptr(), None, None, None, None,
                                 stream) == 0
    assert int(lens[0]) == 40
    assert lib().akv_query_state(cache.handle, None, None, None, None, None, stream) == 0
    assert lib().akv_query_state(None, lens.data_ptr(), None, None, None, None, stream) != 0


def _rows(cache):
    return cache.query_state(with_last_src=True)[4].cpu().numpy()


def test_last_src_is_the_oracle_gather_map():
    """last_src after drop / drop+reposition / reposition / fork against the
    oracle's src (the pre-op index of each survivor), bit for bit; -1 before
    any such call, unchanged by appends, -1 after a rejected call."""
    sh = W.Shape(1, 2, 64, 4, 1e4)
    lens = [300, 0, 77, 1000, 0]
    cache = Hn.make_cache(sh, lens, 200)
    cache.reset(np.random.default_rng(6).permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, sh, lens, 82, gen_device="cpu")
    oc = oracle_for(sh, lens, 82, with_kv=False)
    say("case last_src before any op")
    assert (_rows(cache) == -1).all()
    masks = [W.spans_to_mask(300, [(10, 50), (299, 1)]), None, np.zeros(77, np.uint8),
             W.spans_to_mask(1000, [(0, 1), (500, 333)]), None]
    say("case last_src after drop+reposition")
    cache.drop_reposition(Hn.mask_tensor(cache, masks))
    assert cache.sync_status() == 0
    rows = _rows(cache)
    for b, m in enumerate(masks):
        src = oc.drop_reposition(b, m if m is not None else np.zeros(lens[b], np.uint8))[0]
        n = len(src)
        assert np.array_equal(rows[b, :n], src), b
        assert (rows[b, n:] == -1).all()
    say("case last_src unchanged by an append")
    cnt = torch.tensor([5, 0, 0, 3, 0], dtype=torch.int32, device=cache.device)
    kk = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16, device=cache.device)
    cache.append(cnt, 8, kk, kk, torch.arange(8, dtype=torch.int32, device=cache.device) + 7000)
    assert cache.sync_status() == 0
    assert np.array_equal(_rows(cache), rows)
    oc.append(0, np.arange(5) + 7000)
    oc.append(3, np.arange(5, 8) + 7000)
    say("case last_src after a drop (no reposition)")
    m3 = np.zeros(len(oc.seqs[3]), np.uint8)
    m3[[3, 4, 5, len(m3) - 1]] = 1
    mk = [None, None, None, m3, None]
    cache.drop(Hn.mask_tensor(cache, mk))
    assert cache.sync_status() == 0
    rows = _rows(cache)
    for b in range(len(lens)):
        m = mk[b] if mk[b] is not None else np.zeros(len(oc.seqs[b]), np.uint8)
        src = oc.drop(b, m)
        assert np.array_equal(rows[b, :len(src)], src) and (rows[b, len(src):] == -1).all(), b
    say("case last_src after a reposition (identity map)")
    cache.reposition()
    assert cache.sync_status() == 0
    rows = _rows(cache)
    for b in range(len(lens)):
        n = len(oc.seqs[b])
        assert np.array_equal(rows[b, :n], np.arange(n)) and (rows[b, n:] == -1).all()
    say("case last_src after a fork: the destination row indexes its source")
    fm = np.zeros(len(oc.seqs[3]), np.uint8)
    fm[100:250] = 1
    cache.fork([-1, -1, -1, 1, -1], Hn.mask_tensor(cache, [None, None, None, fm, None]),
               reposition=True)
    assert cache.sync_status() == 0
    rows = _rows(cache)
    ref = oracle_for(sh, [0, 0, 0, len(oc.seqs[3])], 1, with_kv=False)
    ref.seqs[3].token_ids = oc.seqs[3].token_ids.copy()
    src = ref.drop(3, fm)
    assert np.array_equal(rows[1, :len(src)], src) and (rows[1, len(src):] == -1).all()
    for b in (0, 2, 3, 4):
        assert (rows[b] == -1).all(), b
    say("case last_src after a rejected call")
    bad = [np.array([0, 0])] + [None] * 4
    cache.reposition(None, Hn.pos_tensor(cache, [np.r_[np.arange(5), np.arange(len(oc.seqs[0]) - 5)]]
                                           + [None] * 4))
    assert cache.sync_status() == 2
    assert (_rows(cache) == -1).all()
    del bad
