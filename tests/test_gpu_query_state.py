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
    assert lib().akv_query_state(cache.handle, lens.data_ptr(), None, None, None, stream) == 0
    assert int(lens[0]) == 40
    assert lib().akv_query_state(cache.handle, None, None, None, None, stream) == 0
    assert lib().akv_query_state(None, lens.data_ptr(), None, None, None, stream) != 0
