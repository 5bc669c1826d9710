"""akv_decode_attention_noalloc (the decode for callers that cannot allocate)
against akv_decode_attention with a caller workspace, through the C ABI:
bit-identical outputs on two calls in a row, the second one smaller; the
split-K path (which uses the static per-GPU array) and the single-split path
(which does not); the size limit is rejected on the host."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from agent_kv_cache_amd import harness as Hn  # noqa: E402
from agent_kv_cache_amd import workloads as W  # noqa: E402
from agent_kv_cache_amd.binding import AkvError, lib  # noqa: E402

from gpu_util import check_attention, oracle_for, say  # noqa: E402

LIMIT = 8 << 20      # AKV_NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib()


def _both(cache, q, active=None, layer_begin=0, n_layers=None):
    nL = q.shape[1]
    ref = torch.full_like(q, float("nan"))
    ws = torch.empty(max(256, cache.decode_workspace_bytes(nL, q.shape[2])), dtype=torch.uint8,
                     device=cache.device)
    cache.decode_attention(q, ref, ws, active_len=active, layer_begin=layer_begin,
                           n_layers=n_layers)
    got = torch.full_like(q, float("nan"))
    cache.decode_attention_noalloc(q, got, active_len=active, layer_begin=layer_begin,
                                   n_layers=n_layers)
    assert cache.sync_status() == 0
    return ref, got


def _bitwise(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_noalloc_matches_workspace_decode_two_calls():
    sh = W.Shape(2, 8, 128, 32, 1.0e4)
    lens = [1500]
    cache = Hn.make_cache(sh, lens, 8, max_blocks_per_seq=128)
    cache.reset()
    Hn.fill(cache, sh, lens, 31, gen_device="cpu")
    ns_bytes = cache.decode_workspace_bytes(2, sh.n_q_heads)
    assert 256 < ns_bytes <= LIMIT, ns_bytes           # split-K: the static array is used
    dev = cache.device
    # call 1: both layers, the whole sequence
    q1 = W.randn_bf16((1, 2, sh.n_q_heads, sh.head_dim), 32).to(dev)
    ref1, got1 = _both(cache, q1)
    assert _bitwise(ref1, got1)
    oc = oracle_for(sh, lens, 31)
    err1 = check_attention(cache, oc, q1, got1)
    # call 2, smaller: one layer, a shorter active length
    q2 = W.randn_bf16((1, 1, sh.n_q_heads, sh.head_dim), 33).to(dev)
    act = torch.tensor([611], dtype=torch.int32, device=dev)
    ref2, got2 = _both(cache, q2, active=act, layer_begin=1, n_layers=1)
    assert _bitwise(ref2, got2)
    err2 = check_attention(cache, oracle_for(sh, lens, 31, layers=[1]), q2, got2, active=[611])
    say(f"noalloc: bitwise equal to the workspace decode on both calls; "
        f"max |got - oracle| {err1:.2e} / {err2:.2e}")


def test_noalloc_single_split_batch():
    sh = W.Shape(4, 8, 64, 64, 1.5e5)      # 64 sequences x 4 layers x 8 kv heads: one split
    lens = [int(x) for x in np.random.default_rng(5).integers(1, 90, size=64)]
    cache = Hn.make_cache(sh, lens, 8)
    cache.reset()
    Hn.fill(cache, sh, lens, 41, gen_device="cpu")
    assert cache.decode_workspace_bytes(4, sh.n_q_heads) == 256    # one split: no partials
    q = W.randn_bf16((64, 4, sh.n_q_heads, sh.head_dim), 42).to(cache.device)
    ref, got = _both(cache, q)
    assert _bitwise(ref, got)


def test_noalloc_rejects_calls_beyond_the_limit():
    # 19 sequences x 9 layers x 1 kv head = 171 rows and 16 query heads per
    # kv head: with 256 (or 512) resident decode workgroups the fullest last
    # round takes 7 (11) splits, 171 x 7 x 16 split records of 130 floats
    # = 9.96 MB (15.6 MB) > 8 MiB
    sh = W.Shape(9, 1, 128, 16, 1.0e4)
    lens = [40] * 19
    cache = Hn.make_cache(sh, lens, 8, max_blocks_per_seq=48)
    cache.reset()
    Hn.fill(cache, sh, lens, 51, gen_device="cpu")
    need = cache.decode_workspace_bytes(9, 16)
    say(f"noalloc limit case: the workspace decode needs {need} bytes (limit {LIMIT})")
    q = W.randn_bf16((19, 9, 16, 128), 52).to(cache.device)
    out = torch.zeros_like(q)
    if need <= LIMIT:
        pytest.skip(f"this GPU's split count needs only {need} bytes")
    with pytest.raises(AkvError) as e:
        cache.decode_attention_noalloc(q, out)
    assert e.value.code == 7
    assert cache.sync_status() == 0
    assert not out.view(torch.int16).any()            # nothing was launched
    q3 = q[:, 8:9].contiguous()
    ref, got = _both(cache, q3, layer_begin=8, n_layers=1)   # a smaller call still runs
    assert _bitwise(ref, got)
