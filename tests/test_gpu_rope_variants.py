"""GPU parity of the RoPE variants against the fp64 oracle, through the C ABI:
partial RoPE (the rest of K copied bit for bit), caller frequency tables
(Llama 3.1 and YaRN schedules), sliding-window read ranges across position
gaps in decode and segment attention.

Bars: token ids / positions / lengths / next_pos bit-exact; K within one bf16
step per rotation and its non-rotary tail bit-exact; V bit-exact; attention
within 1e-2 max abs error.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from agent_kv_cache_amd import harness as Hn  # noqa: E402
from agent_kv_cache_amd import workloads as W  # noqa: E402
from oracle import akv_oracle as O  # noqa: E402

from gpu_util import (append_seeded, bits, check_attention, check_kv, check_meta,  # noqa: E402
                      check_segments, oracle_for, run_segments, say, snapshot)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from agent_kv_cache_amd.binding import lib
    lib()


def _decode(cache, q, active=None):
    out = torch.empty_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(q.shape[1], q.shape[2])),
                     dtype=torch.uint8, device=cache.device)
    act = None if active is None else torch.tensor(active, dtype=torch.int32, device=cache.device)
    cache.decode_attention(q, out, ws, active_len=act)
    return out


def _check_tail(cache, oc, r):
    """The non-rotary dims [r, d) of every key equal the oracle's bit for bit."""
    for b, s in enumerate(oc.seqs):
        for l in range(cache.L):
            got = bits(cache.gather_rows(b, l, "k"))[..., r:]
            want = O.bf16_bits(s.k[:, l])[..., r:]
            assert np.array_equal(got, want), (b, l)


# ---------------------------------------------------------------------------
# partial RoPE
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d,r", [(128, 64), (128, 16), (64, 32), (64, 48)])
def test_partial_rope_op_chain(d, r):
    rng = np.random.default_rng(d + r)
    sh = W.Shape(2, 2, d, 8, 1.0e4)
    lens = [0, 5, 40, 130, 300]
    B = len(lens)
    say(f"case partial rope d={d} r={r}")
    cache = Hn.make_cache(sh, lens, 80, max_blocks_per_seq=32, rotary_dim=r)
    cache.reset(np.random.default_rng(r).permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, sh, lens, 11, gen_device="cpu")
    oc = oracle_for(sh, lens, 11, rotary_dim=r)
    for step, kind in enumerate(["drop_repos", "repos_shift", "drop", "drop_repos_explicit"]):
        masks = [(rng.uniform(size=len(oc.seqs[b])) < 0.3).astype(np.uint8) for b in range(B)]
        say(" step", kind)
        if kind == "drop_repos":
            cache.drop_reposition(Hn.mask_tensor(cache, masks))
            for b in range(B):
                oc.drop_reposition(b, masks[b])
        elif kind == "repos_shift":                # every entry moves: in-place rotation
            old = [oc.seqs[b].pos.copy() for b in range(B)]
            new = [p + 1000 for p in old]
            cache.reposition(Hn.pos_tensor(cache, old), Hn.pos_tensor(cache, new))
            for b in range(B):
                oc.reposition(b, new[b])
        elif kind == "drop":
            cache.drop(Hn.mask_tensor(cache, masks))
            for b in range(B):
                oc.drop(b, masks[b])
        else:
            newp = []
            for b in range(B):
                rr = len(oc.seqs[b]) - int(masks[b].sum())
                newp.append(np.cumsum(rng.integers(1, 4, size=rr)) + 3)
            cache.drop_reposition(Hn.mask_tensor(cache, masks), Hn.pos_tensor(cache, newp))
            for b in range(B):
                oc.drop_reposition(b, masks[b], newp[b])
        assert cache.sync_status() == 0
        check_meta(cache, oc)
        check_kv(cache, oc, k_ulp=step + 1)
        _check_tail(cache, oc, r)
    q = W.randn_bf16((B, sh.n_layers, sh.n_q_heads, d), 21).to(cache.device)
    check_attention(cache, oc, q, _decode(cache, q))


def test_partial_rope_fork():
    sh = W.Shape(2, 2, 128, 8, 1.0e4)
    lens = [500, 0]
    cache = Hn.make_cache(sh, lens, 40, rotary_dim=64)
    cache.reset()
    Hn.fill(cache, sh, lens, 12, gen_device="cpu")
    oc = oracle_for(sh, lens, 12, rotary_dim=64)
    say("case partial rope fork")
    src = snapshot(cache, 0)
    m = np.zeros(500, np.uint8); m[100:260] = 1
    cache.fork([1, -1], Hn.mask_tensor(cache, [m]), reposition=True)
    oc.fork(0, 1, m, reposition=True)
    assert cache.sync_status() == 0
    check_meta(cache, oc)
    check_kv(cache, oc, k_ulp=1)
    _check_tail(cache, oc, 64)
    now = snapshot(cache, 0)
    for x, y in zip(src[3] + src[4], now[3] + now[4]):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# caller frequency tables
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("which", ["llama3", "yarn"])
def test_frequency_tables(which):
    if which == "llama3":           # Llama 3.1 8B: d 128, base 5e5, factor 8, low 1, high 4, 8192
        sh = W.Shape(2, 2, 128, 8, 5.0e5)
        th = O.llama3_theta(O.rope_theta(128, 5.0e5), 8.0, 1.0, 4.0, 8192)
    else:                           # GPT-OSS-like: d 64, base 1.5e5, factor 32, original 4096
        sh = W.Shape(2, 2, 64, 16, 1.5e5)
        th = O.yarn_theta(64, 1.5e5, 32.0, 4096)
    lens = [3000, 777]
    rng = np.random.default_rng(3)
    masks = [(rng.uniform(size=n) < 0.4).astype(np.uint8) for n in lens]
    say(f"case frequency table {which}")
    cache = Hn.make_cache(sh, lens, sum(Hn.pages_for(n) for n in lens), inv_freq=th)
    cache.reset()
    Hn.fill(cache, sh, lens, 13, gen_device="cpu")
    oc = oracle_for(sh, lens, 13, theta=th)
    cache.drop_reposition(Hn.mask_tensor(cache, masks))
    for b in range(2):
        oc.drop_reposition(b, masks[b])
    assert cache.sync_status() == 0
    check_meta(cache, oc)
    worst = check_kv(cache, oc, k_ulp=1)
    say(" worst K ulp", worst)
    # plain base^(-2i/d) frequencies give different keys: the table is used
    plain = oracle_for(sh, lens, 13)
    for b in range(2):
        plain.drop_reposition(b, masks[b])
    assert not np.array_equal(O.bf16_bits(plain.seqs[0].k), O.bf16_bits(oc.seqs[0].k))


# ---------------------------------------------------------------------------
# sliding windows
# ---------------------------------------------------------------------------
def _gapped(window, d=128, G=4, lens=(0, 3, 40, 333, 1500), seed=14):
    sh = W.Shape(len(window), 2, d, 2 * G, 1.0e4)
    rng = np.random.default_rng(seed)
    cache = Hn.make_cache(sh, lens, sum(Hn.pages_for(n) for n in lens), layer_window=window)
    cache.reset(np.random.default_rng(seed).permutation(cache.NB).astype(np.int32))
    Hn.fill(cache, sh, lens, seed, gen_device="cpu")
    oc = oracle_for(sh, lens, seed, window=window)
    # drop without reposition: positions keep gaps
    masks = [(rng.uniform(size=n) < 0.5).astype(np.uint8) for n in lens]
    cache.drop(Hn.mask_tensor(cache, masks))
    for b in range(len(lens)):
        oc.drop(b, masks[b])
    assert cache.sync_status() == 0
    check_meta(cache, oc)
    return sh, cache, oc, rng


@pytest.mark.parametrize("d", [64, 128])
def test_window_decode_across_gaps(d):
    window = [0, 1, 7, 64, 300, 5000]
    say(f"case window decode d={d}")
    sh, cache, oc, rng = _gapped(window, d=d)
    B = len(oc.seqs)
    q = W.randn_bf16((B, sh.n_layers, sh.n_q_heads, d), 15).to(cache.device)
    err = check_attention(cache, oc, q, _decode(cache, q))
    act = [int(rng.integers(0, len(s) + 1)) for s in oc.seqs]
    check_attention(cache, oc, q, _decode(cache, q, act), active=act)
    say(" window decode max abs err", err)


@pytest.mark.parametrize("G", [1, 4, 16])
def test_window_segments_across_gaps(G):
    window = [0, 3, 50, 700]
    say(f"case window segments G={G}")
    sh, cache, oc, rng = _gapped(window, G=G)
    tb = 16 // G
    lens = [len(s) for s in oc.seqs]
    # long segments (prefill kernel), then segments of at most 16/G rows (split kernel)
    long_segs = [(b, min(lens[b], n)) for b, n in ((1, 2), (2, 19), (3, 150), (4, 700), (4, 1))]
    short_segs = [(b, min(lens[b], int(rng.integers(0, tb + 1)))) for b in range(1, 5)]
    for segs, mq in ((long_segs, None), (short_segs, tb)):
        nq = max(1, sum(n for _, n in segs))
        q = W.randn_bf16((nq, sh.n_layers, sh.n_q_heads, sh.head_dim), 16 + G).to(cache.device)
        out = run_segments(cache, q, segs, max_q=mq)
        assert cache.sync_status() == 0
        err = check_segments(oc, q, out, segs)
        say(" segments max abs err", err, "max_q", mq)


def test_window_with_partial_rope_after_reposition():
    """Windows and partial RoPE together, positions compacted by a reposition
    and then appended to, decode and segments."""
    window = [0, 32]
    sh = W.Shape(2, 2, 128, 8, 1.0e4)
    lens = [200, 900]
    cache = Hn.make_cache(sh, lens, 40, rotary_dim=32, layer_window=window)
    cache.reset()
    Hn.fill(cache, sh, lens, 17, gen_device="cpu")
    oc = oracle_for(sh, lens, 17, rotary_dim=32, window=window)
    say("case window + partial rope")
    rng = np.random.default_rng(17)
    masks = [(rng.uniform(size=n) < 0.6).astype(np.uint8) for n in lens]
    cache.drop_reposition(Hn.mask_tensor(cache, masks))
    for b in range(2):
        oc.drop_reposition(b, masks[b])
    append_seeded(cache, oc, sh, [10, 70], 18, 1 << 27)
    assert cache.sync_status() == 0
    check_kv(cache, oc, k_ulp=1)
    q = W.randn_bf16((2, 2, 8, 128), 19).to(cache.device)
    check_attention(cache, oc, q, _decode(cache, q))
    segs = [(0, 10), (1, 70)]
    qs = W.randn_bf16((80, 2, 8, 128), 20).to(cache.device)
    out = run_segments(cache, qs, segs)
    assert cache.sync_status() == 0
    check_segments(oc, qs, out, segs)


# ---------------------------------------------------------------------------
# the benchmark's variant runs at full size (Llama-8B shape, 32768 tokens)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["rotary64", "llama3", "window128"])
def test_variants_full_size_sampled(variant):
    """The Llama-8B-shaped drop + reposition and decode as the benchmark runs
    it with partial RoPE (r = 64), the Llama 3.1 frequency table, or
    128-token windows on every other layer; lengths, positions and ids
    everywhere, K / V and attention on sampled layers (a windowed and two
    full layers) against the oracle."""
    wl = W.llama8b_32k()
    sh = wl.shape
    kw, okw = {}, {}
    if variant == "rotary64":
        kw["rotary_dim"] = okw["rotary_dim"] = 64
    elif variant == "llama3":
        th = O.llama3_theta(O.rope_theta(sh.head_dim, sh.rope_base), 8.0, 1.0, 4.0, 8192)
        kw["inv_freq"] = okw["theta"] = th
    else:
        win = [128 if l % 2 == 0 else 0 for l in range(sh.n_layers)]
        kw["layer_window"] = okw["window"] = win
    layers = [0, 17, 30]
    say(f"case variant {variant} full size")
    extra = Hn.moved_pages(wl.seq_lens[0], wl.masks[0])
    cache = Hn.make_cache(sh, wl.seq_lens, extra, **kw)
    cache.reset()
    Hn.fill(cache, sh, wl.seq_lens, wl.data_seed, gen_device="cuda")
    oc = oracle_for(sh, wl.seq_lens, wl.data_seed, layers=layers, gen_device="cuda", **okw)
    cache.drop_reposition(Hn.mask_tensor(cache, wl.masks))
    assert cache.sync_status() == 0
    oc.drop_reposition(0, wl.masks[0])
    check_meta(cache, oc)
    worst = check_kv(cache, oc, layers=layers, k_ulp=1)
    say(" worst K ulp on sampled layers", worst)
    q = W.randn_bf16((1, sh.n_layers, sh.n_q_heads, sh.head_dim), 202, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(256, cache.decode_workspace_bytes(sh.n_layers, sh.n_q_heads)),
                     dtype=torch.uint8, device=cache.device)
    cache.decode_attention(q, out, ws)
    assert cache.sync_status() == 0
    check_attention(cache, oc, q, out, layers=layers, what=f"{variant} attention")
