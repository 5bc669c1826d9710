"""Pins of the oracle's RoPE variants: partial RoPE, caller frequency tables
(Llama 3.1 and YaRN rules), sliding-window read ranges.

[AKV] section 5.5: the rest of K that RoPE does not rotate is copied like V;
the model binding tells partial RoPE and sliding-window layers apart; with a
sliding window each query's read range follows positions, which have gaps
after a drop without reposition.  The Llama 3.1 and YaRN frequency rules are
not on the pages; they are pinned here by closed forms and limits of their
published definitions.
"""
import math

import numpy as np
import pytest

from oracle import akv_oracle as O


def _bits_equal(a, b):
    return np.array_equal(np.asarray(a).view(np.int64), np.asarray(b).view(np.int64))


# ---------------------------------------------------------------------------
# partial RoPE
# ---------------------------------------------------------------------------
def test_rotary_dim_equal_to_head_dim_is_full_rope():
    for d, base in ((64, 1e4), (128, 5e5)):
        assert _bits_equal(O.rope_theta(d, base, d), O.rope_theta(d, base))
    k = np.random.default_rng(0).standard_normal((5, 128))
    th = O.rope_theta(128, 5e5)
    assert _bits_equal(O.rotate_pairs(k, np.arange(5) * 7, th),
                       O.rotate_pairs(k, np.arange(5) * 7, O.rope_theta(128, 5e5, 128)))


def test_partial_rope_unit_vectors_pin_pairing_and_frequencies():
    d, r, base, delta = 16, 8, 1e4, 3
    th = O.rope_theta(d, base, r)
    assert th.shape == (r // 2,)
    assert th[1] == pytest.approx(0.1, rel=1e-15)        # 1e4^(-2/8): frequencies over r, not d
    e = np.eye(d)
    out = O.rotate_pairs(e, delta, th)
    # e_0 -> (cos 3, sin 3) at dims 0 and r/2 = 4
    assert out[0, 0] == pytest.approx(math.cos(3.0)) and out[0, 4] == pytest.approx(math.sin(3.0))
    assert np.count_nonzero(out[0]) == 2
    # e_4 -> (-sin 3, cos 3)
    assert out[4, 0] == pytest.approx(-math.sin(3.0)) and out[4, 4] == pytest.approx(math.cos(3.0))
    # e_1 turns by 3 * 0.1
    assert out[1, 1] == pytest.approx(math.cos(0.3)) and out[1, 5] == pytest.approx(math.sin(0.3))
    # the non-rotary dimensions are copied bit for bit (the zero rotary part
    # of such a vector may come back as -0)
    for j in range(r, d):
        assert _bits_equal(out[j, r:], e[j, r:]) and not out[j, :r].any()


def test_partial_rope_is_full_rope_on_the_rotary_slice():
    rng = np.random.default_rng(1)
    d, r, base = 128, 64, 5e5
    k = O.bf16_round(rng.standard_normal((9, 2, 3, d)))
    delta = rng.integers(-5000, 5000, size=9).reshape(9, 1, 1)
    got = O.rotate_pairs(k, delta, O.rope_theta(d, base, r))
    assert _bits_equal(got[..., :r], O.rotate_pairs(k[..., :r], delta, O.rope_theta(r, base)))
    assert _bits_equal(got[..., r:], k[..., r:])


def test_partial_rope_relative_position_law():
    rng = np.random.default_rng(2)
    d, r = 128, 32
    th = O.rope_theta(d, 1e4, r)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for a, b, s in ((3, 11, 5), (100, 7, -40), (0, 0, 12345)):
        lhs = O.rotate_pairs(q, a + s, th) @ O.rotate_pairs(k, b + s, th)
        rhs = O.rotate_pairs(q, a, th) @ O.rotate_pairs(k, b, th)
        assert lhs == pytest.approx(rhs, abs=1e-11)


def test_partial_rerotate_identity_tail_and_round_trip():
    rng = np.random.default_rng(3)
    d, r = 64, 16
    th = O.rope_theta(d, 1.5e5, r)
    k = O.bf16_round(rng.standard_normal((40, 1, 2, d)))
    assert _bits_equal(O.rerotate_keys(k, np.zeros(40, np.int64), th), k)
    delta = rng.integers(-3000, 3000, size=40)
    k1 = O.rerotate_keys(k, delta, th)
    assert _bits_equal(k1[..., r:], k[..., r:])           # tail copied bit for bit
    back = O.rerotate_keys(k1, -delta, th)
    pair_norm = np.sqrt(k[..., :r // 2] ** 2 + k[..., r // 2:r] ** 2)
    err = np.abs(back[..., :r] - k[..., :r])
    bound = 2.0 ** -7 * np.concatenate([pair_norm, pair_norm], axis=-1) + 1e-30
    assert np.all(err <= bound)


def test_partial_rope_cache_reposition_moves_only_the_rotary_part():
    rng = np.random.default_rng(4)
    d, r = 64, 32
    c = O.OracleCache(2, 2, d, 1e4, rotary_dim=r)
    k = O.bf16_round(rng.standard_normal((30, 2, 2, d)))
    v = O.bf16_round(rng.standard_normal((30, 2, 2, d)))
    c.append(0, np.arange(30), k, v)
    m = np.zeros(30, np.uint8); m[4:12] = 1
    c.drop_reposition(0, m)
    keep = np.flatnonzero(m == 0)
    s = c.seqs[0]
    assert _bits_equal(s.k[..., r:], k[keep][..., r:])
    assert _bits_equal(s.v, v[keep])
    ref = O.bf16_round(O.rotate_pairs(k[keep], (np.arange(22) - keep).reshape(22, 1, 1),
                                      O.rope_theta(d, 1e4, r)))
    assert _bits_equal(s.k[..., :r], ref[..., :r])


# ---------------------------------------------------------------------------
# frequency tables: Llama 3.1 rule
# ---------------------------------------------------------------------------
def test_llama3_rule_factor_one_is_identity():
    th = O.rope_theta(128, 5e5)
    for lo, hi in ((1.0, 4.0), (2.0, 8.0)):
        assert np.allclose(O.llama3_theta(th, 1.0, lo, hi, 8192), th, rtol=1e-15, atol=0)


def test_llama3_rule_bands_closed_form():
    """Llama 3.1 8B settings: factor 8, low 1, high 4, original 8192, base
    5e5, d 128.  Pair i has wavelength 2 pi base^(2i/d); it is kept while that
    is below 8192/4 and divided by 8 once it is above 8192/1."""
    d, base, C = 128, 5e5, 8192
    th = O.rope_theta(d, base)
    new = O.llama3_theta(th, 8.0, 1.0, 4.0, C)
    i_keep = (d / 2) * math.log(C / (2 * math.pi * 4.0)) / math.log(base)   # ~28.2
    i_scale = (d / 2) * math.log(C / (2 * math.pi * 1.0)) / math.log(base)  # ~35.0
    i = np.arange(d // 2)
    kept, scaled = i < i_keep, i > i_scale
    assert kept.sum() == 29 and scaled.sum() == 29
    assert np.array_equal(new[kept], th[kept])
    assert np.allclose(new[scaled], th[scaled] / 8.0, rtol=1e-15, atol=0)
    mid = ~kept & ~scaled
    assert np.all((new[mid] > th[mid] / 8.0) & (new[mid] < th[mid]))
    assert np.all(np.diff(new) < 0)                       # still strictly decreasing


def test_llama3_rule_is_continuous_at_both_band_edges():
    C, lo, hi, f = 8192, 1.0, 4.0, 8.0
    for w_edge in (C / hi, C / lo):
        t = 2 * math.pi / w_edge
        a = O.llama3_theta(np.array([t * (1 - 1e-9)]), f, lo, hi, C)[0]
        b = O.llama3_theta(np.array([t * (1 + 1e-9)]), f, lo, hi, C)[0]
        assert a == pytest.approx(b, rel=1e-7)


# ---------------------------------------------------------------------------
# frequency tables: YaRN
# ---------------------------------------------------------------------------
def test_yarn_factor_one_is_identity():
    th = O.rope_theta(64, 1.5e5)
    assert np.allclose(O.yarn_theta(64, 1.5e5, 1.0, 4096), th, rtol=1e-15, atol=0)


def _pair_with_turns(turns, r, base, C):
    """Real pair index whose frequency turns `turns` times over C positions,
    found by bisection on the turn count (independent of the closed form)."""
    lo, hi = 0.0, r / 2.0
    f = lambda i: C * base ** (-2.0 * i / r) / (2 * math.pi) - turns
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if f(mid) > 0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


@pytest.mark.parametrize("r,base,factor,C", [(64, 1.5e5, 32.0, 4096), (128, 1e4, 4.0, 4096)])
def test_yarn_ramp_ends_follow_the_turn_counts(r, base, factor, C):
    th = O.rope_theta(r, base)
    new = O.yarn_theta(r, base, factor, C, beta_fast=32.0, beta_slow=1.0)
    i_fast = _pair_with_turns(32.0, r, base, C)
    i_slow = _pair_with_turns(1.0, r, base, C)
    i = np.arange(r // 2)
    keep = i <= math.floor(i_fast)
    interp = i >= math.ceil(i_slow)
    assert keep.any() and interp.any()
    assert np.allclose(new[keep], th[keep], rtol=1e-15, atol=0)
    assert np.allclose(new[interp], th[interp] / factor, rtol=1e-15, atol=0)
    mid = ~keep & ~interp
    assert np.all((new[mid] < th[mid]) & (new[mid] > th[mid] / factor))


def test_cache_with_explicit_frequencies_rotates_by_them():
    rng = np.random.default_rng(5)
    d = 64
    th = O.yarn_theta(d, 1.5e5, 32.0, 4096)
    c = O.OracleCache(1, 1, d, 1.5e5, theta=th)
    k = O.bf16_round(rng.standard_normal((10, 1, 1, d)))
    c.append(0, np.arange(10), k, k)
    c.reposition(0, np.arange(10) + 1000)
    want = O.bf16_round(O.rotate_pairs(k, np.full((10, 1, 1), 1000), th))
    assert _bits_equal(c.seqs[0].k, want)
    with pytest.raises(ValueError):
        O.OracleCache(1, 1, d, 1e4, theta=th[:-1])


# ---------------------------------------------------------------------------
# sliding window read ranges
# ---------------------------------------------------------------------------
def _gapped_cache(window):
    rng = np.random.default_rng(6)
    c = O.OracleCache(2, 1, 16, 1e4, window=window)
    k = O.bf16_round(rng.standard_normal((20, 2, 1, 16)))
    v = O.bf16_round(rng.standard_normal((20, 2, 1, 16)))
    c.append(0, np.arange(20), k, v)
    keep_pos = [0, 1, 2, 5, 6, 9, 14, 15, 17, 19]
    m = np.ones(20, np.uint8); m[keep_pos] = 0
    c.drop(0, m)                                          # positions keep their gaps
    return c, k[keep_pos], v[keep_pos], rng


def test_window_decode_uses_positions_not_indices():
    c, k, v, rng = _gapped_cache([0, 6])
    s = c.seqs[0]
    assert list(s.pos) == [0, 1, 2, 5, 6, 9, 14, 15, 17, 19] and s.next_pos == 20
    q = O.bf16_round(rng.standard_normal((2, 2, 16)))
    out = c.decode_attention(0, q)
    # layer 0 full; layer 1: window 6 for the query at position 20 -> pos >= 15
    for h in range(2):
        assert np.allclose(out[0, h], O.attend(q[0, h], k[:, 0, 0], v[:, 0, 0]), atol=1e-14)
        assert np.allclose(out[1, h], O.attend(q[1, h], k[7:, 1, 0], v[7:, 1, 0]), atol=1e-14)
    # the last 6 indices would include positions 6, 9, 14: not what a window means
    assert not np.allclose(out[1, 0], O.attend(q[1, 0], k[4:, 1, 0], v[4:, 1, 0]), atol=1e-6)


def test_window_limits():
    c, k, v, rng = _gapped_cache([21, 1])
    q = O.bf16_round(rng.standard_normal((2, 1, 16)))
    out = c.decode_attention(0, q)
    assert np.allclose(out[0, 0], O.attend(q[0, 0], k[:, 0, 0], v[:, 0, 0]), atol=1e-14)
    assert np.array_equal(out[1, 0], np.zeros(16))        # only the query's own position


def test_window_segment_rows_follow_their_own_positions():
    c, k, v, rng = _gapped_cache([0, 4])
    q = O.bf16_round(rng.standard_normal((3, 2, 1, 16)))
    (out,) = O.segment_attention(c, [(0, q)])
    # rows are the entries at positions 15, 17, 19 (indices 7, 8, 9)
    # window 4: pos >= 12 / 14 / 16, up to the row itself
    want_sets = {0: [6, 7], 1: [6, 7, 8], 2: [8, 9]}
    for i in range(3):
        idx = want_sets[i]
        assert np.allclose(out[i, 1, 0], O.attend(q[i, 1, 0], k[idx, 1, 0], v[idx, 1, 0]),
                           atol=1e-14)
        full = list(range(7 + i + 1))
        assert np.allclose(out[i, 0, 0], O.attend(q[i, 0, 0], k[full, 0, 0], v[full, 0, 0]),
                           atol=1e-14)


def test_planted_mistakes_in_variants_are_caught(monkeypatch):
    # a window counted in indices instead of positions
    def by_index(self, b, upto, qpos, layer):
        w = self.window[layer]
        return np.arange(max(0, upto - w + 1) if w else 0, upto)
    monkeypatch.setattr(O.OracleCache, "visible", by_index)
    with pytest.raises(AssertionError):
        test_window_decode_uses_positions_not_indices()
    monkeypatch.undo()
    # partial RoPE paired at d/2 instead of r/2
    orig = O.rotate_pairs

    def wrong_pairing(k, delta, theta):
        k = np.asarray(k, dtype=np.float64)
        half = k.shape[-1] // 2
        th = np.zeros(half); th[:np.asarray(theta).shape[-1]] = theta
        return orig(k, delta, th)
    monkeypatch.setattr(O, "rotate_pairs", wrong_pairing)
    with pytest.raises(AssertionError):
        test_partial_rope_unit_vectors_pin_pairing_and_frequencies()
    monkeypatch.undo()
    # Llama 3.1 bands swapped
    orig3 = O.llama3_theta
    monkeypatch.setattr(O, "llama3_theta", lambda th, f, lo, hi, C: orig3(th, f, hi, lo, C))
    with pytest.raises(AssertionError):
        test_llama3_rule_bands_closed_form()


# ---------------------------------------------------------------------------
# append with the RoPE rotation fused in, release
# ---------------------------------------------------------------------------
def test_append_rotated_unit_vectors_and_position_zero():
    d, r = 16, 8
    c = O.OracleCache(1, 1, d, 1e4, rotary_dim=r)
    e = np.eye(d)
    k_raw = np.stack([e[0], e[4], e[1], e[12]])[:, None, None, :]      # 4 tokens at 0..3
    c.append_rotated(0, np.arange(4), k_raw, k_raw)
    k = c.seqs[0].k[:, 0, 0]
    assert _bits_equal(k[0], e[0])                          # position 0: unchanged
    # e_4 at position 1: pair 0 turns by 1 rad -> (-sin 1, cos 1) at dims 0, 4
    assert k[1, 0] == O.bf16_round(np.array(-math.sin(1.0)))[()]
    assert k[1, 4] == O.bf16_round(np.array(math.cos(1.0)))[()]
    # e_1 at position 2: pair 1 (theta = 0.1) turns by 0.2
    assert k[2, 1] == O.bf16_round(np.array(math.cos(0.2)))[()]
    assert k[2, 5] == O.bf16_round(np.array(math.sin(0.2)))[()]
    assert _bits_equal(k[3, r:], e[12, r:])                  # tail copied at position 3
    assert c.seqs[0].next_pos == 4 and list(c.seqs[0].pos) == [0, 1, 2, 3]


def test_append_rotated_commutes_with_reposition():
    """Keys appended at positions s.. equal keys appended at 0.. and then
    moved by s (two roundings against one: within 2^-7 of the pair norm)."""
    rng = np.random.default_rng(8)
    d, s_shift = 64, 777
    k_raw = O.bf16_round(rng.standard_normal((20, 2, 2, d)))
    v = O.bf16_round(rng.standard_normal((20, 2, 2, d)))
    a = O.OracleCache(2, 2, d, 1.5e5)
    a.append_rotated(0, np.arange(20), k_raw, v)
    a.reposition(0, np.arange(20) + s_shift)
    b = O.OracleCache(2, 2, d, 1.5e5)
    b.append(0, [10 ** 6], np.zeros((1, 2, 2, d)), np.zeros((1, 2, 2, d)))
    b.seqs[0].next_pos = s_shift                            # as after dropping earlier tokens
    b.drop(0, [1])
    b.append_rotated(0, np.arange(20), k_raw, v)
    assert list(b.seqs[0].pos) == list(a.seqs[0].pos)
    half = d // 2
    norm = np.sqrt(k_raw[..., :half] ** 2 + k_raw[..., half:] ** 2)
    bound = 2.0 ** -7 * np.concatenate([norm, norm], axis=-1) + 1e-30
    assert np.all(np.abs(a.seqs[0].k - b.seqs[0].k) <= bound)
    assert _bits_equal(a.seqs[0].v, b.seqs[0].v)


def test_release_empties_and_resets_positions():
    rng = np.random.default_rng(9)
    c = O.OracleCache(1, 1, 16, 1e4, n_seqs=2)
    for b in range(2):
        k = O.bf16_round(rng.standard_normal((5, 1, 1, 16)))
        c.append_rotated(b, np.arange(5), k, k)
    c.release(0)
    assert len(c.seqs[0]) == 0 and c.seqs[0].next_pos == 0
    assert len(c.seqs[1]) == 5 and c.seqs[1].next_pos == 5
    k = O.bf16_round(rng.standard_normal((2, 1, 1, 16)))
    c.append_rotated(0, [7, 8], k, k)
    assert list(c.seqs[0].pos) == [0, 1] and _bits_equal(c.seqs[0].k[0], k[0])


def test_planted_mistakes_in_append_rotated_are_caught(monkeypatch):
    orig = O.OracleCache.append_rotated

    def off_by_one(self, b, token_ids, k_raw, v):
        self.seqs[b].next_pos += 1
        orig(self, b, token_ids, k_raw, v)
        self.seqs[b].next_pos -= 1
        self.seqs[b].pos = self.seqs[b].pos - 1
    monkeypatch.setattr(O.OracleCache, "append_rotated", off_by_one)
    with pytest.raises(AssertionError):
        test_append_rotated_unit_vectors_and_position_zero()
